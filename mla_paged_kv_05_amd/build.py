"""Build libmla.so (gfx950 only) in-tree with hipcc.

Two gates run on every build:

* Scratch.  Every kernel's register use is read from the compiler's
  resource-usage remarks.  The FlashMLA build fails on any register spill
  ("FlashMLA" AI Wiki, section "Requirements and build"); here each kernel
  has a scratch budget (SCRATCH_BUDGET, bytes per lane: zero unless listed)
  and ``strict=True`` fails the build when a kernel exceeds it, so a spill
  can only grow by changing the table on purpose.
* MFMA result hazards.  The decode kernels issue their MFMAs as inline asm
  (to pin the accumulators), so the compiler cannot see that a later
  instruction reads an MFMA's result before it is written: the hardware
  does not interlock that read.  The built gfx950 code object is
  disassembled and every instruction that touches an MFMA's destination
  registers within MFMA_RESULT_WAIT wait states of it, other than an MFMA
  accumulating into the same registers, fails the build.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmla.so")
SOURCES = ["mla_kernels.hip", "mla_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LLVM_BIN = "/opt/rocm/llvm/bin"

# Scratch (spill) budget per kernel in bytes per lane, as measured today;
# the plain bf16 decode has none, the others' spills sit in the per-piece
# prologue and finalize, not in their step loops.  Any kernel not listed
# must have none.
SCRATCH_BUDGET = {
    "_ZN3mla8k_decodeILi0ELb1ELb0EEEvNS_10DecodeArgsE": 84,    # bf16 sparse
    "_ZN3mla8k_decodeILi0ELb0ELb1EEEvNS_10DecodeArgsE": 224,   # bf16 dense fused
    "_ZN3mla8k_decodeILi0ELb1ELb1EEEvNS_10DecodeArgsE": 164,   # bf16 sparse fused
    "_ZN3mla8k_decodeILi1ELb0ELb0EEEvNS_10DecodeArgsE": 148,   # V3.2 FP8 dense
    "_ZN3mla8k_decodeILi1ELb1ELb0EEEvNS_10DecodeArgsE": 68,    # V3.2 FP8 sparse
    "_ZN3mla8k_decodeILi1ELb0ELb1EEEvNS_10DecodeArgsE": 236,   # V3.2 FP8 dense fused
    "_ZN3mla8k_decodeILi1ELb1ELb1EEEvNS_10DecodeArgsE": 164,   # V3.2 FP8 sparse fused
    "_ZN3mla8k_decodeILi2ELb1ELb0EEEvNS_10DecodeArgsE": 68,    # V4.1 FP8 sparse
}
# Wait states an MFMA result needs before anything else reads or rewrites
# its registers (at least the 16-pass XDL requirement; the kernels' own
# settle sequences give 24).
MFMA_RESULT_WAIT = 18
ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # O lives in AGPRs through inline-asm operands; a VGPR spilled into an
    # "unused" AGPR would overwrite it, so spills never go to AGPRs
    "-mllvm", "-amdgpu-spill-vgpr-to-agpr=0",
    "-I", INCLUDE, "-I", CSRC,
]


def _parse_resources(text: str) -> dict:
    out, name = {}, None
    for line in text.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        if name is None:
            continue
        for key in ("VGPRs", "AGPRs", "ScratchSize [bytes/lane]", "LDS Size [bytes/block]",
                    "Occupancy [waves/SIMD]"):
            m = re.search(re.escape(key) + r": (\d+)", line)
            if m:
                out[name][key.split(" ")[0]] = int(m.group(1))
    return out


_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def _regs(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            for r in range(int(m.group(2)), int(m.group(3)) + 1):
                out.add((kind, r))
    return out


def mfma_hazards(disasm: str) -> list:
    """Instructions that read or write an MFMA's destination registers
    fewer than MFMA_RESULT_WAIT wait states after it, in straight-line code
    (tracking stops at a branch).  A dependent MFMA whose accumulator is the
    same register range is exempt: the hardware orders those."""
    found, func = [], "?"
    insts = []
    for line in disasm.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if m:
            func = m.group(1)
            insts.append(None)
            continue
        m = re.match(r"^\s+([a-z_][a-z0-9_]*)\s*(.*?)\s*(//.*)?$", line)
        if m and not line.strip().startswith("//"):
            insts.append((func, m.group(1), m.group(2)))
    for i, ins in enumerate(insts):
        if ins is None or not ins[1].startswith("v_mfma"):
            continue
        ops = [o.strip() for o in ins[2].split(",")]
        dst, dst_text = _regs(ops[0]), ops[0]
        waits = 0
        for j in range(i + 1, min(i + 64, len(insts))):
            nxt = insts[j]
            if nxt is None or nxt[1].startswith("s_branch") or nxt[1].startswith("s_cbranch") or \
                    nxt[1].startswith("s_setpc") or nxt[1] == "s_endpgm":
                break
            if waits >= MFMA_RESULT_WAIT:
                break
            name, text = nxt[1], nxt[2]
            if name.startswith("s_nop"):
                waits += int(text or "0") + 1
                continue
            if name.startswith("v_mfma"):
                nops = [o.strip() for o in text.split(",")]
                if nops[0] == dst_text and nops[-1] == dst_text:
                    break  # dependent accumulation: ordered by the hardware
            if _regs(text) & dst:
                found.append(f"{nxt[0]}: `{name} {text}` {waits} wait states after `{ins[1]} {ins[2]}`")
                break
            waits += 1
    return found


def check_hazards(obj: str) -> list:
    """Disassemble the gfx950 code object inside a hipcc object file (code
    built here) and return the MFMA result hazards it holds."""
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        fat, co = os.path.join(d, "fat.bin"), os.path.join(d, "k.co")
        subprocess.run([f"{LLVM_BIN}/llvm-objcopy", f"--dump-section=.hip_fatbin={fat}", obj, os.devnull],
                       check=True, capture_output=True)
        subprocess.run([f"{LLVM_BIN}/clang-offload-bundler", "--unbundle", "--type=o", f"--input={fat}",
                        f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--output={co}"],
                       check=True, capture_output=True)
        dis = subprocess.run([f"{LLVM_BIN}/llvm-objdump", "-d", f"--mcpu={ARCH}", co], check=True,
                             capture_output=True, text=True).stdout
    return mfma_hazards(dis)


def build(strict: bool = False, verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libmla.so; returns its path."""
    build_dir = os.path.join(ROOT, "_build")
    os.makedirs(build_dir, exist_ok=True)
    objs, resources = [], {}
    for src in SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        cmd = [HIPCC, *COMMON, "-Rpass-analysis=kernel-resource-usage", "-c",
               os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        resources.update(_parse_resources(r.stderr))
        objs.append(obj)
    tmp = LIB + f".tmp{os.getpid()}"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    if verbose:
        for k, v in sorted(resources.items()):
            print(f"  {k[:70]:70s} {v}")
    over = {k: v["ScratchSize"] for k, v in resources.items()
            if v.get("ScratchSize", 0) > SCRATCH_BUDGET.get(k, 0)}
    problems = []
    if over:
        problems.append("kernels over their scratch budget: " + ", ".join(
            f"{k} ({n} B/lane > {SCRATCH_BUDGET.get(k, 0)})" for k, n in sorted(over.items())))
    hazards = check_hazards(os.path.join(build_dir, "mla_kernels.hip.o"))
    if hazards:
        problems.append(f"{len(hazards)} MFMA result hazards, first: " + "; ".join(hazards[:3]))
    if problems:
        msg = "; ".join(problems)
        if strict:
            raise RuntimeError(msg)
        print("WARNING: " + msg, file=sys.stderr)
    return LIB


TRACE_LIB = os.path.join(HERE, "libmla_phase_trace.so")


def build_phase_trace() -> str:
    """The measurement library: the same sources with -DMLA_PHASE_TRACE, so
    each decode workgroup records its phase timeline (read back by
    mla_phase_trace_copy; see phase_trace.py).  Not the product library."""
    build_dir = os.path.join(ROOT, "_build", "phase_trace")
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        r = subprocess.run([HIPCC, *COMMON, "-DMLA_PHASE_TRACE", "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src} (phase trace build)")
        objs.append(obj)
    tmp = TRACE_LIB + f".tmp{os.getpid()}"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed (phase trace build)")
    os.replace(tmp, TRACE_LIB)
    return TRACE_LIB


if __name__ == "__main__":
    build(strict="--strict" in sys.argv, verbose=True)
    print(LIB)
