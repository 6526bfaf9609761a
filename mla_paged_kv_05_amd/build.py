"""Build libmla.so (gfx950 only) in-tree with hipcc.

Every kernel's register use is read from the compiler's resource-usage
remarks; a kernel that needs scratch memory (register spills) is reported,
and with ``strict=True`` fails the build.  The FlashMLA build fails on any
register spill ("FlashMLA" AI Wiki, section "Requirements and build"); this
is the gfx950 analogue.
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
    spills = {k: v for k, v in resources.items() if v.get("ScratchSize", 0) > 0}
    if verbose:
        for k, v in sorted(resources.items()):
            print(f"  {k[:70]:70s} {v}")
    if spills:
        msg = "kernels using scratch (register spills): " + ", ".join(
            f"{k} ({v['ScratchSize']} B/lane)" for k, v in sorted(spills.items()))
        if strict:
            raise RuntimeError(msg)
        print("WARNING: " + msg, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(strict="--strict" in sys.argv, verbose=True)
    print(LIB)
