"""Phase timeline of one decode launch, from the measurement library
(libmla_phase_trace.so, built by build.build_phase_trace()): where a
workgroup's time goes between its start, each piece's prologue, main loop and
finalize, and its end, and how long the launch's tail waits for the slowest
workgroup; then where a 32-key step's time goes, from wave 0's per-phase
sums of the shader clock.

    python -m mla_paged_kv_05_amd.phase_trace --workload dense_b64_h128_L1k-8k

Prints a markdown summary.  The timed launch runs after warm-up launches on
the same inputs (KV rotated over three copies), so caches are as in a run of
steps.  Needs a GPU; measurement only.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

from . import binding as B
from . import build as hip_build
from . import workloads as W

KTR_PER, KTR_PIECES = 40, 7   # the layout the traced kernel writes
KTR_STEP_OFF, KTR_STEPS = 32, 6
KTR_META, KTR_PASS1, KTR_PASS2 = 29, 30, 31   # first-piece stamps
STEP_PHASES = ["load wait", "barrier (fused bf16: with the fp16 conversion; one-tile FP8: with the dequantisation)",
               "load issue", "S^T (two-tile FP8: with the next tile's dequantisation)", "softmax and lazy rescale",
               "P.V issue"]
CLOCK_MHZ = 100.0             # s_memrealtime


def run(name: str, warmup: int = 6) -> str:
    import torch

    if not os.path.exists(hip_build.TRACE_LIB):
        raise SystemExit(f"{hip_build.TRACE_LIB} is not built: run build.build_phase_trace()")
    lib = B.load_library(hip_build.TRACE_LIB)
    lib.mla_phase_trace_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.mla_phase_trace_copy.restype = ctypes.c_int
    lib.mla_phase_trace_clear.restype = ctypes.c_int
    B._lib = lib  # every binding call below goes to the measurement library
    dev = torch.device("cuda", 0)
    p = W.by_name(name)
    kv_np = p.kv.view(np.int16) if p.kv_format == "bf16" else p.kv
    kvs = [torch.from_numpy(kv_np).to(dev) for _ in range(3)]
    if p.kv_format == "bf16":
        kvs = [k.view(torch.bfloat16) for k in kvs]
    q = torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16).to(dev)
    bt = torch.from_numpy(np.ascontiguousarray(p.block_table)).to(dev)
    sl = torch.from_numpy(np.ascontiguousarray(p.seqlens)).to(dev)
    idx = None if p.indices is None else torch.from_numpy(p.indices).to(dev)
    rows = p.s_q * p.h_q
    S = B.num_sched_slots(rows, dev)
    meta, ns = B.get_mla_metadata(sl, rows, 1, topk=p.topk if idx is not None else 0, num_slots=S,
                                  piece_cost=B.PIECE_COST_FUSED if p.fused else 0)
    fz = None
    if p.fused:
        fz = {"norm_weight": torch.from_numpy(p.norm_w.view(np.int16)).view(torch.bfloat16).to(dev),
              "eps": p.eps, "rope_base": p.rope_base}

    def launch(i):
        B.mla_decode_with_kvcache(q, kvs[i % 3], bt if idx is None else None, sl, 512, meta, ns, causal=p.causal,
                                  indices=idx, softmax_scale=p.scale, kv_format=p.kv_format, fused=fz)

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    if lib.mla_phase_trace_clear() != 0:
        raise RuntimeError("mla_phase_trace_clear failed")
    launch(warmup)
    torch.cuda.synchronize()
    nwg = S * ((rows + 127) // 128)
    tr = np.zeros(nwg * KTR_PER, np.uint64)
    items = np.zeros(nwg * KTR_PIECES, np.int32)
    if lib.mla_phase_trace_copy(tr.ctypes.data, items.ctypes.data, nwg) != 0:
        raise RuntimeError("mla_phase_trace_copy failed")
    tr = tr.reshape(nwg, KTR_PER).astype(np.int64)
    items = items.reshape(nwg, KTR_PIECES)
    act = tr[:, 0] > 0
    t0 = tr[act, 0].min()
    us = lambda x: (x - t0) / CLOCK_MHZ
    start, end = us(tr[act, 0]), us(tr[act, KTR_PER - 1])
    pro, loop, fin, nit = [], [], [], []
    for w in np.nonzero(act)[0]:
        for pc in range(KTR_PIECES):
            a, b, c, d = tr[w, 1 + 4 * pc: 5 + 4 * pc]
            if a == 0:
                break
            pro.append((b - a) / CLOCK_MHZ)
            loop.append((c - b) / CLOCK_MHZ)
            fin.append((d - c) / CLOCK_MHZ)
            nit.append(items[w, pc])
    pro, loop, fin, nit = map(np.array, (pro, loop, fin, nit))
    nact = int(act.sum())
    acc = tr[act, KTR_STEP_OFF:KTR_STEP_OFF + KTR_STEPS].sum(0)
    nsteps = int(tr[act, KTR_STEP_OFF + KTR_STEPS].sum())
    # shader-clock ticks per microsecond: the step sums against the same
    # steps' main-loop time on the 100 MHz clock
    ticks_per_us = acc.sum() / max(loop.sum(), 1e-9)
    first = (tr[act, 1] - tr[act, 0]) / CLOCK_MHZ

    def span(a, b):  # median of slot b - slot a over the workgroups that stamped both
        ta, tb = tr[act, a], tr[act, b]
        ok = (ta > 0) & (tb > 0)
        return float(np.median((tb[ok] - ta[ok]) / CLOCK_MHZ)) if ok.any() else float("nan")
    lines = [
        f"Phase timeline of one `{name}` decode launch (`python -m mla_paged_kv_05_amd.phase_trace "
        f"--workload {name}`):",
        "",
        "| Quantity | Value |", "|---|---|",
        f"| active workgroups | {nact} of {nwg} |",
        f"| launch span (first start to last end) | {end.max():.1f} us |",
        f"| workgroup start spread | {start.max():.1f} us |",
        f"| workgroup end: min / median / max | {end.min():.1f} / {np.median(end):.1f} / {end.max():.1f} us |",
        f"| pieces | {len(pro)} ({len(pro) / nact:.2f} per workgroup) |",
        f"| start to first piece, median | {np.median(first):.2f} us "
        f"(to the slot's metadata read {span(0, KTR_META):.2f}, then {span(KTR_META, 1):.2f}) |",
        f"| piece prologue (query, first loads, drain): median / p90 | {np.median(pro):.2f} / {np.percentile(pro, 90):.2f} us |",
        *([f"| first piece's fused prologue: pass 1 (query reads, first KV loads, row sum) / pass 2 (q-hat) / "
           f"drain, median | {span(1, KTR_PASS1):.2f} / {span(KTR_PASS1, KTR_PASS2):.2f} / {span(KTR_PASS2, 2):.2f} us |"]
          if p.fused else []),
        f"| main loop per 64-key item, median | {np.median(loop / np.maximum(nit, 1)):.3f} us |",
        f"| piece finalize: median / p90 | {np.median(fin):.2f} / {np.percentile(fin, 90):.2f} us |",
        f"| per workgroup: prologue / main loop / finalize | {pro.sum() / nact:.1f} / {loop.sum() / nact:.1f} / "
        f"{fin.sum() / nact:.1f} us |",
        f"| tail: mean of (last end - own end) | {np.mean(end.max() - end):.1f} us |",
        "",
        f"Per 32-key step (wave 0 of each workgroup, {nsteps} steps; shader clock {ticks_per_us:.0f} "
        f"cycles per us; a step is {acc.sum() / max(nsteps, 1):.0f} cycles = "
        f"{acc.sum() / max(nsteps, 1) / ticks_per_us:.3f} us):",
        "",
        "| Phase | cycles per step | share |", "|---|---|---|",
    ]
    for name_, v in zip(STEP_PHASES, acc):
        lines.append(f"| {name_} | {v / max(nsteps, 1):.0f} | {100 * v / max(acc.sum(), 1):.1f} % |")
    lines.append("")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="dense_b64_h128_L1k-8k", choices=sorted(W.WORKLOADS))
    args = ap.parse_args(argv)
    print(run(args.workload), flush=True)


if __name__ == "__main__":
    sys.exit(main())
