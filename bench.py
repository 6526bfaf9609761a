"""Benchmark of the paged MLA decode hot path on one MI355X.

A step is one pass of the whole path over one batch: the split-KV metadata
call, the decode kernel and the LSE combine kernel.  The default workload is the
memory-bound bf16 decode (batch 64, s_q 1, h_q 128, d_qk 576, d_v 512,
seqlens ~ U{1024..8192}, 64-token pages, shuffled block table over a 1.2x
pool), seeded and synthetic.  Inputs are resident in HBM before timing; the
KV pool and queries are replicated into several copies that steps rotate
through, so a step never finds its KV in the 256 MB Infinity Cache left by
the previous step.  The timed steps launch their calls from the host
(``--graph`` replays one captured hipGraph per copy instead); the decode
kernel's own duration comes from a second, untimed pass.

Prints one JSON line with the metric (effective HBM GB/s of algorithmic
bytes per step), the TFLOPS, the decode kernel's roofline position and the
CPU oracle's rate on the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(p):
    """Bytes and flops the method must move / do (visible keys only)."""
    L = p.seqlens.astype(np.int64)
    rows = p.s_q * p.h_q
    if p.indices is None:
        if p.causal:
            vis = np.stack([np.clip(L - p.s_q + t + 1, 0, L) for t in range(p.s_q)], 1)
        else:
            vis = np.repeat(L[:, None], p.s_q, 1)
        keys_flops = int(vis.sum()) * p.h_q
        kv = int(L.sum()) * 1152
        tables = int(((L + 63) // 64).sum()) * 4
    else:
        valid = (p.indices >= 0)
        keys_flops = int(valid.sum()) * p.h_q
        per = {"fp8v32": 656, "fp8v41": 528}.get(p.kv_format, 1152)
        kv = sum(len(np.unique(p.indices[b][p.indices[b] >= 0])) for b in range(p.batch)) * per
        tables = p.indices.size * 4
    q = p.batch * rows * p.d_qk * 2
    o = p.batch * rows * (512 + 4 if p.fused else 512 * 2)
    lse = p.batch * rows * 4
    nbytes = kv + q + o + lse + tables + p.batch * 4
    flops = 2 * keys_flops * (p.d_qk + p.d_v)
    return nbytes, flops


WORKLOADS = ("dense_b64_h128_L1k-8k", "splitkv_b128_sq2_causal", "sparse_fp8_b64_top2048", "fused_b32_h128",
             "fused_b1_h128", "sparse_fp8v41_b64_top2048")


def make_workload(name):
    from mla_paged_kv_05_amd import workloads as W
    return W.by_name(name)


def traffic_record(kernel_src, workload):
    """HBM traffic measured by rocprofv3 PMC counters for the current kernel
    source on this workload, or None when the counters were taken on other
    code or another workload."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()[:16]
    return rec if rec.get("kernel_sha") == h and rec.get("workload") == workload else None


def measured_peaks(dev):
    """The box's own ceilings, a second denominator beside the published
    peaks: a 1 GiB device-to-device copy (bytes read + written per second)
    and a large bf16 GEMM on the vendor library (flop/s), best of 5 each."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    c = torch.empty(8192, 8192, device=dev, dtype=torch.bfloat16)

    def best(fn):
        ts = []
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts[1:])
    copy_s = best(lambda: dst.copy_(src))
    gemm_s = best(lambda: torch.mm(a, b, out=c))
    del src, dst, a, b, c
    return {"copy_gbs": round(2 * n / copy_s / 1e9, 1), "gemm_bf16_tflops": round(2 * 8192 ** 3 / gemm_s / 1e12, 1),
            "copy": "1 GiB device-to-device copy, read + written bytes", "gemm": "8192^3 bf16 torch.mm"}


def cpu_baseline(p, nbytes, flops):
    import oracle
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    runs = []
    for _ in range(3):  # the median of three runs
        t0 = time.perf_counter()
        oracle.decode(p, nthreads=cores)
        runs.append(time.perf_counter() - t0)
    dt = float(np.median(runs))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"whole workload ({p.batch} sequences), fp64, median of 3 runs, {dt:.2f} s",
            "seconds": round(dt, 3), "gflops": round(flops / dt / 1e9, 2), "cpu_model": model, "threads": cores,
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense_b64_h128_L1k-8k", choices=WORKLOADS)
    ap.add_argument("--rotate", type=int, default=0, help="KV copies (0 = enough for >= 1 GiB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--graph", action="store_true",
                    help="capture each step's three calls once as a hipGraph and replay it "
                         "(default: launch them from the host)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times) and exit: "
                         "the known-size kernel that scales HBM counter readings")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sequences shard across GPUs with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from mla_paged_kv_05_amd import binding as B

    dev = torch.device("cuda", 0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)
        return
    t0 = time.time()
    p = make_workload(args.workload)
    nbytes, flops = algorithmic(p)
    log(f"workload {p.name}: generated in {time.time() - t0:.1f}s; algorithmic "
        f"{nbytes / 1e6:.1f} MB, {flops / 1e9:.1f} GFLOP per step")

    kv_np = p.kv.view(np.int16) if p.kv_format == "bf16" else p.kv
    kv_bytes = kv_np.nbytes
    R = args.rotate or max(2, int(np.ceil(1.0 * 2 ** 30 / kv_bytes)))
    kv_host = torch.from_numpy(kv_np)
    kvs = [kv_host.to(dev) for _ in range(R)]
    if p.kv_format == "bf16":
        kvs = [k.view(torch.bfloat16) for k in kvs]
    qs = [torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16).to(dev) for _ in range(R)]
    bt = torch.from_numpy(np.ascontiguousarray(p.block_table)).to(dev)
    sl = torch.from_numpy(np.ascontiguousarray(p.seqlens)).to(dev)
    idx = None if p.indices is None else torch.from_numpy(p.indices).to(dev)
    topk = p.topk if idx is not None else 0
    # the fused decode's query prologue costs about four items per piece
    piece_cost = B.PIECE_COST_FUSED if p.fused else 0
    rows = p.s_q * p.h_q
    lib = B.load_library()
    S = B.num_sched_slots(rows, dev)
    meta = torch.empty((S, 8), dtype=torch.int32, device=dev)
    ns = torch.empty(int(lib.mla_num_splits_ints(p.batch)), dtype=torch.int32, device=dev)
    ws = torch.empty(B.workspace_bytes(p.batch, p.s_q, p.h_q, S), dtype=torch.uint8, device=dev)
    out = torch.empty((p.batch, p.s_q, p.h_q, 512), dtype=torch.uint8 if p.fused else torch.bfloat16,
                      device=dev)
    lse = torch.empty((p.batch, p.s_q, p.h_q), dtype=torch.float32, device=dev)
    fused = None
    if p.fused:
        fused = {"norm_weight": torch.from_numpy(p.norm_w.view(np.int16)).view(torch.bfloat16).to(dev),
                 "eps": p.eps, "rope_base": p.rope_base,
                 "out_scale": torch.empty((p.batch, p.s_q, p.h_q), dtype=torch.float32, device=dev)}
    params = []
    for r in range(R):
        pr = B._params(qs[r], kvs[r], bt if idx is None else None, sl, meta, ns, p.causal, idx, p.scale,
                       p.kv_format, ws, out, lse, fused)
        pr.flags = B.MLA_FLAG_DEFER_COMBINE
        params.append(pr)
    sl_p, meta_p, ns_p = ctypes.c_void_p(sl.data_ptr()), ctypes.c_void_p(meta.data_ptr()), ctypes.c_void_p(ns.data_ptr())

    # The decode kernel's own start/end timestamps (mla_decode_timed records
    # the events at the kernel dispatch), on the launch stream.
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime already loaded by torch
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def hip_event():
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def step(i, kev=None):
        # the stream is looked up at call time: under graph capture it is the
        # capturing stream
        pr = params[i % R]
        sh = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        st = lib.mla_get_metadata(sl_p, p.batch, rows, 1, topk, S, piece_cost, meta_p, ns_p, sh)
        if kev is not None:
            st |= lib.mla_decode_timed(ctypes.byref(pr), sh, kev[0], kev[1])
        else:
            st |= lib.mla_decode(ctypes.byref(pr), sh)
        st |= lib.mla_combine(ctypes.byref(pr), sh)
        if st != 0:
            raise RuntimeError(lib.mla_last_error().decode())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # One hipGraph per KV copy, each holding a whole step (metadata, decode,
    # combine), as a serving loop would replay it.
    graphs = None
    if args.graph:
        graphs = []
        cap = torch.cuda.Stream(dev)
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(r)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % R].replay()
        torch.cuda.synchronize()

    def run_steps(first):
        if graphs is not None:
            for i in range(args.steps):
                graphs[(first + i) % R].replay()
        else:
            for i in range(args.steps):
                step(first + i)

    # Timed region: the steps only, bracketed by two events on the stream.
    # With eager launches every decode launch also records the kernel's own
    # start and end (mla_decode_timed: HIP events at the dispatch, on the
    # launch stream), so the kernel durations come from the timed steps
    # themselves: the GPU's clock drifts over a run, and a separate pass
    # would time the kernel at another clock.
    stream = torch.cuda.current_stream(dev)
    kevs = [(hip_event(), hip_event()) for _ in range(args.steps)]
    # one event at each step boundary (eager launches): the per-step
    # distribution.  Between graph replays they would cost a few
    # microseconds of the replay pipelining, so graphs go without.
    sevs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    if graphs is not None:
        run_steps(args.warmup)
    else:
        for i in range(args.steps):
            sevs[i].record(stream)
            step(args.warmup + i, kevs[i])
    end.record(stream)
    host = time.perf_counter() - wall0  # host time to enqueue the steps
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(end) / args.steps

    # Second pass, outside the timed region: the metadata call's duration
    # per step, and under --graph (events cannot be recorded at a dispatch
    # inside a captured graph) the decode kernel's.
    mevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        mevs[i][0].record(stream)
        st = lib.mla_get_metadata(sl_p, p.batch, rows, 1, topk, S, piece_cost, meta_p, ns_p,
                                  ctypes.c_void_p(stream.cuda_stream))
        mevs[i][1].record(stream)
        if st != 0:
            raise RuntimeError(lib.mla_last_error().decode())
        if graphs is not None:
            pr = params[(args.warmup + i) % R]
            st = lib.mla_decode_timed(ctypes.byref(pr), ctypes.c_void_p(stream.cuda_stream), kevs[i][0],
                                      kevs[i][1])
            st |= lib.mla_combine(ctypes.byref(pr), ctypes.c_void_p(stream.cuda_stream))
            if st != 0:
                raise RuntimeError(lib.mla_last_error().decode())
    torch.cuda.synchronize()
    dec_ms = []
    for k0, k1 in kevs:
        t = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(t), k0, k1) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        dec_ms.append(t.value)
        hip.hipEventDestroy(k0)
        hip.hipEventDestroy(k1)
    meta_ms = [mevs[i][0].elapsed_time(mevs[i][1]) for i in range(args.steps)]
    step_ms = None if graphs is not None else [
        sevs[i].elapsed_time(sevs[i + 1] if i + 1 < args.steps else end) for i in range(args.steps)]
    dec_avg = float(np.mean(dec_ms))
    log(f"step {ms * 1e3:.1f} us ({'eager launches' if graphs is None else 'hipGraph replay'}; wall "
        f"{wall / args.steps * 1e6:.1f} us, host enqueue {host / args.steps * 1e6:.1f} us); decode kernel avg {dec_avg * 1e3:.1f} us (p10 "
        f"{np.percentile(dec_ms, 10) * 1e3:.1f}, p90 {np.percentile(dec_ms, 90) * 1e3:.1f}); metadata "
        f"{np.mean(meta_ms) * 1e3:.1f} us; rotation {R}")

    value = nbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    # The decode kernel's roofline: HBM-bound below the ridge point (peak
    # flop/s over peak bytes/s, 312.5 flop/B), MFMA-bound above it.
    hbm_gbs = nbytes / (dec_avg * 1e-3) / 1e9
    mfma_tflops = flops / (dec_avg * 1e-3) / 1e12
    intensity = flops / nbytes if nbytes else 0.0
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity > ridge:
        roof = {"bound": "mfma", "achieved": round(mfma_tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(mfma_tflops / BF16_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(hbm_gbs / HBM_PEAK_GBS, 4)}
    src = os.path.join(ROOT, "mla_paged_kv_05_amd", "csrc", "mla_kernels.hip")
    tr = traffic_record(src, p.name)
    traffic = None if tr is None else tr["bytes_per_launch"]
    # the type the products run in: bf16 on a bf16 cache and on V4.1 records
    # (exact bf16 after dequantisation), fp16 on V3.2 records and on every
    # fused decode
    compute_dtype = "f16" if (p.fused or p.kv_format == "fp8v32") else "bf16"
    res = {
        "metric": "MLA paged decode effective HBM GB/s (algorithmic bytes) + TFLOPS, b=64 h_q=128 seq<=8K",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "step_us": None if step_ms is None else {
            "median": round(float(np.median(step_ms)) * 1e3, 2),
            "p10": round(float(np.percentile(step_ms, 10)) * 1e3, 2),
            "p90": round(float(np.percentile(step_ms, 90)) * 1e3, 2),
            "timing": "HIP events at each step boundary in the timed region"},
        "vs_baseline": None, "dtype": compute_dtype, "data": "synthetic (seeded, shaped like the workload)",
        "config": {"workload": p.name, "batch": p.batch, "s_q": p.s_q, "h_q": p.h_q, "d_qk": p.d_qk,
                   "d_v": 512, "page": 64, "kv_format": p.kv_format, "causal": bool(p.causal),
                   "sparse_topk": topk, "fused": bool(p.fused), "sched_piece_cost": piece_cost,
                   "parallelism": "single GPU",
                   "kv_copies_rotated": R,
                   "launch": "eager" if graphs is None else "hipGraph per step (metadata, decode, combine)",
                   "combine": "separate launch"},
        "tflops": round(tflops, 2),
        "roofline": dict(roof, **{
            "traffic": traffic,
            # the same counters' bytes beside it: the decode's over its
            # algorithmic bytes (split partials, query re-reads), and what
            # the combine of those partials reads and writes per step
            "traffic_over_algorithmic": None if tr is None else round(traffic / nbytes, 4),
            "combine_traffic": None if tr is None else {
                "read_bytes": tr["combine_read_bytes_per_launch"],
                "write_bytes": tr["combine_write_bytes_per_launch"]},
            "kernel": "k_decode",
            "kernel_avg_us": round(dec_avg * 1e3, 2),
            "kernel_median_us": round(float(np.median(dec_ms)) * 1e3, 2),
            "kernel_p10_us": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
            "kernel_p90_us": round(float(np.percentile(dec_ms, 90)) * 1e3, 2),
            "kernel_timing": ("HIP events at each decode dispatch in the timed steps" if graphs is None
                              else "HIP events at the decode dispatch, second eager pass"),
            "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": flops,
            "intensity_flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": round(ridge, 1),
            "hbm_gbs": round(hbm_gbs, 1), "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
            "mfma_tflops": round(mfma_tflops, 1), "mfma_frac": round(mfma_tflops / BF16_PEAK_TFLOPS, 4)}),
    }
    # the box's own ceilings beside the published peaks (outside the timed region)
    pk = measured_peaks(dev)
    pk["hbm_frac_of_copy"] = round(hbm_gbs / pk["copy_gbs"], 4)
    pk["mfma_frac_of_gemm"] = round(mfma_tflops / pk["gemm_bf16_tflops"], 4)
    res["roofline"]["measured_peaks"] = pk
    if not args.no_cpu:
        log("timing the CPU oracle on the same workload ...")
        res["cpu_baseline"] = cpu_baseline(p, nbytes, flops)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
