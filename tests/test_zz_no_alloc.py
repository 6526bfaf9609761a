"""The allocation-free entry point (mla_decode_noalloc, static per-GPU
scratch) against mla_decode with a caller workspace: two calls in a row on
the same GPU, the second with a smaller input, each compared with the
workspace entry point's output on the same inputs and with the oracle."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
from gpu_util import check_fp8, check_o_lse, say, upload  # noqa: E402
from mla_paged_kv_05_amd import workloads as W  # noqa: E402

gpu = pytest.mark.gpu


def _torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _both(p, num_slots):
    """Decode p through both entry points; returns numpy outputs of each."""
    torch = _torch_cuda()
    from mla_paged_kv_05_amd import binding as B

    t = upload(p)
    ind = t["indices"]
    meta, ns = B.get_mla_metadata(t["seqlens"], p.s_q * p.h_q, 1, topk=p.topk if ind is not None else 0,
                                  num_slots=num_slots)
    fused = None
    if p.fused:
        fused = {"norm_weight": t["norm_w"], "eps": p.eps, "rope_base": p.rope_base}
    bt = t["block_table"] if ind is None else None
    ref = B.mla_decode_with_kvcache(t["q"], t["kv"], bt, t["seqlens"], 512, meta, ns, causal=p.causal,
                                    indices=ind, softmax_scale=p.scale, kv_format=p.kv_format, fused=fused)
    dev = t["q"].device
    shape = (p.batch, p.s_q, p.h_q)
    out = torch.full(shape + (512,), 0x55, dtype=torch.uint8, device=dev) if p.fused else \
        torch.full(shape + (512,), 7.0, dtype=torch.bfloat16, device=dev)
    lse = torch.full(shape, 7.0, dtype=torch.float32, device=dev)
    fz = None if fused is None else {**fused, "out_scale": torch.full(shape, 7.0, dtype=torch.float32,
                                                                         device=dev)}
    got = B.mla_decode_noalloc(t["q"], t["kv"], bt, t["seqlens"], 512, meta, ns, out, lse, causal=p.causal,
                               indices=ind, softmax_scale=p.scale, kv_format=p.kv_format, fused=fz)
    torch.cuda.synchronize()
    conv = (lambda x: x.cpu().numpy()) if p.fused else (lambda x: x.float().cpu().numpy().astype(np.float64))
    return [conv(x) if i == 0 else x.cpu().numpy().astype(np.float64) for i, x in enumerate(ref)], \
        [conv(x) if i == 0 else x.cpu().numpy().astype(np.float64) for i, x in enumerate(got)], \
        int(ns.cpu().numpy()[p.batch])


def _check(p, num_slots, what):
    say(f"noalloc {what}: b={p.batch} L={list(p.seqlens)} fmt={p.kv_format} fused={p.fused} slots={num_slots}")
    ref, got, nsplit = _both(p, num_slots)
    assert nsplit > p.batch, f"{what}: the schedule must split some sequence to use the scratch"
    # same kernels, same schedule: the two entry points agree bit for bit
    for a, b, name in zip(ref, got, ("o", "lse", "scale")):
        assert np.array_equal(a, b, equal_nan=True), f"{what}: {name} differs from mla_decode"
    r = oracle.decode(p)
    if p.fused:
        check_fp8(got[0], got[2], r["codes"], r["oscale"], r["o"], f"noalloc {what}")
    else:
        check_o_lse(got[0], got[1], r["o"], r["lse"], f"noalloc {what}")
    say(f"noalloc {what}: identical to mla_decode over {nsplit} splits")


@gpu
def test_noalloc_two_calls_second_smaller():
    big = W.make_dense("na1", [3000, 70, 1500, 5, 700, 0], s_q=2, h_q=64, seed=41, causal=True)
    _check(big, 64, "first call")
    small = W.make_dense("na2", [900, 33], s_q=1, h_q=128, seed=42)
    _check(small, 16, "second, smaller call")


@gpu
def test_noalloc_fused_then_sparse_fp8():
    fz = W.make_dense("na3", [70, 1500, 5], s_q=1, h_q=128, seed=43, fused=True)
    _check(fz, 16, "fused")
    sp = W.with_fp8v32(W.make_sparse_bf16_from_dense(W.make_dense("na4", [400, 90], s_q=1, h_q=128, seed=44),
                                                      topk=256, seed=45), seed=46)
    _check(sp, 8, "sparse fp8, smaller")


@gpu
def test_noalloc_rejects_too_large():
    torch = _torch_cuda()
    from mla_paged_kv_05_amd import binding as B

    b = 600
    p = W.make_dense("na5", [64] * 4, s_q=1, h_q=128, seed=47)
    t = upload(p)
    seq = torch.full((b,), 64, dtype=torch.int32, device="cuda:0")
    bt = torch.zeros((b, 1), dtype=torch.int32, device="cuda:0")
    q = torch.zeros((b, 1, 128, 576), dtype=torch.bfloat16, device="cuda:0")
    meta, ns = B.get_mla_metadata(seq, 128, 1, num_slots=8)
    assert B.workspace_bytes(b, 1, 128, 8) > B.NOALLOC_SCRATCH_BYTES
    out = torch.empty((b, 1, 128, 512), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((b, 1, 128), dtype=torch.float32, device="cuda:0")
    with pytest.raises(B.MlaError, match="static array"):
        B.mla_decode_noalloc(q, t["kv"], bt, seq, 512, meta, ns, out, lse)
