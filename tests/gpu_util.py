"""Helpers shared by the GPU tests: upload a workloads.Problem, run the HIP
path through the C-ABI binding, and compare with the oracle at the
tolerances the parity bar sets (bf16 O: max-abs 2e-2 and relative RMS
5e-3; LSE: max-abs 1e-3; FP8 O: one e4m3 step after dequantisation)."""
import math
import sys

import numpy as np
import torch

O_MAX_ABS = 2e-2
O_REL_RMS = 5e-3
LSE_MAX_ABS = 1e-3


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def upload(p, dev="cuda:0"):
    t = {}
    t["q"] = torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16).to(dev)
    if p.kv_format == "bf16":
        t["kv"] = torch.from_numpy(p.kv.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        t["kv"] = torch.from_numpy(p.kv).to(dev)
    t["block_table"] = torch.from_numpy(np.ascontiguousarray(p.block_table)).to(dev)
    t["seqlens"] = torch.from_numpy(np.ascontiguousarray(p.seqlens)).to(dev)
    t["indices"] = None if p.indices is None else torch.from_numpy(p.indices).to(dev)
    if p.fused:
        t["norm_w"] = torch.from_numpy(p.norm_w.view(np.int16)).view(torch.bfloat16).to(dev)
    return t


def run(p, t=None, num_slots=None):
    """Metadata + decode on the GPU; returns numpy results."""
    import mla_paged_kv_05_amd as mla

    if t is None:
        t = upload(p)
    meta, ns = mla.get_mla_metadata(t["seqlens"], p.s_q * p.h_q, 1, topk=p.topk if p.indices is not None else 0,
                                    num_slots=num_slots)
    fused = None
    if p.fused:
        fused = {"norm_weight": t["norm_w"], "eps": p.eps, "rope_base": p.rope_base}
    res = mla.mla_decode_with_kvcache(
        t["q"], t["kv"], t["block_table"] if p.indices is None else None, t["seqlens"], 512, meta, ns,
        causal=p.causal, indices=t["indices"], softmax_scale=p.scale, kv_format=p.kv_format,
        fused=fused)
    torch.cuda.synchronize()
    out = {"meta": meta.cpu().numpy(), "num_splits": ns.cpu().numpy()}
    if p.fused:
        o, lse, sc = res
        out["codes"] = o.cpu().numpy()
        out["lse"] = lse.cpu().numpy().astype(np.float64)
        out["oscale"] = sc.cpu().numpy().astype(np.float64)
    else:
        o, lse = res
        out["o"] = o.float().cpu().numpy().astype(np.float64)
        out["lse"] = lse.cpu().numpy().astype(np.float64)
    return out


def check_o_lse(o, lse, ref_o, ref_lse, what=""):
    """bf16 O and fp32 LSE against fp64 references."""
    assert o.shape == ref_o.shape, (o.shape, ref_o.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    d = np.abs(o - ref_o)
    max_abs = float(d.max()) if d.size else 0.0
    num = math.sqrt(float((d * d).sum()))
    den = math.sqrt(float((ref_o * ref_o).sum()))
    rel = num / den if den > 0 else num
    assert max_abs <= O_MAX_ABS, f"{what}: O max-abs {max_abs:.3e}"
    assert rel <= O_REL_RMS, f"{what}: O rel-RMS {rel:.3e}"
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf LSE pattern differs"
    if (~empty).any():
        le = float(np.abs(lse[~empty] - ref_lse[~empty]).max())
        assert le <= LSE_MAX_ABS, f"{what}: LSE max-abs {le:.3e}"
    if empty.any():
        assert np.all(o[empty] == 0), f"{what}: empty rows must be exactly 0"
    le = float(np.abs(lse[~empty] - ref_lse[~empty]).max()) if (~empty).any() else 0.0
    say(f"{what}: O max-abs {max_abs:.2e} (bar {O_MAX_ABS:.0e}), rel-RMS {rel:.2e} (bar {O_REL_RMS:.0e}), "
        f"LSE max-abs {le:.2e} (bar {LSE_MAX_ABS:.0e})")
    return max_abs, rel


def e4m3_value(codes):
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return c.to(torch.float64).numpy()


def e4m3_step(a):
    """Spacing of e4m3 values at magnitude a (2^-9 below the normal range)."""
    return np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-300))) - 3))


def check_fp8(codes, scale, ref_o, ref_scale, what=""):
    """FP8 output parity: each GPU code, with the GPU's row scale, must be
    within one e4m3 step of the rounding of some O' that meets the bf16-O
    bar against the oracle's fp64 O.  Per element, e = distance from O_ref to
    [(c - step(c)) * scale, (c + step(c)) * scale]; max e <= 2e-2 and
    ||e|| / ||O_ref|| <= 5e-3.  A per-element step at the element's own binade
    (2^-9 * scale near zero) is finer than the accuracy any bf16 P.V path has
    for small elements, so the step is taken around the GPU's code and the O
    error is held to the same bar as the bf16 output.  The row scale must
    equal amax/448 of such an O' (|amax_gpu - amax_ref| <= 2e-2) and each
    row's largest element must encode as +-448."""
    v = e4m3_value(codes)
    st = e4m3_step(np.abs(v))
    lo = (v - st) * scale[..., None]
    hi = (v + st) * scale[..., None]
    e = np.where(ref_o < lo, lo - ref_o, np.where(ref_o > hi, ref_o - hi, 0.0))
    max_e = float(e.max()) if e.size else 0.0
    den = math.sqrt(float((ref_o * ref_o).sum()))
    rel = math.sqrt(float((e * e).sum())) / den if den > 0 else 0.0
    assert max_e <= O_MAX_ABS, f"{what}: fp8 max distance {max_e:.3e}"
    assert rel <= O_REL_RMS, f"{what}: fp8 rel-RMS distance {rel:.3e}"
    assert np.all(np.abs(scale - ref_scale) * 448.0 <= O_MAX_ABS), f"{what}: row scale mismatch"
    nz = ref_scale > 0
    top = (np.asarray(codes) & 0x7F).max(axis=-1)
    assert np.all(top[np.abs(ref_o).max(axis=-1) > 0] == 0x7E), f"{what}: row max does not encode as 448"
    say(f"{what}: FP8 distance max {max_e:.2e} (bar {O_MAX_ABS:.0e}), rel-RMS {rel:.2e} (bar {O_REL_RMS:.0e})")
    return max_e, rel
