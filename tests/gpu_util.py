"""Helpers shared by the GPU tests: upload a workloads.Problem, run the HIP
path through the C-ABI binding, and compare with the oracle at the
tolerances the parity bar sets (bf16 O: max-abs 2e-2 and relative RMS
5e-3 over the tensor, and every row's own relative RMS within 1e-2; LSE:
max-abs 1e-3; FP8 O: one e4m3 step after dequantisation)."""
import math
import sys

import numpy as np
import torch

O_MAX_ABS = 2e-2
O_REL_RMS = 5e-3
# One broken row barely moves the tensor's relative RMS, so every row is
# also held to its own bound (twice the tensor bar).
O_ROW_REL_RMS = 1e-2
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
    from mla_paged_kv_05_amd import binding

    if t is None:
        t = upload(p)
    meta, ns = mla.get_mla_metadata(t["seqlens"], p.s_q * p.h_q, 1, topk=p.topk if p.indices is not None else 0,
                                    num_slots=num_slots, piece_cost=binding.PIECE_COST_FUSED if p.fused else 0)
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


def row_rel_rms(o, ref_o):
    """Relative RMS error of every output row (last axis), 0 for rows whose
    reference is exactly zero and whose output is too."""
    d = (o - ref_o).reshape(-1, o.shape[-1])
    r = ref_o.reshape(-1, o.shape[-1])
    num = np.sqrt((d * d).sum(axis=1))
    den = np.sqrt((r * r).sum(axis=1))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def check_o_lse(o, lse, ref_o, ref_lse, what=""):
    """bf16 O and fp32 LSE against fp64 references."""
    assert o.shape == ref_o.shape, (o.shape, ref_o.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    d = np.abs(o - ref_o)
    max_abs = float(d.max()) if d.size else 0.0
    num = math.sqrt(float((d * d).sum()))
    den = math.sqrt(float((ref_o * ref_o).sum()))
    rel = num / den if den > 0 else num
    rows = row_rel_rms(o, ref_o) if o.size else np.zeros(1)
    worst = int(np.argmax(rows))
    assert max_abs <= O_MAX_ABS, f"{what}: O max-abs {max_abs:.3e}"
    assert rel <= O_REL_RMS, f"{what}: O rel-RMS {rel:.3e}"
    assert rows[worst] <= O_ROW_REL_RMS, f"{what}: row {worst} rel-RMS {rows[worst]:.3e}"
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf LSE pattern differs"
    if (~empty).any():
        le = float(np.abs(lse[~empty] - ref_lse[~empty]).max())
        assert le <= LSE_MAX_ABS, f"{what}: LSE max-abs {le:.3e}"
    if empty.any():
        assert np.all(o[empty] == 0), f"{what}: empty rows must be exactly 0"
    le = float(np.abs(lse[~empty] - ref_lse[~empty]).max()) if (~empty).any() else 0.0
    say(f"{what}: O max-abs {max_abs:.2e} (bar {O_MAX_ABS:.0e}), rel-RMS {rel:.2e} (bar {O_REL_RMS:.0e}), "
        f"worst row rel-RMS {rows[worst]:.2e} (bar {O_ROW_REL_RMS:.0e}), LSE max-abs {le:.2e} (bar {LSE_MAX_ABS:.0e})")
    return max_abs, rel


def e4m3_value(codes):
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return c.to(torch.float64).numpy()


def e4m3_step(a):
    """Spacing of e4m3 values at magnitude a (2^-9 below the normal range)."""
    return np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-300))) - 3))


# FP8 output bar ("within one e4m3 step after dequantisation"): the GPU's
# codes against the oracle's own codes, element by element, with the row
# scales compared on their own.
#  - Row scale: |scale_gpu / scale_ref - 1| <= FP8_SCALE_REL, and each row's
#    largest element encodes as +-448.  The scale is the row's largest |O|
#    over 448, so it carries that element's relative error and is held to
#    O's own relative bar (O_REL_RMS); that moves the largest dequantised
#    element by under 448 * 5e-3 / 32 = 0.07 of its e4m3 step (32 at 256..448).
#  - Elements of at least amax/16: the two codes are equal or adjacent
#    e4m3 values (code distance <= 1 in the ordered list of e4m3 values).
#    An O that sits near a rounding midpoint legitimately rounds either way.
#  - Smaller elements: their e4m3 step is finer than what a P.V with 16-bit
#    operands resolves (its error is a fraction of the row's RMS, not of the
#    element), so the dequantised values must agree to max(one step of the
#    reference binade, 2^-8 * amax) plus what the scale difference itself
#    moves them by: c_g s_g - c_r s_r = (c_g - c_r) s_r + c_g (s_g - s_r), so
#    that term is |s_g - s_r| |c_g|.  Their code distances are reported.
#  - Bias: among elements of at least amax/16, at most FP8_FLIP_SHARE sit one
#    code apart, and the signed sum of their code differences is within
#    FP8_SHIFT_SIGMAS standard deviations of a symmetric +-1 walk over the
#    n elements that differ (|sum| <= 4 sqrt(n)).  Unbiased 16-bit rounding
#    flips only the few elements near a rounding midpoint, in both
#    directions; a one-step bias moves all n the same way (sum = n, which
#    fails once n > 16), a half-step shift about half of them.
FP8_BIG_FRACTION = 1.0 / 16
FP8_FLIP_SHARE = 1.0 / 8
FP8_SHIFT_SIGMAS = 4.0
FP8_SMALL_FLOOR = 2.0 ** -8
FP8_SCALE_REL = O_REL_RMS


def e4m3_order(codes):
    """Position of each e4m3 code in the ordered list of e4m3 values
    (+0 and -0 both at 0): adjacent values differ by 1."""
    c = np.asarray(codes, dtype=np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def check_fp8(codes, scale, ref_codes, ref_scale, ref_o, what=""):
    cdist = np.abs(e4m3_order(codes) - e4m3_order(ref_codes))
    v = e4m3_value(codes) * scale[..., None]
    rvv = e4m3_value(ref_codes)
    rv = rvv * ref_scale[..., None]
    step = e4m3_step(np.abs(rvv)) * ref_scale[..., None]
    amax = np.abs(ref_o).max(axis=-1, keepdims=True)
    big = np.abs(ref_o) >= FP8_BIG_FRACTION * amax
    srel = np.abs(scale / ref_scale - 1.0)
    gvv = e4m3_value(codes)
    allow = np.maximum(step, FP8_SMALL_FLOOR * amax) + np.abs(scale - ref_scale)[..., None] * np.abs(gvv)
    small_bad = ~big & (np.abs(v - rv) > allow * (1 + 1e-9))
    signed = (e4m3_order(codes) - e4m3_order(ref_codes))[big]
    flip = float((signed != 0).mean()) if signed.size else 0.0
    moved = int((signed != 0).sum())
    zshift = float(signed.sum()) / math.sqrt(max(moved, 1))
    hist = {k: int((cdist == k).sum()) for k in range(3)}
    hist[">2"] = int((cdist > 2).sum())
    say(f"{what}: FP8 code distance {hist} over {cdist.size} elements; >= amax/16: "
        f"{int((big & (cdist > 1)).sum())} beyond 1 of {int(big.sum())}; exempt share {float((~big).mean()):.3f}; "
        f"row scale rel err max {float(srel.max()) if srel.size else 0:.2e} (bar {FP8_SCALE_REL:.0e}); "
        f">= amax/16 one code apart {flip:.4f} (bar {FP8_FLIP_SHARE}), signed shift {zshift:+.2f} sigma "
        f"(bar {FP8_SHIFT_SIGMAS:.0f})")
    assert int((big & (cdist > 1)).sum()) == 0, f"{what}: elements >= amax/16 more than one e4m3 step apart"
    assert flip <= FP8_FLIP_SHARE, f"{what}: {flip:.3f} of elements >= amax/16 one code apart"
    assert abs(zshift) <= FP8_SHIFT_SIGMAS, f"{what}: code shift {zshift:+.2f} sigma over {moved} moved codes"
    assert int(small_bad.sum()) == 0, f"{what}: {int(small_bad.sum())} small elements beyond max(step, 2^-8 amax)"
    assert np.all(srel <= FP8_SCALE_REL), f"{what}: row scale rel err {float(srel.max()):.2e}"
    top = (np.asarray(codes) & 0x7F).max(axis=-1)
    assert np.all(top[amax[..., 0] > 0] == 0x7E), f"{what}: row max does not encode as 448"
    return int(cdist.max()) if cdist.size else 0
