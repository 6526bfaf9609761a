"""The binding's argument checks (CPU only: nothing here reaches a kernel).

mla_paged_kv_05_amd.binding hands raw addresses to the C ABI, which reads
memory in the layouts include/mla.h states; a tensor of the wrong dtype,
layout, device or shape would be read silently there.  These tests build
valid host tensors, check that the parameter block is accepted, then plant
one mistake at a time and check that it raises before any address crosses
the boundary.
"""
import pytest
import torch

from mla_paged_kv_05_amd import binding as B

B_, S_Q, H_Q, BLOCKS, MAXB, SLOTS = 2, 1, 16, 6, 3, 8


def args(fmt="bf16", sparse=False, fused_mode=False, **over):
    tok = {"bf16": 576, "fp8v32": 656, "fp8v41": 528}[fmt]
    d_qk = 512 if fmt == "fp8v41" else 576
    kv_dtype = torch.bfloat16 if fmt == "bf16" else torch.uint8
    a = dict(
        q=torch.zeros((B_, S_Q, H_Q, d_qk), dtype=torch.bfloat16),
        kvcache=torch.zeros((BLOCKS, 64, tok), dtype=kv_dtype),
        block_table=None if sparse else torch.zeros((B_, MAXB), dtype=torch.int32),
        cache_seqlens=torch.full((B_,), 100, dtype=torch.int32),
        sched_meta=torch.zeros((SLOTS, 8), dtype=torch.int32),
        num_splits=torch.zeros((B_ + 1,), dtype=torch.int32),
        causal=False,
        indices=torch.zeros((B_, S_Q, 64), dtype=torch.int32) if sparse else None,
        softmax_scale=None,
        kv_format=fmt,
        workspace=torch.zeros((1024,), dtype=torch.uint8),
        out=torch.zeros((B_, S_Q, H_Q, 512), dtype=torch.uint8 if fused_mode else torch.bfloat16),
        lse=torch.zeros((B_, S_Q, H_Q), dtype=torch.float32),
        fused={"norm_weight": torch.ones((576,), dtype=torch.bfloat16),
               "out_scale": torch.zeros((B_, S_Q, H_Q), dtype=torch.float32)} if fused_mode else None,
    )
    a.update(over)
    return a


def params(**kw):
    return B._params(**kw)


@pytest.mark.parametrize("kw", [
    {},
    {"sparse": True},
    {"fmt": "fp8v32"},
    {"fmt": "fp8v32", "sparse": True},
    {"fmt": "fp8v41", "sparse": True},
    {"fused_mode": True},
])
def test_valid_arguments_pass(kw):
    a = args(**kw)
    p = params(**a)
    assert p.batch == B_ and p.s_q == S_Q and p.h_q == H_Q
    assert p.num_slots == SLOTS
    assert p.softmax_scale == pytest.approx(a["q"].shape[-1] ** -0.5)
    assert p.topk == (64 if kw.get("sparse") else 0)


def q_strided():
    return torch.zeros((B_, S_Q, 2 * H_Q, 576), dtype=torch.bfloat16)[:, :, ::2]


@pytest.mark.parametrize("what,over,exc", [
    ("int64 block_table", {"block_table": torch.zeros((B_, MAXB), dtype=torch.int64)}, TypeError),
    ("block_table of another batch", {"block_table": torch.zeros((B_ + 1, MAXB), dtype=torch.int32)}, ValueError),
    ("no block_table and no indices", {"block_table": None}, ValueError),
    ("int64 cache_seqlens", {"cache_seqlens": torch.zeros((B_,), dtype=torch.int64)}, TypeError),
    ("short cache_seqlens", {"cache_seqlens": torch.zeros((B_ - 1,), dtype=torch.int32)}, ValueError),
    ("fp32 q", {"q": torch.zeros((B_, S_Q, H_Q, 576), dtype=torch.float32)}, TypeError),
    ("strided q", {"q": q_strided()}, ValueError),
    ("q of 512 dims on a 576-dim cache", {"q": torch.zeros((B_, S_Q, H_Q, 512), dtype=torch.bfloat16)}, ValueError),
    ("3-d q", {"q": torch.zeros((B_, H_Q, 576), dtype=torch.bfloat16)}, ValueError),
    ("uint8 pool as bf16", {"kvcache": torch.zeros((BLOCKS, 64, 1152), dtype=torch.uint8)}, TypeError),
    ("page of 32 tokens", {"kvcache": torch.zeros((BLOCKS, 32, 576), dtype=torch.bfloat16)}, ValueError),
    ("unknown format", {"kv_format": "fp4"}, ValueError),
    ("bf16 out of the wrong shape", {"out": torch.zeros((B_, S_Q, H_Q, 576), dtype=torch.bfloat16)}, ValueError),
    ("fp32 out", {"out": torch.zeros((B_, S_Q, H_Q, 512), dtype=torch.float32)}, TypeError),
    ("short lse", {"lse": torch.zeros((B_, S_Q, H_Q - 1), dtype=torch.float32)}, ValueError),
    ("bf16 lse", {"lse": torch.zeros((B_, S_Q, H_Q), dtype=torch.bfloat16)}, TypeError),
    ("sched_meta of 4 columns", {"sched_meta": torch.zeros((SLOTS, 4), dtype=torch.int32)}, ValueError),
    ("num_splits without its last prefix", {"num_splits": torch.zeros((B_,), dtype=torch.int32)}, ValueError),
    ("int16 workspace", {"workspace": torch.zeros((512,), dtype=torch.int16)}, TypeError),
    ("tensor on another device", {"lse": torch.zeros((B_, S_Q, H_Q), dtype=torch.float32, device="meta")},
     ValueError),
    ("not a tensor", {"cache_seqlens": [100, 100]}, TypeError),
])
def test_dense_mistakes_raise(what, over, exc):
    with pytest.raises(exc):
        params(**args(**over))


@pytest.mark.parametrize("what,over,exc", [
    # torch.topk returns int64 indices: they must be converted first
    ("int64 indices", {"indices": torch.zeros((B_, S_Q, 64), dtype=torch.int64)}, TypeError),
    ("indices of another batch", {"indices": torch.zeros((B_ + 1, S_Q, 64), dtype=torch.int32)}, ValueError),
    ("indices without the s_q axis", {"indices": torch.zeros((B_, 64), dtype=torch.int32)}, ValueError),
    ("strided indices", {"indices": torch.zeros((B_, S_Q, 128), dtype=torch.int32)[:, :, ::2]}, ValueError),
])
def test_sparse_mistakes_raise(what, over, exc):
    with pytest.raises(exc):
        params(**args(sparse=True, **over))


@pytest.mark.parametrize("what,kv_format,over,exc", [
    ("bf16 pool passed as fp8v32", "fp8v32", {"kvcache": torch.zeros((BLOCKS, 64, 656), dtype=torch.bfloat16)},
     TypeError),
    ("V4.1 records passed as fp8v32", "fp8v32", {"kvcache": torch.zeros((BLOCKS, 64, 528), dtype=torch.uint8)},
     ValueError),
    ("576-dim q on the V4.1 cache", "fp8v41", {"q": torch.zeros((B_, S_Q, H_Q, 576), dtype=torch.bfloat16)},
     ValueError),
])
def test_fp8_mistakes_raise(what, kv_format, over, exc):
    with pytest.raises(exc):
        params(**args(fmt=kv_format, sparse=True, **over))


@pytest.mark.parametrize("what,over,exc", [
    ("bf16 out in fused mode", {"out": torch.zeros((B_, S_Q, H_Q, 512), dtype=torch.bfloat16)}, TypeError),
    ("fp32 norm weight", {"fused": {"norm_weight": torch.ones((576,), dtype=torch.float32),
                                    "out_scale": torch.zeros((B_, S_Q, H_Q), dtype=torch.float32)}}, TypeError),
    ("norm weight of 512 dims", {"fused": {"norm_weight": torch.ones((512,), dtype=torch.bfloat16),
                                           "out_scale": torch.zeros((B_, S_Q, H_Q), dtype=torch.float32)}},
     ValueError),
    ("out_scale of the wrong shape", {"fused": {"norm_weight": torch.ones((576,), dtype=torch.bfloat16),
                                                "out_scale": torch.zeros((B_, H_Q), dtype=torch.float32)}},
     ValueError),
])
def test_fused_mistakes_raise(what, over, exc):
    with pytest.raises(exc):
        params(**args(fused_mode=True, **over))
