"""The decode launch that merges the splits itself (MLA_FLAG_MERGE_IN_KERNEL:
cooperative, counters in the metadata's control area) writes exactly what a
decode launch followed by a separate combine launch writes, call after call
on the same metadata, and leaves the control area cleared for the next
call."""
import ctypes

import numpy as np
import pytest

from mla_paged_kv_05_amd import workloads as W

from gpu_util import say, upload

gpu = pytest.mark.gpu


def _case(kind):
    if kind == "dense":
        return W.make_dense("ikc", [300, 1000, 64, 5, 2500, 0, 777], s_q=1, h_q=128, seed=41)
    if kind == "causal_sq2":  # two row groups
        return W.make_dense("ikc2", [700, 65, 3000, 1], s_q=2, h_q=128, seed=42, causal=True)
    return W.make_sparse_fp8("ikc_fp8", batch=3, s_q=1, h_q=128, cache_len=4096, topk=512, seed=43)


@gpu
@pytest.mark.parametrize("kind", ["dense", "causal_sq2", "sparse_fp8"])
def test_inkernel_combine_matches_separate(kind):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_paged_kv_05_amd import binding as B

    p = _case(kind)
    dev = torch.device("cuda", 0)
    t = upload(p)
    lib = B.load_library()
    rows = p.s_q * p.h_q
    sparse = p.indices is not None
    S = 16  # few slots: most sequences split
    meta = torch.empty((S, 8), dtype=torch.int32, device=dev)
    ns = torch.empty(int(lib.mla_num_splits_ints(p.batch)), dtype=torch.int32, device=dev)
    ws = torch.empty(B.workspace_bytes(p.batch, p.s_q, p.h_q, S), dtype=torch.uint8, device=dev)
    sh = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    assert lib.mla_get_metadata(ctypes.c_void_p(t["seqlens"].data_ptr()), p.batch, rows, 1,
                                p.topk if sparse else 0, S, ctypes.c_void_p(meta.data_ptr()),
                                ctypes.c_void_p(ns.data_ptr()), sh) == 0
    torch.cuda.synchronize()
    ctl0 = ns.cpu().numpy().copy()
    nsplit = np.diff(ctl0[:p.batch + 1])
    assert (nsplit > 1).any(), "the case must split some sequence"

    def run(deferred):
        out = torch.full((p.batch, p.s_q, p.h_q, 512), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((p.batch, p.s_q, p.h_q), float("nan"), dtype=torch.float32, device=dev)
        pr = B._params(t["q"], t["kv"], None if sparse else t["block_table"], t["seqlens"], meta, ns,
                       p.causal, t["indices"], p.scale, p.kv_format, ws, out, lse, None)
        pr.flags = B.MLA_FLAG_DEFER_COMBINE if deferred else B.MLA_FLAG_MERGE_IN_KERNEL
        st = lib.mla_decode(ctypes.byref(pr), sh)
        if deferred:
            st |= lib.mla_combine(ctypes.byref(pr), sh)
        assert st == 0, lib.mla_last_error()
        torch.cuda.synchronize()
        return out.view(torch.int16).cpu().numpy(), lse.cpu().numpy()

    say(f"in-kernel combine {kind}: separate launches")
    ref_o, ref_l = run(True)
    for rep in range(3):
        say(f"in-kernel combine {kind}: call {rep}")
        o, l = run(False)
        assert np.array_equal(o, ref_o), f"call {rep}: O differs"
        assert np.array_equal(l, ref_l), f"call {rep}: LSE differs"
        assert np.array_equal(ns.cpu().numpy(), ctl0), f"call {rep}: control area not restored"
