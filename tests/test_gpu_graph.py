"""The decode step (metadata, decode, combine) captured as a hipGraph: every
replay, with eager work and synchronisations in between, writes exactly
what the eager calls write."""
import ctypes

import numpy as np
import pytest

from mla_paged_kv_05_amd import workloads as W

from gpu_util import say, upload

gpu = pytest.mark.gpu


def _step_fn(torch, lib, B, p, t, S):
    dev = torch.device("cuda", 0)
    rows = p.s_q * p.h_q
    sparse = p.indices is not None
    meta = torch.empty((S, 8), dtype=torch.int32, device=dev)
    ns = torch.empty(int(lib.mla_num_splits_ints(p.batch)), dtype=torch.int32, device=dev)
    ws = torch.empty(B.workspace_bytes(p.batch, p.s_q, p.h_q, S), dtype=torch.uint8, device=dev)
    out = torch.empty((p.batch, p.s_q, p.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((p.batch, p.s_q, p.h_q), dtype=torch.float32, device=dev)
    pr = B._params(t["q"], t["kv"], None if sparse else t["block_table"], t["seqlens"], meta, ns, p.causal,
                   t["indices"], p.scale, p.kv_format, ws, out, lse, None)
    pr.flags = B.MLA_FLAG_DEFER_COMBINE
    topk = p.topk if sparse else 0

    def step():
        sh = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        st = lib.mla_get_metadata(ctypes.c_void_p(t["seqlens"].data_ptr()), p.batch, rows, 1, topk, S, 0,
                                  ctypes.c_void_p(meta.data_ptr()), ctypes.c_void_p(ns.data_ptr()), sh)
        st |= lib.mla_decode(ctypes.byref(pr), sh)
        st |= lib.mla_combine(ctypes.byref(pr), sh)
        assert st == 0, lib.mla_last_error()

    return step, (meta, ns, ws, out, lse)


@gpu
@pytest.mark.parametrize("kind", ["dense_causal", "sparse_fp8"])
def test_graph_replay_matches_eager(kind):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_paged_kv_05_amd import binding as B

    if kind == "dense_causal":
        p = W.make_dense("graph", [300, 1000, 64, 5, 2500], s_q=2, h_q=128, seed=31, causal=True)
    else:
        p = W.make_sparse_fp8("graph_fp8", batch=3, s_q=1, h_q=128, cache_len=4096, topk=512, seed=32)
    say(f"graph replay {kind} {p.name}")
    t = upload(p)
    lib = B.load_library()
    step, bufs = _step_fn(torch, lib, B, p, t, S=16)
    meta, ns, ws, out, lse = bufs

    step()
    torch.cuda.synchronize()
    ref_o = out.view(torch.int16).cpu().numpy().copy()
    ref_l = lse.cpu().numpy().copy()
    ref_m = meta.cpu().numpy().copy()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: clobber every buffer the step writes
        for x in (meta, ns, ws, out, lse):
            x.view(torch.uint8).fill_(0x5A + rep)
        torch.cuda.synchronize()
        say(f"graph replay {kind} #{rep}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(meta.cpu().numpy(), ref_m), f"replay {rep}: metadata differs"
        assert np.array_equal(out.view(torch.int16).cpu().numpy(), ref_o), f"replay {rep}: O differs"
        assert np.array_equal(lse.cpu().numpy(), ref_l), f"replay {rep}: LSE differs"
