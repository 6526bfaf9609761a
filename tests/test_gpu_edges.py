"""GPU edge cases of the decode through the C ABI, against the oracle: an
empty batch, a batch whose sequences are all empty, the largest batch the
metadata call takes (16384 sequences), and the largest query-row count
(s_q * h_q = 65536, causal, with rows that see no key).  Large cases are
checked on rows the oracle computes one by one."""
import numpy as np
import pytest

import oracle
from mla_paged_kv_05_amd import workloads as W

from gpu_util import check_o_lse, run, say

gpu = pytest.mark.gpu


def _torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _visible(p, b, t):
    L = int(p.seqlens[b])
    n = L if not p.causal else max(0, min(L, L - p.s_q + t + 1))
    return np.arange(n, dtype=np.int64)


def _check_rows(p, g, rows, what):
    for (b, t, h) in rows:
        ro, rl = oracle.decode_row_subset(p, b, t, h, _visible(p, b, t))
        check_o_lse(g["o"][b, t, h][None], g["lse"][b, t, h][None], ro[None], np.array([rl]),
                    f"{what} row {(b, t, h)}")


@gpu
def test_empty_batch():
    _torch_cuda()
    p = W.make_dense("empty_batch", [], s_q=1, h_q=128, seed=40)
    say("empty batch")
    g = run(p)
    assert g["o"].shape == (0, 1, 128, 512) and g["lse"].shape == (0, 1, 128)
    assert int(g["num_splits"][0]) == 0


@gpu
def test_all_sequences_empty():
    _torch_cuda()
    p = W.make_dense("all_empty", [0, 0, 0], s_q=2, h_q=64, seed=41, causal=True)
    say("all sequences empty")
    g = run(p, num_slots=8)
    assert np.all(g["o"] == 0)
    assert np.all(np.isneginf(g["lse"]))


@gpu
def test_max_batch_sampled():
    """16384 sequences of 1..40 tokens (one page each), h_q = 16."""
    _torch_cuda()
    rng = np.random.default_rng(42)
    lens = rng.integers(1, 41, size=16384).astype(np.int32)
    p = W.make_dense("max_batch", lens, s_q=1, h_q=16, seed=42)
    say(f"max batch b={p.batch} h_q={p.h_q} tokens={int(lens.sum())}")
    g = run(p)
    rows = [(int(rng.integers(p.batch)), 0, int(rng.integers(p.h_q))) for _ in range(24)]
    rows += [(0, 0, 0), (p.batch - 1, 0, p.h_q - 1)]
    _check_rows(p, g, rows, "max-batch")


@gpu
def test_max_rows_sampled():
    """s_q = 512, h_q = 128 (65536 rows, 512 row groups), causal; the second
    sequence is shorter than s_q, so its first query tokens see no key."""
    _torch_cuda()
    p = W.make_dense("max_rows", [700, 300], s_q=512, h_q=128, seed=43, causal=True)
    say(f"max rows s_q={p.s_q} h_q={p.h_q} L={list(p.seqlens)}")
    g = run(p)
    rng = np.random.default_rng(43)
    rows = [(int(rng.integers(2)), int(rng.integers(512)), int(rng.integers(128))) for _ in range(20)]
    rows += [(0, 0, 0), (0, 511, 127), (1, 0, 5), (1, 211, 9), (1, 212, 9), (1, 511, 64)]
    _check_rows(p, g, rows, "max-rows")
    # rows of the short sequence before its first visible key are empty
    assert np.all(g["o"][1, :212] == 0) and np.all(np.isneginf(g["lse"][1, :212]))
