"""Seeded synthetic inputs for paged MLA decoding.

This module only draws random numbers and lays them out; it holds none of
the attention arithmetic.  Both the HIP path (tests, bench) and the CPU
oracle take their inputs from here.

Layouts (row-major, contiguous):
  q            bf16 bits  uint16 [batch][s_q][h_q][576]
  kv (bf16)    bf16 bits  uint16 [num_blocks][64][576]
  kv (fp8)     bytes      uint8  [num_blocks][64][656]: 512 e4m3 codes,
               4 little-endian fp32 scales (one per 128 dims), 64 bf16 RoPE
  kv (fp8 V4.1) bytes     uint8  [num_blocks][64][528]: 512 e4m3 codes of all
               512 dims, 16 e8m0 scales (one per 32 dims); q is then
               [batch][s_q][h_q][512] and d_qk = d_v = 512
  block_table  int32 [batch][max_blocks], -1 past a sequence's blocks
  seqlens      int32 [batch]
  indices      int32 [batch][s_q][topk] flat token ids (block*64+offset), -1 masked
  norm_w       bf16 bits  uint16 [576]

Poison: blocks no sequence references and slots past a sequence's length
hold NaN (bf16 0x7FC0; fp8 code 0x7F, NaN scales, NaN RoPE values), so a
kernel that reads them shows it in its output.

Recipe: numpy Generator(PCG64(seed)); values are drawn as float32 N(0,1)
and rounded to bf16 by torch's round-to-nearest-even cast; draws happen in
the order seqlens, pool permutation, q, KV, indices, norm weight.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

PAGE = 64
D_QK = 576
D_V = 512
FP8_TOKEN_BYTES = 656
FP8V41_TOKEN_BYTES = 528
D_QK_V41 = 512
BF16_NAN = 0x7FC0
FP8_NAN = 0x7F


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (round to nearest even, torch cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 array (|x| <= 448) -> OCP e4m3fn codes via torch's cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(np.clip(x, -448.0, 448.0), dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@dataclass
class Problem:
    name: str
    batch: int
    s_q: int
    h_q: int
    seqlens: np.ndarray
    block_table: np.ndarray
    num_blocks: int
    q: np.ndarray
    kv: np.ndarray
    kv_format: str = "bf16"          # "bf16", "fp8v32" or "fp8v41"
    causal: bool = False
    indices: Optional[np.ndarray] = None
    topk: int = 0
    scale: float = D_QK ** -0.5
    fused: bool = False
    norm_w: Optional[np.ndarray] = None
    eps: float = 1e-6
    rope_base: float = 10000.0
    h_kv: int = 1
    d_qk: int = D_QK
    d_v: int = D_V
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.s_q * self.h_q

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


def _draw_bf16(rng: np.random.Generator, n: int) -> np.ndarray:
    return _bf16_bits(rng.standard_normal(n, dtype=np.float32))


def make_dense(name, seqlens, s_q, h_q, seed, causal=False, pool_factor=1.2,
               fused=False, max_blocks=None, extra_pool_blocks=0) -> Problem:
    """Dense bf16 paged problem with a shuffled block table over a pool of
    ceil(pool_factor * needed) blocks; unreferenced data is NaN."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seqlens = np.asarray(seqlens, dtype=np.int32)
    return _dense_from_lengths(name, rng, seqlens, s_q, h_q, causal, pool_factor, fused,
                               max_blocks, extra_pool_blocks)


def _dense_from_lengths(name, rng, seqlens, s_q, h_q, causal, pool_factor, fused,
                        max_blocks, extra_pool_blocks) -> Problem:
    b = int(seqlens.shape[0])
    nblk = (seqlens.astype(np.int64) + PAGE - 1) // PAGE
    need = int(nblk.sum())
    pool = max(int(math.ceil(pool_factor * need)), 1) + int(extra_pool_blocks)
    perm = rng.permutation(pool).astype(np.int32)
    mb = int(max(int(nblk.max()) if b else 0, 1)) if max_blocks is None else int(max_blocks)
    bt = np.full((b, mb), -1, dtype=np.int32)
    off = 0
    for i in range(b):
        bt[i, : nblk[i]] = perm[off: off + nblk[i]]
        off += int(nblk[i])
    q = _draw_bf16(rng, b * s_q * h_q * D_QK).reshape(b, s_q, h_q, D_QK)
    kv = np.full((pool, PAGE, D_QK), BF16_NAN, dtype=np.uint16)
    total = int(seqlens.astype(np.int64).sum())
    vals = _draw_bf16(rng, total * D_QK).reshape(total, D_QK)
    pos = 0
    for i in range(b):
        L = int(seqlens[i])
        if L == 0:
            continue
        j = np.arange(L)
        phys = bt[i, j // PAGE]
        kv[phys, j % PAGE] = vals[pos: pos + L]
        pos += L
    p = Problem(name=name, batch=b, s_q=s_q, h_q=h_q, seqlens=seqlens, block_table=bt,
                num_blocks=pool, q=q, kv=kv, causal=causal)
    if fused:
        p.fused = True
        w = rng.uniform(0.5, 1.5, size=D_QK).astype(np.float32)
        p.norm_w = _bf16_bits(w)
    return p


def make_sparse_fp8(name, batch, s_q, h_q, cache_len, topk, seed, pad_frac=0.1,
                    pool_factor=1.2) -> Problem:
    """Token-level sparse decode over a V3.2 FP8 paged cache.

    Each sequence holds cache_len tokens.  Each query row draws topk distinct
    logical positions uniformly, sorted ascending, mapped to flat physical ids
    through a shuffled block table.  round(pad_frac*batch*s_q) rows keep only a
    prefix of k_valid entries (the first of them none) and pad the rest with -1.
    Latent values are x/scale rounded to e4m3 with x ~ N(0,1) and one scale per
    128 dims drawn as 2^U(-4,4); RoPE values are bf16 N(0,1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seqlens = np.full(batch, cache_len, dtype=np.int32)
    nblk = (cache_len + PAGE - 1) // PAGE
    need = nblk * batch
    pool = int(math.ceil(pool_factor * need))
    perm = rng.permutation(pool).astype(np.int32)
    bt = perm[: need].reshape(batch, nblk).copy()
    q = _draw_bf16(rng, batch * s_q * h_q * D_QK).reshape(batch, s_q, h_q, D_QK)
    # indices: logical positions, sorted, then physical ids
    idx = np.empty((batch, s_q, topk), dtype=np.int64)
    for b in range(batch):
        for t in range(s_q):
            lp = np.sort(rng.choice(cache_len, size=topk, replace=False))
            idx[b, t] = bt[b, lp // PAGE].astype(np.int64) * PAGE + lp % PAGE
    npad = int(round(pad_frac * batch * s_q))
    pad_rows = rng.choice(batch * s_q, size=npad, replace=False)
    for r_i, r in enumerate(pad_rows):
        b, t = divmod(int(r), s_q)
        k_valid = 0 if r_i == 0 else int(rng.integers(0, topk))
        idx[b, t, k_valid:] = -1
    used = np.unique(idx[idx >= 0])
    kv = np.zeros((pool * PAGE, FP8_TOKEN_BYTES), dtype=np.uint8)
    kv[:, :512] = FP8_NAN
    kv[:, 512:528] = np.frombuffer(np.full(4, np.nan, dtype=np.float32).tobytes(), dtype=np.uint8)
    kv[:, 528:] = np.frombuffer(np.full(64, BF16_NAN, dtype=np.uint16).tobytes(), dtype=np.uint8)
    n = int(used.shape[0])
    x = rng.standard_normal((n, 512), dtype=np.float32)
    sc = np.exp2(rng.uniform(-4.0, 4.0, size=(n, 4))).astype(np.float32)
    codes = _e4m3_codes(x / np.repeat(sc, 128, axis=1))
    rope = _draw_bf16(rng, n * 64).reshape(n, 64)
    kv[used, :512] = codes
    kv[used, 512:528] = sc.view(np.uint8).reshape(n, 16)
    kv[used, 528:] = rope.view(np.uint8).reshape(n, 128)
    kv = kv.reshape(pool, PAGE, FP8_TOKEN_BYTES)
    return Problem(name=name, batch=batch, s_q=s_q, h_q=h_q, seqlens=seqlens, block_table=bt,
                   num_blocks=pool, q=q, kv=kv, kv_format="fp8v32",
                   indices=idx.astype(np.int32), topk=topk)


def make_sparse_fp8_v41(name, batch, s_q, h_q, cache_len, topk, seed, pad_frac=0.1,
                        pool_factor=1.2) -> Problem:
    """Token-level sparse decode over a V4.1 FP8 paged cache (528 B per
    token, head dim 512 with V = K).

    Indices are drawn as in make_sparse_fp8.  Values are x/scale rounded to
    e4m3 with x ~ N(0,1) and one power-of-two scale per 32 dims, 2^k with k
    uniform in -4..4 (stored as the e8m0 byte k + 127).  Unused records hold
    NaN codes and NaN (0xFF) scales."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seqlens = np.full(batch, cache_len, dtype=np.int32)
    nblk = (cache_len + PAGE - 1) // PAGE
    need = nblk * batch
    pool = int(math.ceil(pool_factor * need))
    perm = rng.permutation(pool).astype(np.int32)
    bt = perm[: need].reshape(batch, nblk).copy()
    q = _draw_bf16(rng, batch * s_q * h_q * D_QK_V41).reshape(batch, s_q, h_q, D_QK_V41)
    idx = np.empty((batch, s_q, topk), dtype=np.int64)
    for b in range(batch):
        for t in range(s_q):
            lp = np.sort(rng.choice(cache_len, size=topk, replace=False))
            idx[b, t] = bt[b, lp // PAGE].astype(np.int64) * PAGE + lp % PAGE
    npad = int(round(pad_frac * batch * s_q))
    pad_rows = rng.choice(batch * s_q, size=npad, replace=False)
    for r_i, r in enumerate(pad_rows):
        b, t = divmod(int(r), s_q)
        k_valid = 0 if r_i == 0 else int(rng.integers(0, topk))
        idx[b, t, k_valid:] = -1
    used = np.unique(idx[idx >= 0])
    kv = np.zeros((pool * PAGE, FP8V41_TOKEN_BYTES), dtype=np.uint8)
    kv[:, :512] = FP8_NAN
    kv[:, 512:] = 0xFF
    n = int(used.shape[0])
    x = rng.standard_normal((n, 512), dtype=np.float32)
    k = rng.integers(-4, 5, size=(n, 16))
    codes = _e4m3_codes(x / np.repeat(np.exp2(k).astype(np.float32), 32, axis=1))
    kv[used, :512] = codes
    kv[used, 512:] = (k + 127).astype(np.uint8)
    kv = kv.reshape(pool, PAGE, FP8V41_TOKEN_BYTES)
    return Problem(name=name, batch=batch, s_q=s_q, h_q=h_q, seqlens=seqlens, block_table=bt,
                   num_blocks=pool, q=q, kv=kv, kv_format="fp8v41", indices=idx.astype(np.int32),
                   topk=topk, scale=D_QK_V41 ** -0.5, d_qk=D_QK_V41, d_v=D_V)


def make_sparse_bf16_from_dense(p: Problem, topk: int, seed: int) -> Problem:
    """Sparse indices over an existing dense bf16 problem (s_q rows share
    nothing): each (b, t) draws topk positions < L_b with replacement off
    when possible; short sequences pad with -1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = np.full((p.batch, p.s_q, topk), -1, dtype=np.int64)
    for b in range(p.batch):
        L = int(p.seqlens[b])
        for t in range(p.s_q):
            k = min(topk, L)
            if k == 0:
                continue
            lp = np.sort(rng.choice(L, size=k, replace=False))
            idx[b, t, :k] = p.block_table[b, lp // PAGE].astype(np.int64) * PAGE + lp % PAGE
    q = Problem(**{**p.__dict__})
    q.indices = idx.astype(np.int32)
    q.topk = topk
    q.causal = False
    return q


def with_fp8v32(p: Problem, seed: int) -> Problem:
    """The same problem over a V3.2 FP8 cache: every stored token (a bf16 row
    that is not the NaN poison) becomes a 656 B record whose latent dims are
    its bf16 values divided by one scale per 128 dims, 2^U(-4,4), rounded to
    e4m3, and whose RoPE dims are its bf16 values unchanged.  Poisoned rows
    stay poisoned (NaN codes, scales and RoPE)."""
    assert p.kv_format == "bf16" and p.d_qk == D_QK
    rng = np.random.Generator(np.random.PCG64(seed))
    flat = p.kv.reshape(-1, D_QK)
    used = np.nonzero(flat[:, 0] != BF16_NAN)[0]
    kv = np.zeros((flat.shape[0], FP8_TOKEN_BYTES), dtype=np.uint8)
    kv[:, :512] = FP8_NAN
    kv[:, 512:528] = np.frombuffer(np.full(4, np.nan, dtype=np.float32).tobytes(), dtype=np.uint8)
    kv[:, 528:] = np.frombuffer(np.full(64, BF16_NAN, dtype=np.uint16).tobytes(), dtype=np.uint8)
    n = int(used.shape[0])
    x = (flat[used, :512].astype(np.uint32) << 16).view(np.float32)
    sc = np.exp2(rng.uniform(-4.0, 4.0, size=(n, 4))).astype(np.float32)
    kv[used, :512] = _e4m3_codes(x / np.repeat(sc, 128, axis=1))
    kv[used, 512:528] = sc.view(np.uint8).reshape(n, 16)
    kv[used, 528:] = np.ascontiguousarray(flat[used, 512:]).view(np.uint8).reshape(n, 128)
    q = Problem(**{**p.__dict__})
    q.kv = kv.reshape(-1, PAGE, FP8_TOKEN_BYTES)
    q.kv_format = "fp8v32"
    return q


# ---------------------------------------------------------------------------
# The five standard workloads
# ---------------------------------------------------------------------------

def config1(seed=1001) -> Problem:
    """Tiny: batch 2, h_q 16, seqlens {37, 100}, non-causal."""
    return make_dense("tiny_b2_h16", [37, 100], s_q=1, h_q=16, seed=seed)


def config2(seed=1002, batch=64) -> Problem:
    """Memory-bound: batch 64, h_q 128, seqlens ~ U{1024..8192}."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seqlens = rng.integers(1024, 8192 + 1, size=batch).astype(np.int32)
    return _dense_from_lengths(f"dense_b{batch}_h128_L1k-8k", rng, seqlens, 1, 128, False, 1.2,
                               False, None, 0)


def config3(seed=1003, batch=128) -> Problem:
    """Split-KV: batch 128, s_q 2 causal, seqlens log-uniform [256, 32768],
    4 sequences fixed at 65536."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seqlens = np.floor(np.exp(rng.uniform(math.log(256), math.log(32768), size=batch)))
    seqlens = seqlens.astype(np.int32)
    long_rows = rng.choice(batch, size=min(4, batch), replace=False)
    seqlens[long_rows] = 65536
    return _dense_from_lengths(f"splitkv_b{batch}_sq2_causal", rng, seqlens, 2, 128, True, 1.2,
                               False, None, 0)


def config4(seed=1004, batch=64, cache_len=65536, topk=2048) -> Problem:
    """Sparse top-k over an FP8 V3.2 cache."""
    return make_sparse_fp8(f"sparse_fp8_b{batch}_top{topk}", batch, 1, 128, cache_len, topk,
                           seed)


def config_v41(seed=1006, batch=64, cache_len=65536, topk=2048) -> Problem:
    """Config 4's shape over a V4.1 FP8 cache (528 B per token, head dim 512):
    the workload of the format the pages name as current."""
    return make_sparse_fp8_v41(f"sparse_fp8v41_b{batch}_top{topk}", batch, 1, 128, cache_len, topk, seed)


def config5(batch=32, seed=None) -> Problem:
    """Fused RMSNorm/RoPE prologue + conjugate RoPE/FP8 epilogue, h_q 128,
    seqlens ~ U{2048..16384}; batch 1 (seed 1051) or 32 (seed 1052)."""
    if seed is None:
        seed = 1051 if batch == 1 else 1052
    rng = np.random.Generator(np.random.PCG64(seed))
    seqlens = rng.integers(2048, 16384 + 1, size=batch).astype(np.int32)
    return _dense_from_lengths(f"fused_b{batch}_h128", rng, seqlens, 1, 128, False, 1.2, True,
                               None, 0)


# The standard workloads by the names bench.py and the profiles use.
WORKLOADS = {
    "dense_b64_h128_L1k-8k": config2,
    "splitkv_b128_sq2_causal": config3,
    "sparse_fp8_b64_top2048": config4,
    "fused_b32_h128": lambda: config5(32),
    "fused_b1_h128": lambda: config5(1),
    "sparse_fp8v41_b64_top2048": config_v41,
}


def by_name(name: str) -> Problem:
    return WORKLOADS[name]()
