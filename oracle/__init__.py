"""CPU oracle for paged MLA decoding -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package.  It loads ``liboracle.so`` built from
``mla_oracle.c`` (plain C, fp64, OpenMP, no fast-math) and never touches
the HIP library.  ``build()`` compiles it with gcc.

Functions mirror the C entry points; arrays are numpy.  See mla_oracle.c
for what each computes and which passage of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP, IEEE semantics)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("s_q", ctypes.c_int32), ("h_q", ctypes.c_int32),
        ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("kv_format", ctypes.c_int32), ("num_blocks", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("kv", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int32),
        ("seqlens", ctypes.c_void_p), ("causal", ctypes.c_int32),
        ("indices", ctypes.c_void_p), ("topk", ctypes.c_int32),
        ("scale", ctypes.c_double), ("fused", ctypes.c_int32),
        ("norm_w", ctypes.c_void_p), ("eps", ctypes.c_double), ("rope_base", ctypes.c_double),
    ]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER
    lib.orc_bf16_to_f64.restype = ctypes.c_double
    lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e8m0_decode.restype = ctypes.c_double
    lib.orc_e8m0_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_encode_rne.restype = ctypes.c_uint8
    lib.orc_e4m3_encode_rne.argtypes = [ctypes.c_double]
    lib.orc_rmsnorm.restype = None
    lib.orc_rmsnorm.argtypes = [P(ctypes.c_double), P(ctypes.c_double), ctypes.c_int,
                                ctypes.c_double, P(ctypes.c_double)]
    lib.orc_rope.restype = None
    lib.orc_rope.argtypes = [P(ctypes.c_double), ctypes.c_int, ctypes.c_double,
                             ctypes.c_double, ctypes.c_double]
    lib.orc_attend.restype = None
    lib.orc_attend.argtypes = [P(ctypes.c_double), ctypes.c_int64, P(ctypes.c_double),
                               ctypes.c_int, ctypes.c_int, ctypes.c_double,
                               P(ctypes.c_double), P(ctypes.c_double)]
    lib.orc_combine.restype = None
    lib.orc_combine.argtypes = [ctypes.c_int, P(ctypes.c_double), P(ctypes.c_double),
                                ctypes.c_int, P(ctypes.c_double), P(ctypes.c_double)]
    lib.orc_decode.restype = ctypes.c_int
    lib.orc_decode.argtypes = [P(_Problem), P(ctypes.c_double), P(ctypes.c_double),
                               P(ctypes.c_uint8), P(ctypes.c_double), ctypes.c_int]
    lib.orc_decode_row.restype = ctypes.c_int
    lib.orc_decode_row.argtypes = [P(_Problem), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   P(ctypes.c_double), P(ctypes.c_double), P(ctypes.c_uint8),
                                   P(ctypes.c_double)]
    lib.orc_decode_row_subset.restype = ctypes.c_int
    lib.orc_decode_row_subset.argtypes = [P(_Problem), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int64, P(ctypes.c_int64),
                                          P(ctypes.c_double), P(ctypes.c_double)]
    lib.orc_sched_plan.restype = ctypes.c_int
    lib.orc_sched_plan.argtypes = [P(ctypes.c_int32), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, P(ctypes.c_int32), P(ctypes.c_int32)]
    _lib = lib
    return lib


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _vp(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- scalars
def bf16_to_f64(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.orc_bf16_to_f64(int(x)) for x in b], dtype=np.float64)


def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([lib.orc_e4m3_decode(int(x)) for x in c], dtype=np.float64)


def e8m0_decode(codes) -> np.ndarray:
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([lib.orc_e8m0_decode(int(x)) for x in c], dtype=np.float64)


def e4m3_encode(x) -> np.ndarray:
    lib = _load()
    v = np.asarray(x, dtype=np.float64).ravel()
    return np.array([lib.orc_e4m3_encode_rne(float(a)) for a in v], dtype=np.uint8)


def rmsnorm(x, w, eps) -> np.ndarray:
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    y = np.empty_like(x)
    lib.orc_rmsnorm(_dptr(x), _dptr(w), int(x.shape[0]), float(eps), _dptr(y))
    return y


def rope(x, pos, base=10000.0, sign=1.0) -> np.ndarray:
    lib = _load()
    y = np.ascontiguousarray(x, dtype=np.float64).copy()
    lib.orc_rope(_dptr(y), int(y.shape[0] // 2), float(pos), float(base), float(sign))
    return y


def attend(q, keys, d_v, scale):
    """Softmax attention of one fp64 row over explicit fp64 keys [n][d_qk]."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float64)
    keys = np.ascontiguousarray(keys, dtype=np.float64).reshape(-1, q.shape[0])
    o = np.empty(d_v, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    lib.orc_attend(_dptr(q), int(keys.shape[0]), _dptr(keys), int(q.shape[0]), int(d_v),
                   float(scale), _dptr(o), _dptr(lse))
    return o, float(lse[0])


def combine(lse_parts, o_parts):
    lib = _load()
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    n, d_v = o_parts.shape
    o = np.empty(d_v, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    lib.orc_combine(int(n), _dptr(lse_parts), _dptr(o_parts), int(d_v), _dptr(o), _dptr(lse))
    return o, float(lse[0])


# ---------------------------------------------------------------- problems
def _problem_struct(p, keep):
    q = np.ascontiguousarray(p.q, dtype=np.uint16)
    kv = np.ascontiguousarray(p.kv)
    bt = np.ascontiguousarray(p.block_table, dtype=np.int32)
    sl = np.ascontiguousarray(p.seqlens, dtype=np.int32)
    idx = None if p.indices is None else np.ascontiguousarray(p.indices, dtype=np.int32)
    w = None if p.norm_w is None else np.ascontiguousarray(p.norm_w, dtype=np.uint16)
    keep.extend([q, kv, bt, sl, idx, w])
    s = _Problem()
    s.batch, s.s_q, s.h_q, s.d_qk, s.d_v = p.batch, p.s_q, p.h_q, p.d_qk, p.d_v
    s.kv_format = {"bf16": 0, "fp8v32": 1, "fp8v41": 2}[p.kv_format]
    s.num_blocks = int(p.num_blocks)
    s.q, s.kv, s.block_table, s.seqlens = _vp(q), _vp(kv), _vp(bt), _vp(sl)
    s.max_blocks = int(bt.shape[1])
    s.causal = int(bool(p.causal))
    s.indices = _vp(idx)
    s.topk = int(p.topk)
    s.scale = float(p.scale)
    s.fused = int(bool(p.fused))
    s.norm_w = _vp(w)
    s.eps = float(p.eps)
    s.rope_base = float(p.rope_base)
    return s


def decode(p, nthreads: int = 0) -> dict:
    """Oracle decode of a workloads.Problem: dict with o [b,s_q,h_q,d_v] and
    lse [b,s_q,h_q] (fp64); in fused mode also codes (uint8) and oscale."""
    lib = _load()
    keep = []
    s = _problem_struct(p, keep)
    rows = p.batch * p.s_q * p.h_q
    o = np.zeros((rows, p.d_v), dtype=np.float64)
    lse = np.zeros(rows, dtype=np.float64)
    codes = np.zeros((rows, p.d_v), dtype=np.uint8)
    oscale = np.zeros(rows, dtype=np.float64)
    rc = lib.orc_decode(ctypes.byref(s), _dptr(o), _dptr(lse),
                        codes.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), _dptr(oscale),
                        int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    shp = (p.batch, p.s_q, p.h_q)
    out = {"o": o.reshape(*shp, p.d_v), "lse": lse.reshape(shp)}
    if p.fused:
        out["codes"] = codes.reshape(*shp, p.d_v)
        out["oscale"] = oscale.reshape(shp)
    return out


def decode_row(p, b, t, h) -> dict:
    """One output row (b, t, h) exactly as decode() computes it: o (d_v,),
    lse; in fused mode also codes (uint8, d_v) and oscale."""
    lib = _load()
    keep = []
    s = _problem_struct(p, keep)
    o = np.zeros(p.d_v, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    codes = np.zeros(p.d_v, dtype=np.uint8)
    oscale = np.zeros(1, dtype=np.float64)
    rc = lib.orc_decode_row(ctypes.byref(s), int(b), int(t), int(h), _dptr(o), _dptr(lse),
                            codes.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), _dptr(oscale))
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    out = {"o": o, "lse": float(lse[0])}
    if p.fused:
        out["codes"] = codes
        out["oscale"] = float(oscale[0])
    return out


def decode_row_subset(p, b, t, h, key_pos):
    """One row over an explicit subset of keys (logical positions when dense,
    flat token ids when sparse): returns (o, lse)."""
    lib = _load()
    keep = []
    s = _problem_struct(p, keep)
    kp = np.ascontiguousarray(key_pos, dtype=np.int64)
    o = np.zeros(p.d_v, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    lib.orc_decode_row_subset(ctypes.byref(s), int(b), int(t), int(h), int(kp.shape[0]),
                              kp.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _dptr(o),
                              _dptr(lse))
    return o, float(lse[0])


def sched_plan(seqlens, rows, topk, num_slots, piece_cost=0):
    """The split-KV plan: (meta int32 [S][8], num_splits int32 [B+1]);
    piece_cost 0 takes the default piece cost."""
    lib = _load()
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    B = int(sl.shape[0])
    meta = np.zeros((num_slots, 8), dtype=np.int32)
    ns = np.zeros(B + 1, dtype=np.int32)
    rc = lib.orc_sched_plan(sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), B, int(rows),
                            int(topk), int(num_slots), int(piece_cost),
                            meta.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                            ns.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if rc != 0:
        raise ValueError("bad schedule arguments")
    return meta, ns
