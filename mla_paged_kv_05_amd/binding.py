"""ctypes binding of libmla.so: argument marshalling only.

Every step of the decode runs in the library's HIP kernels; this module
turns torch tensors into pointers, sizes and the current HIP stream, and
raises on a non-OK status.  It never computes anything itself and has no
fallback: if libmla.so is missing, importing it fails loudly.

Call order follows the FlashMLA Ampere-adaptation README (section "Usage"):
metadata once per decoding step, then one decode per layer reusing it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_OK = 0
MLA_KV_BF16 = 0
MLA_KV_FP8_V32 = 1
MLA_KV_FP8_V41 = 2
KV_FORMATS = {"bf16": MLA_KV_BF16, "fp8v32": MLA_KV_FP8_V32, "fp8v41": MLA_KV_FP8_V41}
PAGE = 64
D_QK = 576
D_V = 512

_STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED", 3: "MLA_ERR_WORKSPACE",
           4: "MLA_ERR_HIP"}


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class DecodeParams(ctypes.Structure):
    """Mirror of mla_decode_params in include/mla.h (same field order)."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("batch", ctypes.c_int32), ("s_q", ctypes.c_int32), ("h_q", ctypes.c_int32),
        ("h_kv", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("kv", ctypes.c_void_p),
        ("kv_format", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("block_table", ctypes.c_void_p),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("cache_seqlens", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("indices", ctypes.c_void_p),
        ("topk", ctypes.c_int32),
        ("sched_meta", ctypes.c_void_p),
        ("num_splits", ctypes.c_void_p),
        ("num_slots", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("fused", ctypes.c_int32),
        ("norm_weight", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
        ("rope_base", ctypes.c_float),
        ("out_scale", ctypes.c_void_p),
        ("flags", ctypes.c_uint32),
    ]


MLA_FLAG_DEFER_COMBINE = 1


EXPORTED = ["mla_num_sched_slots", "mla_sched_meta_ints", "mla_num_splits_ints", "mla_get_metadata",
            "mla_workspace_bytes", "mla_decode", "mla_decode_timed", "mla_decode_noalloc", "mla_combine", "mla_debug_gather",
            "mla_status_string", "mla_last_error"]

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmla.so and declare every exported signature."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() or "
                          "python -m mla_paged_kv_05_amd.build")
    lib = ctypes.CDLL(path)
    c = ctypes
    lib.mla_num_sched_slots.restype = c.c_int32
    lib.mla_num_sched_slots.argtypes = [c.c_int32, c.c_int32]
    lib.mla_sched_meta_ints.restype = c.c_size_t
    lib.mla_sched_meta_ints.argtypes = [c.c_int32]
    lib.mla_num_splits_ints.restype = c.c_size_t
    lib.mla_num_splits_ints.argtypes = [c.c_int32]
    lib.mla_get_metadata.restype = c.c_int
    lib.mla_get_metadata.argtypes = [c.c_void_p, c.c_int32, c.c_int32, c.c_int32, c.c_int32,
                                     c.c_int32, c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p]
    lib.mla_workspace_bytes.restype = c.c_size_t
    lib.mla_workspace_bytes.argtypes = [c.c_int32, c.c_int32, c.c_int32, c.c_int32]
    lib.mla_decode.restype = c.c_int
    lib.mla_decode.argtypes = [c.POINTER(DecodeParams), c.c_void_p]
    lib.mla_decode_timed.restype = c.c_int
    lib.mla_decode_timed.argtypes = [c.POINTER(DecodeParams), c.c_void_p, c.c_void_p, c.c_void_p]
    lib.mla_decode_noalloc.restype = c.c_int
    lib.mla_decode_noalloc.argtypes = [c.POINTER(DecodeParams), c.c_void_p]
    lib.mla_combine.restype = c.c_int
    lib.mla_combine.argtypes = [c.POINTER(DecodeParams), c.c_void_p]
    lib.mla_debug_gather.restype = c.c_int
    lib.mla_debug_gather.argtypes = [c.POINTER(DecodeParams), c.c_int32, c.c_int32, c.c_int32,
                                     c.c_void_p, c.c_void_p]
    lib.mla_status_string.restype = c.c_char_p
    lib.mla_status_string.argtypes = [c.c_int]
    lib.mla_last_error.restype = c.c_char_p
    lib.mla_last_error.argtypes = []
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(status: int):
    if status != MLA_OK:
        raise MlaError(status, load_library().mla_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def num_sched_slots(rows_per_kv_head: int, device=None) -> int:
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    n = load_library().mla_num_sched_slots(dev.index or 0, int(rows_per_kv_head))
    if n <= 0:
        raise MlaError(1, f"mla_num_sched_slots failed for rows={rows_per_kv_head}")
    return n


# Piece cost for metadata that fused decode calls use (MLA_PIECE_COST_FUSED).
PIECE_COST_FUSED = 4


def get_mla_metadata(cache_seqlens: torch.Tensor, rows_per_kv_head: int, h_kv: int = 1,
                     topk: int = 0, num_slots: Optional[int] = None, piece_cost: int = 0):
    """Split-KV schedule for one decoding step: (sched_meta int32 [S][8],
    num_splits int32 [batch+1]), both on cache_seqlens' device.  piece_cost
    0 takes the default piece cost; PIECE_COST_FUSED suits fused decodes."""
    lib = load_library()
    dev = cache_seqlens.device
    if cache_seqlens.dim() != 1:
        raise ValueError("cache_seqlens must be int32 [batch]")
    _need(cache_seqlens, "cache_seqlens", torch.int32)
    if dev.type != "cuda":
        raise ValueError("cache_seqlens must be on a GPU")
    S = num_slots if num_slots is not None else num_sched_slots(rows_per_kv_head, dev)
    B = cache_seqlens.shape[0]
    meta = torch.empty((S, 8), dtype=torch.int32, device=dev)
    ns = torch.empty(int(lib.mla_num_splits_ints(B)), dtype=torch.int32, device=dev)
    _check(lib.mla_get_metadata(_ptr(cache_seqlens), B, int(rows_per_kv_head), int(h_kv), int(topk),
                                S, int(piece_cost), _ptr(meta), _ptr(ns), _stream(dev)))
    return meta, ns


def workspace_bytes(batch: int, s_q: int, h_q: int, num_slots: int) -> int:
    return int(load_library().mla_workspace_bytes(batch, s_q, h_q, num_slots))


_TOKEN_SHAPE = {"bf16": (torch.bfloat16, D_QK), "fp8v32": (torch.uint8, 656), "fp8v41": (torch.uint8, 528)}


def _need(t, name, dtype, shape=None, device=None):
    """Argument check before a pointer crosses the C ABI: the library reads
    raw memory with the layout include/mla.h states, so a wrong dtype,
    stride, device or shape would be read silently."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _params(q, kvcache, block_table, cache_seqlens, sched_meta, num_splits, causal, indices,
            softmax_scale, kv_format, workspace, out, lse, fused):
    if kv_format not in _TOKEN_SHAPE:
        raise ValueError(f"kv_format must be one of {sorted(_TOKEN_SHAPE)}")
    if q.dim() != 4:
        raise ValueError(f"q must be [batch, s_q, h_q, d_qk], got {tuple(q.shape)}")
    b, s_q, h_q, d_qk = q.shape
    dev = q.device
    _need(q, "q", torch.bfloat16, device=dev)
    kv_dtype, tok = _TOKEN_SHAPE[kv_format]
    _need(kvcache, "kvcache", kv_dtype, device=dev)
    kv_tail = tuple(kvcache.shape[2:])
    if kvcache.dim() < 3 or kvcache.shape[1] != PAGE or kv_tail not in ((tok,), (1, tok)):
        raise ValueError(f"kvcache for {kv_format} must be [blocks, {PAGE}, {tok}] or "
                         f"[blocks, {PAGE}, 1, {tok}], got {tuple(kvcache.shape)}")
    if kv_format == "fp8v41" and d_qk != 512:
        raise ValueError("the fp8v41 cache has head dim 512: q must be [b, s_q, h_q, 512]")
    if kv_format != "fp8v41" and d_qk != D_QK:
        raise ValueError(f"q must have {D_QK} dims per head, got {d_qk}")
    _need(cache_seqlens, "cache_seqlens", torch.int32, (b,), dev)
    if indices is None:
        if block_table is None or block_table.dim() != 2 or block_table.shape[0] != b:
            raise ValueError("dense decode needs block_table int32 [batch, max_blocks_per_seq]")
        _need(block_table, "block_table", torch.int32, device=dev)
    else:
        if indices.dim() != 3 or tuple(indices.shape[:2]) != (b, s_q):
            raise ValueError(f"indices must be int32 [batch, s_q, topk], got {tuple(indices.shape)}")
        _need(indices, "indices", torch.int32, device=dev)
    _need(sched_meta, "sched_meta", torch.int32, device=dev)
    if sched_meta.dim() != 2 or sched_meta.shape[1] != 8:
        raise ValueError(f"sched_meta must be int32 [num_slots, 8], got {tuple(sched_meta.shape)}")
    _need(num_splits, "num_splits", torch.int32, device=dev)
    if num_splits.numel() < int(load_library().mla_num_splits_ints(b)):
        raise ValueError(f"num_splits holds {num_splits.numel()} ints, fewer than batch + 1")
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, device=dev)
    _need(out, "out", torch.uint8 if fused is not None else torch.bfloat16, (b, s_q, h_q, D_V), dev)
    _need(lse, "lse", torch.float32, (b, s_q, h_q), dev)
    if fused is not None:
        _need(fused["norm_weight"], "norm_weight", torch.bfloat16, (D_QK,), dev)
        _need(fused["out_scale"], "out_scale", torch.float32, (b, s_q, h_q), dev)
    p = DecodeParams()
    p.struct_size = ctypes.sizeof(DecodeParams)
    p.batch, p.s_q, p.h_q, p.h_kv, p.d_qk, p.d_v = b, s_q, h_q, 1, d_qk, D_V
    p.q = q.data_ptr()
    p.kv = kvcache.data_ptr()
    p.kv_format = KV_FORMATS[kv_format]
    p.page_size = kvcache.shape[1]
    p.num_blocks = kvcache.shape[0]
    if block_table is not None:
        p.block_table = block_table.data_ptr()
        p.max_blocks_per_seq = block_table.shape[1]
    p.cache_seqlens = cache_seqlens.data_ptr()
    p.softmax_scale = float(d_qk ** -0.5 if softmax_scale is None else softmax_scale)
    p.causal = int(bool(causal))
    if indices is not None:
        p.indices = indices.data_ptr()
        p.topk = indices.shape[-1]
    p.sched_meta = sched_meta.data_ptr()
    p.num_splits = num_splits.data_ptr()
    p.num_slots = sched_meta.shape[0]
    if workspace is not None:
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    p.out = out.data_ptr()
    p.lse = lse.data_ptr()
    if fused is not None:
        p.fused = 1
        p.norm_weight = fused["norm_weight"].data_ptr()
        p.norm_eps = float(fused.get("eps", 1e-6))
        p.rope_base = float(fused.get("rope_base", 10000.0))
        p.out_scale = fused["out_scale"].data_ptr()
    return p


def mla_decode_with_kvcache(q: torch.Tensor, kvcache: torch.Tensor, block_table: Optional[torch.Tensor],
                            cache_seqlens: torch.Tensor, dv: int, sched_meta: torch.Tensor,
                            num_splits: torch.Tensor, causal: bool = False,
                            indices: Optional[torch.Tensor] = None,
                            softmax_scale: Optional[float] = None, kv_format: str = "bf16",
                            workspace: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                            fused: Optional[dict] = None):
    """Paged MLA decode.  q bf16 [b, s_q, h_q, 576]; kvcache bf16
    [blocks, 64, 1, 576] / [blocks, 64, 576] or uint8 [blocks, 64, 656]
    (kv_format "fp8v32"), or with q [b, s_q, h_q, 512] a uint8
    [blocks, 64, 528] V4.1 cache (kv_format "fp8v41", sparse only);
    returns (o, lse) with o bf16 [b, s_q, h_q, 512]
    (uint8 e4m3 codes when fused) and lse fp32 [b, s_q, h_q].  Fused mode
    takes fused={"norm_weight": bf16 [576], "eps", "rope_base"} and also
    returns the per-row fp32 scale as a third value."""
    assert dv == D_V, "d_v must be 512"
    b, s_q, h_q, _ = q.shape
    dev = q.device
    if workspace is None:
        nbytes = workspace_bytes(b, s_q, h_q, sched_meta.shape[0])
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((b, s_q, h_q, D_V), dtype=torch.uint8 if fused is not None else torch.bfloat16,
                          device=dev)
    if lse is None:
        lse = torch.empty((b, s_q, h_q), dtype=torch.float32, device=dev)
    fz = None
    if fused is not None:
        fz = dict(fused)
        fz.setdefault("out_scale", torch.empty((b, s_q, h_q), dtype=torch.float32, device=dev))
    p = _params(q, kvcache, block_table, cache_seqlens, sched_meta, num_splits, causal, indices,
                softmax_scale, kv_format, workspace, out, lse, fz)
    _check(load_library().mla_decode(ctypes.byref(p), _stream(dev)))
    if fz is not None:
        return out, lse, fz["out_scale"]
    return out, lse


NOALLOC_SCRATCH_BYTES = 64 << 20


def mla_decode_noalloc(q: torch.Tensor, kvcache: torch.Tensor, block_table: Optional[torch.Tensor],
                       cache_seqlens: torch.Tensor, dv: int, sched_meta: torch.Tensor,
                       num_splits: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                       causal: bool = False, indices: Optional[torch.Tensor] = None,
                       softmax_scale: Optional[float] = None, kv_format: str = "bf16",
                       fused: Optional[dict] = None):
    """mla_decode_with_kvcache through the library's allocation-free entry
    point: the caller passes every output (out, lse, and fused["out_scale"]
    when fused) and no workspace; the split partials use the library's
    static per-GPU scratch array.  Calls that overlap on one GPU race."""
    assert dv == D_V, "d_v must be 512"
    p = _params(q, kvcache, block_table, cache_seqlens, sched_meta, num_splits, causal, indices,
                softmax_scale, kv_format, None, out, lse, fused)
    _check(load_library().mla_decode_noalloc(ctypes.byref(p), _stream(q.device)))
    if fused is not None:
        return out, lse, fused["out_scale"]
    return out, lse


def debug_gather(q, kvcache, block_table, cache_seqlens, sched_meta, num_splits, b, t, j,
                 indices=None, kv_format="bf16", workspace=None):
    """The bf16 [64, 576] tile the loader stages for work item j of sequence
    b (query token t when sparse)."""
    bsz, s_q, h_q, _ = q.shape
    dev = q.device
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(bsz, s_q, h_q, sched_meta.shape[0]), 256),
                                dtype=torch.uint8, device=dev)
    out = torch.empty((bsz, s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)  # not written
    lse = torch.empty((bsz, s_q, h_q), dtype=torch.float32, device=dev)
    p = _params(q, kvcache, block_table, cache_seqlens, sched_meta, num_splits, False, indices, None,
                kv_format, workspace, out, lse, None)
    dst = torch.empty((PAGE, D_QK), dtype=torch.bfloat16, device=dev)
    _check(load_library().mla_debug_gather(ctypes.byref(p), int(b), int(t), int(j), _ptr(dst),
                                           _stream(dev)))
    return dst
