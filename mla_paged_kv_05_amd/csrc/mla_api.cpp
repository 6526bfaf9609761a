// C ABI of libmla.so: argument validation, workspace sizing and kernel
// launches for paged MLA decoding (see include/mla.h for the contract).
// Validation reads scalar arguments only; nothing here reads device memory
// or synchronises the host.
#include "mla.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "mla_internal.h"

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mla_status hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Per-device compute-unit counts, filled on first use.
std::mutex g_dev_mu;
std::vector<int> g_cu_count;

int cu_count(int device) {
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (device < 0) return 0;
  if ((int)g_cu_count.size() <= device) g_cu_count.resize(device + 1, 0);
  if (g_cu_count[device] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
      return 0;
    g_cu_count[device] = n;
  }
  return g_cu_count[device];
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t partials_max(int32_t batch, int32_t num_slots) { return (size_t)batch + (size_t)num_slots; }

}  // namespace

extern "C" {

int32_t mla_num_sched_slots(int32_t device, int32_t rows_per_kv_head) {
  if (rows_per_kv_head < 1) return 0;
  const int cus = cu_count(device);
  if (cus <= 0) return 0;
  const int G = mla::row_groups(rows_per_kv_head);
  if (G == 1) return cus;
  int s = cus / G / 8 * 8;  // row groups of a slot share an XCD: slots in multiples of 8
  return s < 8 ? 8 : s;
}

size_t mla_sched_meta_ints(int32_t num_slots) { return num_slots > 0 ? 8 * (size_t)num_slots : 0; }

size_t mla_num_splits_ints(int32_t batch) { return batch >= 0 ? mla::splits_ints(batch) : 0; }

mla_status mla_get_metadata(const int32_t* cache_seqlens, int32_t batch, int32_t rows_per_kv_head,
                            int32_t h_kv, int32_t topk, int32_t num_slots, int32_t piece_cost,
                            int32_t* sched_meta, int32_t* num_splits, void* stream) {
  if (batch < 0 || rows_per_kv_head < 1 || num_slots < 1 || topk < 0 || piece_cost < 0 ||
      piece_cost > MLA_MAX_PIECE_COST)
    return fail(MLA_ERR_INVALID_ARG, "mla_get_metadata: batch=%d rows=%d num_slots=%d topk=%d piece_cost=%d",
                batch, rows_per_kv_head, num_slots, topk, piece_cost);
  if (h_kv != 1) return fail(MLA_ERR_UNSUPPORTED, "mla_get_metadata: h_kv=%d (only 1)", h_kv);
  if (batch > MLA_MAX_BATCH)
    return fail(MLA_ERR_UNSUPPORTED, "mla_get_metadata: batch %d > %d", batch, MLA_MAX_BATCH);
  if (!sched_meta || !num_splits || (batch > 0 && !cache_seqlens))
    return fail(MLA_ERR_INVALID_ARG, "mla_get_metadata: null pointer");
  hipError_t e = mla::launch_sched(cache_seqlens, batch, mla::sched_piece_cost(rows_per_kv_head, piece_cost),
                                   topk, num_slots, sched_meta, num_splits, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mla_get_metadata launch");
  return MLA_OK;
}

size_t mla_workspace_bytes(int32_t batch, int32_t s_q, int32_t h_q, int32_t num_slots) {
  if (batch < 0 || s_q < 1 || h_q < 1 || num_slots < 1) return 0;
  const size_t G = (size_t)mla::row_groups(s_q * h_q);
  const size_t P = partials_max(batch, num_slots) * G;
  return P * (mla::kPartialOElems * sizeof(uint16_t) + mla::kPartialLseFloats * sizeof(float));
}

static mla_status build_args(const mla_decode_params* p, mla::DecodeArgs& a, bool& sparse) {
  if (!p) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
  if (p->struct_size != sizeof(mla_decode_params))
    return fail(MLA_ERR_INVALID_ARG, "struct_size %u != %zu", p->struct_size, sizeof(mla_decode_params));
  if (p->batch < 0 || p->s_q < 1 || p->h_q < 1)
    return fail(MLA_ERR_INVALID_ARG, "batch=%d s_q=%d h_q=%d", p->batch, p->s_q, p->h_q);
  if (p->h_kv != 1) return fail(MLA_ERR_UNSUPPORTED, "h_kv=%d (only 1)", p->h_kv);
  if (p->kv_format == MLA_KV_FP8_V41) {
    if (p->d_qk != MLA_D_QK_V41) return fail(MLA_ERR_UNSUPPORTED, "d_qk=%d (the V4.1 format has 512)", p->d_qk);
  } else if (p->d_qk != MLA_D_QK) {
    return fail(MLA_ERR_UNSUPPORTED, "d_qk=%d (only 576)", p->d_qk);
  }
  if (p->d_v != MLA_D_V) return fail(MLA_ERR_UNSUPPORTED, "d_v=%d (only 512)", p->d_v);
  if (p->page_size != MLA_PAGE_SIZE) return fail(MLA_ERR_UNSUPPORTED, "page_size=%d (only 64)", p->page_size);
  if (p->kv_format != MLA_KV_BF16 && p->kv_format != MLA_KV_FP8_V32 && p->kv_format != MLA_KV_FP8_V41)
    return fail(MLA_ERR_INVALID_ARG, "kv_format=%d", p->kv_format);
  if (p->kv_format == MLA_KV_FP8_V41 && (!p->indices || p->fused))
    return fail(MLA_ERR_UNSUPPORTED, "the V4.1 FP8 format is decoded sparse (indices) and unfused only");
  const int64_t rows = (int64_t)p->s_q * p->h_q;
  if (rows > mla::kMaxRows) return fail(MLA_ERR_UNSUPPORTED, "s_q*h_q=%lld > %d", (long long)rows, mla::kMaxRows);
  if (p->batch > MLA_MAX_BATCH) return fail(MLA_ERR_UNSUPPORTED, "batch %d > %d", p->batch, MLA_MAX_BATCH);
  // an empty batch reads and writes none of the per-sequence arrays, so
  // they may be NULL then (zero-size tensors have no address)
  const bool empty = p->batch == 0;
  if (!empty && (!p->q || !p->kv || !p->out || !p->lse || !p->cache_seqlens))
    return fail(MLA_ERR_INVALID_ARG, "q, kv, out, lse and cache_seqlens must be non-NULL");
  if (!aligned(p->q, 16) || !aligned(p->kv, 16) || !aligned(p->out, 16))
    return fail(MLA_ERR_INVALID_ARG, "q, kv and out must be 16-byte aligned");
  if (p->flags & ~MLA_FLAG_DEFER_COMBINE)
    return fail(MLA_ERR_INVALID_ARG, "unknown flags 0x%x", p->flags);
  if (p->num_blocks < 0) return fail(MLA_ERR_INVALID_ARG, "num_blocks=%lld", (long long)p->num_blocks);
  if (!(p->softmax_scale > 0.f) || !std::isfinite(p->softmax_scale))
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be positive and finite (got %g)", (double)p->softmax_scale);
  sparse = p->indices != nullptr;
  if (sparse) {
    if (p->topk < 1) return fail(MLA_ERR_INVALID_ARG, "topk=%d with indices", p->topk);
    if (p->causal) return fail(MLA_ERR_INVALID_ARG, "causal must be 0 with sparse indices");
    if (!(p->s_q == 1 || p->h_q % mla::kRowsPerWg == 0))
      return fail(MLA_ERR_UNSUPPORTED, "sparse needs s_q == 1 or h_q %% 128 == 0 (s_q=%d h_q=%d)",
                  p->s_q, p->h_q);
  } else {
    if ((!empty && !p->block_table) || p->max_blocks_per_seq < 1)
      return fail(MLA_ERR_INVALID_ARG, "dense decode needs block_table and max_blocks_per_seq >= 1");
    if (p->topk != 0) return fail(MLA_ERR_INVALID_ARG, "topk=%d without indices", p->topk);
  }
  if (p->fused) {
    if (!p->norm_weight || !p->out_scale || !aligned(p->norm_weight, 16))
      return fail(MLA_ERR_INVALID_ARG, "fused needs a 16-byte aligned norm_weight and out_scale");
    if (!(p->rope_base > 0.f) || !(p->norm_eps >= 0.f))
      return fail(MLA_ERR_INVALID_ARG, "fused needs rope_base > 0 and norm_eps >= 0");
  }
  if (!p->sched_meta || !p->num_splits || p->num_slots < 1)
    return fail(MLA_ERR_INVALID_ARG, "sched_meta, num_splits and num_slots >= 1 are required");
  const int G = mla::row_groups((int)rows);
  if (G > 1 && p->num_slots % 8 != 0)
    return fail(MLA_ERR_INVALID_ARG, "num_slots %d must be a multiple of 8 when s_q*h_q > 128",
                p->num_slots);
  const size_t need = mla_workspace_bytes(p->batch, p->s_q, p->h_q, p->num_slots);
  if (!p->workspace || p->workspace_bytes < need || !aligned(p->workspace, 256))
    return fail(MLA_ERR_WORKSPACE, "workspace: need %zu bytes (256-byte aligned), got %zu", need,
                p->workspace_bytes);

  const size_t P = partials_max(p->batch, p->num_slots) * G;
  a.q = static_cast<const uint16_t*>(p->q);
  a.kv = static_cast<const uint8_t*>(p->kv);
  a.block_table = p->block_table;
  a.seqlens = p->cache_seqlens;
  a.indices = p->indices;
  a.meta = p->sched_meta;
  a.num_splits = p->num_splits;
  a.part_o = static_cast<uint16_t*>(p->workspace);
  a.part_lse = reinterpret_cast<float*>(a.part_o + P * mla::kPartialOElems);
  a.out = p->out;
  a.lse = p->lse;
  a.out_scale = p->out_scale;
  a.norm_w = static_cast<const uint16_t*>(p->norm_weight);
  a.num_blocks = p->num_blocks;
  a.batch = p->batch;
  a.s_q = p->s_q;
  a.h_q = p->h_q;
  a.rows = (int)rows;
  a.groups = G;
  a.max_blocks = sparse ? 0 : p->max_blocks_per_seq;
  a.topk = sparse ? p->topk : 0;
  a.causal = p->causal ? 1 : 0;
  a.num_slots = p->num_slots;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  a.norm_eps = p->norm_eps;
  a.rope_base = p->rope_base;
  a.rope_log2_base = std::log2((double)p->rope_base);
  return MLA_OK;
}

static mla_status decode_impl(const mla_decode_params* p, void* stream, hipEvent_t start,
                              hipEvent_t stop) {
  mla::DecodeArgs a{};
  bool sparse = false;
  mla_status st = build_args(p, a, sparse);
  if (st != MLA_OK) return st;
  if (p->batch == 0) return MLA_OK;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = mla::launch_decode(a, p->kv_format, sparse, p->fused != 0, s, start, stop);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (p->flags & MLA_FLAG_DEFER_COMBINE) return MLA_OK;
  e = mla::launch_combine(a, p->fused != 0, s);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return MLA_OK;
}

mla_status mla_decode(const mla_decode_params* p, void* stream) {
  return decode_impl(p, stream, nullptr, nullptr);
}

mla_status mla_decode_timed(const mla_decode_params* p, void* stream, void* start_event,
                            void* stop_event) {
  return decode_impl(p, stream, (hipEvent_t)start_event, (hipEvent_t)stop_event);
}

mla_status mla_decode_noalloc(const mla_decode_params* p, void* stream) {
  if (!p) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
  if (p->flags != 0)
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_noalloc takes no flags (got 0x%x)", p->flags);
  const size_t need = mla_workspace_bytes(p->batch, p->s_q, p->h_q, p->num_slots);
  if (need > mla::kNoAllocScratchBytes)
    return fail(MLA_ERR_WORKSPACE,
                "mla_decode_noalloc: the call needs %zu bytes of scratch, the static array holds %zu "
                "(batch + num_slots split partials per 128-row group); use mla_decode with a workspace",
                need, (size_t)mla::kNoAllocScratchBytes);
  void* scratch = nullptr;
  hipError_t e = mla::noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "scratch symbol lookup");
  mla_decode_params q = *p;
  q.workspace = scratch;
  q.workspace_bytes = mla::kNoAllocScratchBytes;
  return decode_impl(&q, stream, nullptr, nullptr);
}

mla_status mla_combine(const mla_decode_params* p, void* stream) {
  mla::DecodeArgs a{};
  bool sparse = false;
  mla_status st = build_args(p, a, sparse);
  if (st != MLA_OK) return st;
  if (p->batch == 0) return MLA_OK;
  hipError_t e = mla::launch_combine(a, p->fused != 0, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return MLA_OK;
}

mla_status mla_debug_gather(const mla_decode_params* p, int32_t b, int32_t t, int32_t j, void* dst,
                            void* stream) {
  mla::DecodeArgs a{};
  bool sparse = false;
  mla_status st = build_args(p, a, sparse);
  if (st != MLA_OK) return st;
  if (p->kv_format == MLA_KV_FP8_V41)
    return fail(MLA_ERR_UNSUPPORTED, "mla_debug_gather: not available for the V4.1 FP8 format");
  if (!dst || b < 0 || b >= p->batch || t < 0 || t >= p->s_q || j < 0 ||
      (!sparse && j >= p->max_blocks_per_seq) || (sparse && j * MLA_PAGE_SIZE >= p->topk))
    return fail(MLA_ERR_INVALID_ARG, "mla_debug_gather: bad (b=%d, t=%d, j=%d) or dst", b, t, j);
  hipError_t e = mla::launch_debug_gather(a, p->kv_format, sparse, b, t, j,
                                          static_cast<uint16_t*>(dst), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "debug gather launch");
  return MLA_OK;
}

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
