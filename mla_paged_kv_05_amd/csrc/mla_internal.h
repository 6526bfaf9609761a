// Internal interface between the C ABI (mla_api.cpp) and the gfx950 kernels
// (mla_kernels.hip).  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace mla {

constexpr int kPage = 64;             // tokens per KV block
constexpr int kDqk = 576;             // 512 latent + 64 RoPE dims
constexpr int kDv = 512;              // V = K[:, :512]
constexpr int kRowsPerWg = 128;       // query rows one workgroup owns
constexpr int kWaves = 4;             // one wave per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kFp8TokenBytes = 656;
constexpr int kMaxBatch = 16384;
constexpr int kMaxRows = 65536;

// Piece cost F of the split rule (in 64-key items): the caller's value, or
// by default ceil(min(rows, 128) / 64), about two items at 128 rows (a
// plain piece's query load, pipeline fill and finalize).
inline int sched_piece_cost(int rows, int piece_cost) {
  if (piece_cost > 0) return piece_cost;
  int m = rows < kRowsPerWg ? rows : kRowsPerWg;
  int f = (m + 63) / 64;
  return f < 1 ? 1 : f;
}

// Row groups of 128 rows a decode call is cut into.
inline int row_groups(int rows) { return (rows + kRowsPerWg - 1) / kRowsPerWg; }

// The num_splits buffer: the prefix offsets of each sequence's splits [batch+1].
inline size_t splits_ints(int batch) { return (size_t)batch + 1; }

// Partial results of one (split, row group): 128 rows x 512 fp32 in the
// decode kernel's register order plus 128 fp32 LSEs.
constexpr size_t kPartialOElems = (size_t)kRowsPerWg * kDv;   // bf16 elements
constexpr size_t kPartialLseFloats = kRowsPerWg;

struct DecodeArgs {
  const uint16_t* q;         // bf16 [batch][rows][576]
  const uint8_t* kv;         // paged pool
  const int32_t* block_table;
  const int32_t* seqlens;
  const int32_t* indices;    // sparse only
  const int32_t* meta;       // [S][8]
  const int32_t* num_splits; // [batch+1] split prefix
  uint16_t* part_o;          // bf16 [max_partials][G][128*512] (register order)
  float* part_lse;           // [max_partials][G][128]
  void* out;                 // bf16 or e4m3 [batch][rows][512]
  float* lse;                // [batch][rows]
  float* out_scale;          // fused only
  const uint16_t* norm_w;    // fused only
  int64_t num_blocks;
  int batch, s_q, h_q, rows, groups, max_blocks, topk, causal, num_slots;
  float scale_log2;          // softmax_scale * log2(e)
  float norm_eps, rope_base;
  double rope_log2_base;     // fused only: log2(rope_base), in fp64
};

enum KvFormat { kKvBf16 = 0, kKvFp8V32 = 1, kKvFp8V41 = 2 };
constexpr int kFp8V41TokenBytes = 528;  // 512 e4m3 codes (all dims) + 16 e8m0 scales

// Size of the static scratch array behind mla_decode_noalloc: the partials
// of up to 510 (split, row group) pairs.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
// Device address of the current device's scratch array (looked up once).
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_sched(const int32_t* seqlens, int batch, int piece_cost, int topk, int num_slots,
                        int32_t* meta, int32_t* num_splits, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int kv_format, bool sparse, bool fused,
                         hipStream_t stream, hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
hipError_t launch_combine(const DecodeArgs& a, bool fused, hipStream_t stream);
hipError_t launch_debug_gather(const DecodeArgs& a, int kv_format, bool sparse, int b, int t,
                               int j, uint16_t* dst, hipStream_t stream);

}  // namespace mla
