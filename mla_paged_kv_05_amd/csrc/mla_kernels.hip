// gfx950 (CDNA4) kernels for paged MLA decoding.
//
// What is computed: for each query row (sequence b, token t, head h) the
// softmax attention of a 576-dim query over the sequence's latent KV head
// held in a paged cache of 64-token blocks, V being the first 512 dims of K;
// outputs O and the log-sum-exp ("FlashMLA", AI Wiki, sections "What is
// FlashMLA?" and "How is FlashMLA designed?"; Ampere-adaptation README,
// section "Usage").  The work of a sequence may be split over several
// workgroups along the KV length; the partial results are merged by their
// LSEs in a second kernel.
//
// Design for MI355X (not a translation of any CUDA kernel):
//  * One workgroup = 4 waves (one per SIMD) owning 128 query rows; wave w
//    owns rows 32w..32w+31 for both contractions, so every per-row
//    operation (mask, max, sum, rescale, epilogue) stays inside the pair of
//    lanes (l, l+32) that hold the row.
//  * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: K (from LDS) is the A
//    operand, Q^T lives in registers as the B operand (36 fragments).  The
//    accumulator layout of S^T is directly the B operand layout P^T of the
//    second product, so P never goes through LDS.
//  * O^T = V^T . P^T: V^T fragments come from the same LDS tile as K via
//    ds_read_b64_tr_b16 transposed reads (V = K[:, :512], no second load).
//  * KV blocks are staged half a block (32 tokens) at a time with LDS-DMA
//    (buffer_load ... lds, 16 B per lane) into a ring of padded, swizzled
//    bf16 half tiles, two steps ahead of their use.  The buffer
//    resource of a block covers only its valid tokens, so rows past the
//    sequence length are written as zeros by the hardware and poisoned
//    (NaN) tail slots are never read.
//  * Lazy rescaling: the running max used for exponentiation only moves
//    when a new block max exceeds it by more than 2^8, so the 256-register
//    O accumulator is almost never rescaled ("skip scale", AI Wiki, section
//    "The Ascend kernel deep-dive"); exact up to rounding.
//  * The fused variant (q RMSNorm + RoPE in the piece prologue, conjugate
//    RoPE + amax + e4m3 cast in the epilogue, "FlashMLA fused norm-RoPE-
//    attention-RoPE-cast kernel" card) runs both products on fp16 operands
//    (v_mfma_f32_32x32x16_f16): q-hat is rounded once to fp16, and each
//    wave converts the bf16 rows it staged to fp16 in place.
//  * FP8 caches: V3.2 records (e4m3 codes with an fp32 scale per 128 dims)
//    dequantise to fp16 tiles, code * scale rounded once, and run on fp16
//    MFMA with q converted to fp16; V4.1 records (power-of-two scales)
//    dequantise exactly to bf16.
//  * Split rows: the decode stores bf16 partial O and fp32 partial LSE; the
//    combine (k_combine) merges them on one 64-lane workgroup per 32x32 tile
//    of O (four waves sharing the splits when few row groups have many).
//    The fused path merges and runs the row epilogue (rotated, scaled e4m3
//    output) in the same launch, or, with few row groups, leaves fp32 tiles
//    that k_fused_epilogue turns into that output.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <cstdint>
#include <cmath>
#include <mutex>
#include <vector>

#include "mla_internal.h"

namespace mla {

// ---------------------------------------------------------------------------
// Phase timeline, compiled only into the measurement library that
// build.build_phase_trace() makes (-DMLA_PHASE_TRACE); the product library
// has none of it.  Lane 0 of wave 0 of each workgroup records the 100 MHz
// s_memrealtime clock at kernel start, at each piece's start, after its
// prologue, after its main loop and at its end (up to kTrPieces pieces), and
// at kernel end (and, in the first piece, after the slot's metadata read and
// the fused prologue's two passes), with vector stores into a static array that
// mla_phase_trace_copy() returns.  Wave 0 also sums the shader clock
// (s_memtime) spent in each phase of its 32-key steps (kTrSteps phases:
// load wait; barrier, with the fused fp16 conversion or the one-tile FP8
// dequantisation; load issue; S^T, with the next tile's dequantisation on
// the two-tile FP8 path; softmax; P.V issue) into slots kTrStepOff..,
// and its step count after them.
// ---------------------------------------------------------------------------
#ifdef MLA_PHASE_TRACE
constexpr int kTrPieces = 7, kTrPer = 40, kTrWgs = 4096, kTrSteps = 6, kTrStepOff = 32;
__device__ uint64_t g_phase_t[kTrWgs * kTrPer];
__device__ int g_phase_items[kTrWgs * kTrPieces];
#define MLA_TR_KERNEL_START                                                               \
  const uint64_t tr_t0 = __builtin_amdgcn_s_memrealtime();                                \
  int tr_p = 0;                                                                           \
  uint64_t tr_acc[kTrSteps] = {};                                                         \
  uint64_t tr_last = 0;                                                                   \
  int tr_steps = 0;
#define MLA_ST_BEGIN do { tr_last = __builtin_amdgcn_s_memtime(); } while (0)
#define MLA_ST(i)                                                                         \
  do {                                                                                    \
    const uint64_t t_ = __builtin_amdgcn_s_memtime();                                     \
    tr_acc[i] += t_ - tr_last;                                                            \
    tr_last = t_;                                                                         \
  } while (0)
#define MLA_ST_STEP do { ++tr_steps; } while (0)
// First piece only: a stamp once `dep` is computed (the scalar-memory wait
// also drains outstanding LDS operations), in slot k (29: the slot's
// metadata read; fused prologue 30: pass 1's row sum, 31: pass 2 done).
#define MLA_TR_FIRST(k, cons, dep)                                                        \
  do {                                                                                    \
    asm volatile("" ::cons(dep));                                                         \
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");                                    \
    if (threadIdx.x == 0 && blockIdx.x < kTrWgs && tr_p == 0)                             \
      g_phase_t[blockIdx.x * kTrPer + (k)] = __builtin_amdgcn_s_memrealtime();            \
  } while (0)
#define MLA_TR_WG_ACTIVE \
  if (threadIdx.x == 0 && blockIdx.x < kTrWgs) g_phase_t[blockIdx.x * kTrPer] = tr_t0;
#define MLA_TR(k)                                                                              \
  do {                                                                                         \
    if (threadIdx.x == 0 && blockIdx.x < kTrWgs && tr_p < kTrPieces)                          \
      g_phase_t[blockIdx.x * kTrPer + 4 * tr_p + (k)] = __builtin_amdgcn_s_memrealtime();    \
  } while (0)
#define MLA_TR_ITEMS(n)                                                                        \
  do {                                                                                         \
    if (threadIdx.x == 0 && blockIdx.x < kTrWgs && tr_p < kTrPieces)                          \
      g_phase_items[blockIdx.x * kTrPieces + tr_p] = (n);                                      \
  } while (0)
#define MLA_TR_NEXT_PIECE ++tr_p;
#define MLA_TR_KERNEL_END                                                                 \
  if (threadIdx.x == 0 && blockIdx.x < kTrWgs) {                                          \
    g_phase_t[blockIdx.x * kTrPer + kTrPer - 1] = __builtin_amdgcn_s_memrealtime();       \
    for (int i_ = 0; i_ < kTrSteps; ++i_) g_phase_t[blockIdx.x * kTrPer + kTrStepOff + i_] = tr_acc[i_]; \
    g_phase_t[blockIdx.x * kTrPer + kTrStepOff + kTrSteps] = (uint64_t)tr_steps;          \
  }
#else
#define MLA_TR_KERNEL_START
#define MLA_TR_WG_ACTIVE
#define MLA_TR(k) do {} while (0)
#define MLA_TR_ITEMS(n) do {} while (0)
#define MLA_TR_NEXT_PIECE
#define MLA_TR_KERNEL_END
#define MLA_ST_BEGIN do {} while (0)
#define MLA_ST(i) do {} while (0)
#define MLA_ST_STEP do {} while (0)
#define MLA_TR_FIRST(k, cons, dep) do {} while (0)
#endif

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((ext_vector_type(2))) short s16x2;

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kRowBytes = kDqk * 2;             // 1152
constexpr int kChunksPerRow = kDqk / 8;         // 72 chunks of 16 B
constexpr int kTileBytes = kPage * kRowBytes;   // 73728
constexpr int kTileChunks = kPage * kChunksPerRow;  // 4608
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;       // log2 units
constexpr uint32_t kBufferFlags = 0x00020000u;  // raw buffer, dword3 for gfx9 family

// Values every lane of the wave holds identically (sequence, block and
// slot indices): move them to scalar registers so buffer descriptors, LDS
// bases and loop bounds stay scalar.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uni_u64(uint64_t v) {
  return ((uint64_t)(uint32_t)uni((int)(v >> 32)) << 32) | (uint32_t)uni((int)(uint32_t)v);
}
// Buffer stores with cache policy sc0 sc1 go past the CU's L1 and the XCD's
// L2 to the memory side.  The split partials are stored this way: lines left
// dirty in L2 would be written back while the next launch streams its KV.
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
constexpr int kPastL2 = 1 | 16;  // sc0 sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// A wave-uniform pointer, forced into SGPRs (for "s" asm operands).
template <typename T>
__device__ __forceinline__ const T* uni_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// Read-only int32 arrays indexed by wave-uniform values (schedule, lengths,
// block table): read through the constant address space so they become
// scalar loads (lgkmcnt), not vector loads whose vmcnt wait would also wait
// for the KV prefetch in flight.
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
__device__ __forceinline__ int sload(const int32_t* p, int64_t i) {
  return ((cint_ptr)(p))[i];
}

// Workgroup barrier for the KV pipeline: waits for this wave's LDS traffic
// only.  __syncthreads() would also drain every outstanding vector memory
// op, i.e. the prefetch of the next two steps.  KV arrival is awaited
// explicitly with vmcnt before this barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS-DMA (global -> LDS, 16 or 4 bytes per lane at M0 + 16*lane) issued as
// inline asm.  Through the builtins the compiler treats every later LDS read
// as possibly aliasing the DMA and waits for all vector memory first, which
// would stall on the KV prefetch each step.  Completion of these loads is
// awaited explicitly (vmcnt) before the barrier that publishes a step.
typedef __attribute__((ext_vector_type(4))) int i32x4;
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)nbytes);                           // num_records
  r[3] = (int)kBufferFlags;
  return r;
}
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint8_t*)p));
}
__device__ __forceinline__ void dma_buf16(uint32_t lds, int voff, i32x4 rs) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rs) : "memory", "m0");
}
__device__ __forceinline__ void dma_buf4(uint32_t lds, int voff, i32x4 rs) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rs) : "memory", "m0");
}
__device__ __forceinline__ void dma_glb16(uint32_t lds, const void* g) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(g) : "memory", "m0");
}

// An opaque copy of a per-lane value: loader address arithmetic derived from
// it is recomputed at each use instead of being hoisted out of the KV loop
// (where 18+ hoisted offsets would only crowd the register file).
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
// The same for a wave-uniform value: e.g. a divisor whose reciprocal would
// otherwise be hoisted to the kernel's start and spilled.
__device__ __forceinline__ int opaque_s(int v) {
  asm volatile("" : "+s"(v));
  return v;
}
// This lane's index, recomputed (mbcnt) where it is used, so per-lane LDS
// address bases live only inside a step, never across the KV loop: there the
// allocator may spill them, and each reload of a spill would cost a full
// vmcnt wait in a loop that keeps KV loads in flight.
__device__ __forceinline__ int fresh_lane() {
  return opaque(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
}

// S^T = K Q^T step on v_mfma_f32_32x32x16 with the accumulator held in
// VGPRs.  Written as inline asm because the builtin lets the compiler move
// every MFMA accumulator to AGPRs, and the 256 AGPRs are exactly the O
// accumulator of a 32-row wave tile; S then overflows and spills.  The asm is
// not volatile, so the scheduler still hoists the LDS reads feeding it.
// F16 selects the fp16 operand form (the fused path over an FP8 cache),
// otherwise bf16; the operands are eight 16-bit values either way.
template <bool F16>
__device__ __forceinline__ void mfma_s_first(f32x16& c, const bf16x8& a, const bf16x8& b) {
  if constexpr (F16) asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
  else asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
template <bool F16>
__device__ __forceinline__ void mfma_s_acc(f32x16& c, const bf16x8& a, const bf16x8& b) {
  if constexpr (F16) asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  else asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// O^T += V^T P^T step with the accumulator pinned to AGPRs for its whole
// life (a builtin leaves O's register class to the allocator, which then
// shuffles the 256 accumulators between VGPRs and AGPRs inside the loop).
// Back-to-back accumulation into the same registers needs no wait states.
template <bool F16>
__device__ __forceinline__ void mfma_o(f32x16& c, const bf16x8& a, const bf16x8& b) {
  if constexpr (F16) asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// One fp32 value as the 16-bit MFMA operand element, round to nearest even:
// bf16, or fp16 (F16).
template <bool F16>
__device__ __forceinline__ __bf16 to_op16(float x) {
  if constexpr (F16) return __builtin_bit_cast(__bf16, (_Float16)x);
  else return (__bf16)x;
}
// VALU-written B operand -> MFMA read.
__device__ __forceinline__ void valu_to_mfma_settle(bf16x8& p0, bf16x8& p1) {
  asm volatile("s_nop 4" : "+v"(p0), "+v"(p1));
}
// Last MFMA into O -> VALU / accvgpr reads of O (finalize): 24 wait states,
// more than a 32x32 XDL op's write -> read requirement.
__device__ __forceinline__ void o_settle(f32x16 (&o)[16]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                 "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]),
                 "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15]));
}
// The hardware does not interlock a VALU read of an MFMA result; the compiler
// inserts those wait states for builtins but cannot see into the asm above,
// so S is passed through 24 explicit wait states before any VALU use (more
// than the XDL-write -> VALU-read requirement of a 32x32 op).
__device__ __forceinline__ void mfma_s_settle(f32x16& c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c));
}

// Max / sum over the lane pair (l, l ^ 32) that holds one query row:
// v_permlane32_swap leaves {v[l], v[l ^ 32]} in the two results of every lane.
__device__ __forceinline__ float row_max2(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_sum2(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// Split-KV scheduler (one workgroup).  Implements the split rule stated in
// mla.h; every per-sequence quantity is a prefix sum, every slot finds its
// first item by binary search, so there is no serial walk.  Batches of up to
// kSchedSmallBatch sequences run on a single wave, whose scans need no
// cross-wave barrier; larger ones on 1024 threads.
// ---------------------------------------------------------------------------
constexpr int kSchedSmallBatch = 256;

template <int NT>
__device__ int block_scan_exclusive(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if constexpr (NT == 64) {
    *total = __shfl(x, 63, 64);
    return x - v;
  } else {
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    if (w == 0) {
      int s = lane < NT / 64 ? wsum[lane] : 0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(s, o, 64);
        if (lane >= o) s += y;
      }
      if (lane < NT / 64) wsum[lane] = s;
    }
    __syncthreads();
    int base = w > 0 ? wsum[w - 1] : 0;
    *total = wsum[NT / 64 - 1];
    __syncthreads();
    return base + x - v;
  }
}

template <int NT, int MAXB>
__global__ void __launch_bounds__(NT)
k_sched(const int32_t* __restrict__ seqlens, int B, int F, int topk, int S,
        int32_t* __restrict__ meta, int32_t* __restrict__ num_splits) {
  constexpr int kSchedThreads = NT;
  __shared__ int32_t U[MAXB + 1];   // cost prefix: start of sequence b on the line
  __shared__ int32_t I[MAXB + 1];   // item prefix
  __shared__ int wsum[NT / 64];
  const int tid = threadIdx.x;
  const int per = (B + kSchedThreads - 1) / kSchedThreads;
  const int lo = tid * per, hi = min(B, lo + per);
  auto nblk = [&](int b) -> int {
    if (topk > 0) return (topk + kPage - 1) / kPage;
    int L = seqlens[b];
    return L > 0 ? (L + kPage - 1) / kPage : 0;
  };
  // pass 1: U and I
  int cs = 0, is = 0;
  for (int b = lo; b < hi; ++b) {
    int n = nblk(b);
    cs += F + n;
    is += n > 0 ? n : 1;
  }
  int tot_c, tot_i;
  int c0 = block_scan_exclusive<NT>(cs, wsum, &tot_c);
  int i0 = block_scan_exclusive<NT>(is, wsum, &tot_i);
  for (int b = lo; b < hi; ++b) {
    int n = nblk(b);
    U[b] = c0;
    I[b] = i0;
    c0 += F + n;
    i0 += n > 0 ? n : 1;
  }
  if (tid == 0) {
    U[B] = tot_c;
    I[B] = tot_i;
  }
  __syncthreads();
  const int T = tot_c;
  const int cap = (T + 1 + S - 1) / S;
  // pass 2: splits per sequence -> num_splits prefix
  int ss = 0;
  for (int b = lo; b < hi; ++b) {
    int items = U[b + 1] - U[b] - F;
    items = items > 0 ? items : 1;
    int p0 = U[b] + F;
    ss += (p0 + items - 1) / cap - p0 / cap + 1;
  }
  int tot_s;
  int s0 = block_scan_exclusive<NT>(ss, wsum, &tot_s);
  for (int b = lo; b < hi; ++b) {
    num_splits[b] = s0;
    int items = U[b + 1] - U[b] - F;
    items = items > 0 ? items : 1;
    int p0 = U[b] + F;
    s0 += (p0 + items - 1) / cap - p0 / cap + 1;
  }
  if (tid == 0) num_splits[B] = tot_s;
  // pass 3: each slot's first and last item
  auto last_pos = [&](int b) {  // position of the last item of sequence b
    int n = U[b + 1] - U[b] - F;
    return U[b] + F + (n > 0 ? n : 1) - 1;
  };
  // first item at position >= x, as (b, j); b == B if none
  auto first_at = [&](int x, int& b, int& j) {
    int l = 0, h = B;  // find the first b with last_pos(b) >= x
    while (l < h) {
      int mid = (l + h) >> 1;
      if (last_pos(mid) >= x) h = mid; else l = mid + 1;
    }
    b = l;
    if (l < B) {
      int p0 = U[l] + F;
      j = x > p0 ? x - p0 : 0;
    } else {
      j = 0;
    }
  };
  for (int s = tid; s < S; s += kSchedThreads) {
    int32_t* ms = meta + 8 * s;
    int ba, ja, bz, jz;
    first_at(s * cap, ba, ja);
    first_at((s + 1) * cap, bz, jz);
    bool empty = (ba >= B) || (U[ba] + F + ja >= (s + 1) * cap);
    if (empty) {
      ms[0] = -1; ms[1] = 0; ms[2] = -1; ms[3] = 0; ms[4] = 0; ms[5] = 0; ms[6] = 0; ms[7] = 0;
      continue;
    }
    // last item = the one before (bz, jz)
    int bl, jl;
    if (jz > 0) { bl = bz; jl = jz - 1; }
    else {
      bl = bz - 1;
      int n = U[bl + 1] - U[bl] - F;
      jl = (n > 0 ? n : 1) - 1;
    }
    ms[0] = ba; ms[1] = ja; ms[2] = bl; ms[3] = jl + 1;
    ms[4] = s - (U[ba] + F) / cap;
    ms[5] = (I[bl] + jl + 1) - (I[ba] + ja);
    ms[6] = 0; ms[7] = 0;
  }
}

// ---------------------------------------------------------------------------
// KV staging.  The unit of work is a half block of 32 tokens.  A bf16 half
// tile in LDS has two parts:
//   main  [32][1040 B]: token r's dims 0..511 at r*1040 (1024 B + 16 B pad);
//   rope  [32][128 B] at kRopeOff: token r's dims 512..575, 16-byte chunk c
//         at r*128 + ((c ^ ((r >> 1) & 7)) << 4).
// The 16-byte pad turns every main row into a one-bank-group shift, and the
// S^T rows are bound to keys in the order key_of_row() below, so the
// 16-lane phases of the K reads (16 keys, one chunk) and the 32-lane phases
// of the transposed V reads (keys b, b+4, b+8, b+12 x 4 chunks) both touch
// 16 distinct 4-bank groups: no bank conflicts, and each read stream needs a
// single per-lane base address plus immediates.  bf16 half tiles rotate
// through a ring of kTileRing slots: one is computed on while the next
// kDepth are in flight.
// ---------------------------------------------------------------------------
constexpr int kHalfRows = 32;
constexpr int kMainStride = 1040;
constexpr int kRopeOff = kHalfRows * kMainStride;               // 33280
constexpr int kRopeStride = 128;
constexpr int kHalfBytes = kRopeOff + kHalfRows * kRopeStride;  // 37376
constexpr int kLoadsPerHalf = kHalfRows / kWaves + 1;           // 9 per wave: 8 rows + rope
// bf16 tiles are prefetched kDepth steps ahead into a ring of kDepth + 1
// slots.  A CU holds ~40 KB of loads in flight before their issue blocks;
// two steps (one half page landing, one issued) keep it there.
constexpr int kDepth = 2;
constexpr int kTileRing = kDepth + 1;  // bf16 half-tile slots
constexpr int kRing = 3;      // FP8 raw slots

// The key held by row m (0..31) of an S^T tile (and by k-slot m of the
// matching P^T / V^T operands): keys 4j+c of a 16-row block sit at rows
// 4c+j, so 4 consecutive rows hold keys 4 apart.
__host__ __device__ constexpr int key_of_row(int m) {
  return 16 * (m >> 4) + 4 * (m & 3) + ((m >> 2) & 3);
}
__device__ __forceinline__ int rope_phys_chunk(int r, int c) { return c ^ ((r >> 1) & 7); }

// All-zero source for rows that hold no token (masked sparse entries).
__device__ __attribute__((aligned(16))) const uint8_t g_zero_row[kRowBytes] = {0};

// global -> LDS with a wave-uniform 64-bit base and a 32-bit per-lane offset.
__device__ __forceinline__ void dma_glb16_s(uint32_t lds, int voff, const void* sbase) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
}

// Dense bf16: half `h` of pool block `phys` whose first `valid` tokens are
// real.  The buffer resource covers exactly those tokens, so the hardware
// writes zeros for the others and never reads past the sequence (valid = 0
// writes a zero half).  A wave's 9 loads: k < 8 stages main row wave + 4k
// (1 KB), k = 8 the rope rows 8*wave .. 8*wave+7.
__device__ __forceinline__ void load_row_bf16_dense(uint8_t* slot, const uint8_t* kv, int64_t phys,
                                                    int valid, int h, int wave, int k) {
  const int l16 = fresh_lane() << 4;
  const i32x4 rs = make_rsrc(kv + phys * (int64_t)kTileBytes, valid * kRowBytes);
  const uint32_t base = lds_off(slot);
  if (k < kHalfRows / kWaves) {
    const int r = wave + kWaves * k;
    dma_buf16(base + r * kMainStride, (h * kHalfRows + r) * kRowBytes + l16, rs);
  } else {
    const int rr = 8 * wave + (l16 >> 7);
    dma_buf16(base + kRopeOff + wave * 1024,
              (h * kHalfRows + rr) * kRowBytes + 1024 + (rope_phys_chunk(rr, (l16 >> 4) & 7) << 4), rs);
  }
}
__device__ __forceinline__ void load_half_bf16_dense(uint8_t* slot, const uint8_t* kv, int64_t phys,
                                                     int valid, int h, int wave, int /*lane*/) {
#pragma unroll
  for (int k = 0; k < kLoadsPerHalf; ++k) load_row_bf16_dense(slot, kv, phys, valid, h, wave, k);
}

// A sparse id names a token of the pool iff 0 <= id < ntok (= num_blocks *
// 64); -1 and every other id outside the pool are masked.
__device__ __forceinline__ bool id_in_pool(int id, int64_t ntok) { return id >= 0 && (int64_t)id < ntok; }

// Sparse bf16: row r is flat pool token ids[r] when r < nvalid and the id
// is in the pool, else zeros.  Same 9 loads per wave as the dense loader
// (k < 8: main row wave + 4k, one id for the whole wave; k = 8: the rope
// rows, one id per lane).  Every id is read before the first load: a load's
// "memory" clobber keeps later LDS reads behind it, so reading each id just
// before its load would wait out one LDS latency per load.
__device__ __forceinline__ void load_half_bf16_sparse(uint8_t* slot, const uint8_t* kv, int64_t ntok,
                                                      const int32_t* ids, int nvalid, int wave, int /*lane*/) {
  const int l16 = fresh_lane() << 4;
  const uint32_t base = lds_off(slot);
  const int rr = 8 * wave + (l16 >> 7);
  int id[kLoadsPerHalf];
#pragma unroll
  for (int k = 0; k < kLoadsPerHalf - 1; ++k) {
    const int r = wave + kWaves * k;
    id[k] = r < nvalid ? ids[r] : -1;
  }
  id[kLoadsPerHalf - 1] = rr < nvalid ? ids[rr] : -1;
#pragma unroll
  for (int k = 0; k < kLoadsPerHalf - 1; ++k) {
    const int r = wave + kWaves * k;
    const int idk = uni(id[k]);
    const uint8_t* src = uni_ptr(id_in_pool(idk, ntok) ? kv + (int64_t)idk * kRowBytes : g_zero_row);
    dma_glb16_s(base + r * kMainStride, l16, src);
  }
  const int cc = rope_phys_chunk(rr, (l16 >> 4) & 7);
  const int idr = id[kLoadsPerHalf - 1];
  const uint8_t* g = id_in_pool(idr, ntok) ? kv + (int64_t)idr * kRowBytes + 1024 + cc * 16
                                           : g_zero_row + 1024 + cc * 16;
  dma_glb16(base + kRopeOff + wave * 1024, g);
}

// FP8 V3.2 records of one half (32 x 656 B = 1312 chunks) are staged raw by
// LDS-DMA into a 24 KB slot (24 loads per half, 6 per wave; the tail of the
// slot is padding), then dequantised LDS -> LDS into a 16-bit half tile
// (fp16 for V3.2 records, bf16 for V4.1).  V4.1 records (32 x 528 B = 1056
// chunks) use the same slot with 20 loads.
constexpr int kRawSlotBytes = 24 * 1024;
constexpr int kRawLoadsPerWave = kRawSlotBytes / 1024 / kWaves;  // 6
template <int KVF>
constexpr int tok_bytes() { return KVF == kKvFp8V41 ? kFp8V41TokenBytes : kFp8TokenBytes; }
template <int KVF>
constexpr int raw_loads_per_wave() {  // 1 KB loads per wave covering a half's records
  return (kHalfRows * tok_bytes<KVF>() / 16 + 64 * kWaves - 1) / (64 * kWaves);
}
static_assert(raw_loads_per_wave<kKvFp8V32>() == kRawLoadsPerWave, "V3.2 slot");
static_assert(raw_loads_per_wave<kKvFp8V41>() * kWaves * 1024 <= kRawSlotBytes, "V4.1 slot");

__device__ __forceinline__ void load_half_fp8_dense(uint8_t* raw, const uint8_t* kv, int64_t phys,
                                                    int valid, int h, int wave, int lane) {
  lane = fresh_lane();
  const uint8_t* page = kv + phys * (int64_t)(kPage * kFp8TokenBytes);
  const i32x4 rs = make_rsrc(page, valid * kFp8TokenBytes);
  const uint32_t base = lds_off(raw);
#pragma unroll
  for (int ii = 0; ii < kRawLoadsPerWave; ++ii) {
    const int i = ii * kWaves + wave;
    dma_buf16(base + i * 1024, h * kHalfRows * kFp8TokenBytes + (i * 64 + lane) * 16, rs);
  }
}

template <int KVF = kKvFp8V32>
__device__ __forceinline__ void load_half_fp8_sparse(uint8_t* raw, const uint8_t* kv, int64_t ntok,
                                                     const int32_t* ids, int nvalid, int wave,
                                                     int lane) {
  constexpr int kTok = tok_bytes<KVF>(), kChunks = kTok / 16, kHalfChunks = kHalfRows * kChunks;
  lane = fresh_lane();
  // every id first, as in the bf16 loader
  constexpr int kLoads = raw_loads_per_wave<KVF>();
  int id[kLoads];
#pragma unroll
  for (int ii = 0; ii < kLoads; ++ii) {
    const int pos_all = (ii * kWaves + wave) * 64 + lane;
    const int r = pos_all / kChunks;
    id[ii] = (pos_all < kHalfChunks && r < nvalid) ? ids[r] : -1;
  }
#pragma unroll
  for (int ii = 0; ii < kLoads; ++ii) {
    const int i = ii * kWaves + wave;
    const int pos_all = i * 64 + lane;
    const int c = pos_all - (pos_all / kChunks) * kChunks;
    const uint64_t rec = reinterpret_cast<uint64_t>(kv) + (uint64_t)((int64_t)id[ii] * kTok + c * 16);
    const uint64_t zero = reinterpret_cast<uint64_t>(uni_ptr(g_zero_row)) + (uint32_t)((pos_all & 63) * 16);
    const uint8_t* g = reinterpret_cast<const uint8_t*>(id_in_pool(id[ii], ntok) ? rec : zero);
    dma_glb16(lds_off(raw) + i * 1024, g);
  }
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two bf16 values -> two fp16 values, round to nearest even (one
// v_cvt_pk_f16_f32 after widening): exact for magnitudes in [2^-14, 65504].
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const f32x2_t f = {__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
}
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v) {
  return make_uint4(bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w));
}
// The fused path over a bf16 cache runs its products on fp16: each wave
// converts in place exactly the chunks its own loads staged in a half tile
// (main rows wave + 4k, k < 8, and its 1 KB of RoPE rows), right after its
// own load wait, so the conversion needs no barrier of its own: the step's
// barrier that follows publishes it to the other waves.
__device__ __forceinline__ void own_chunks_to_f16(uint8_t* slot, int wave) {
  const int l16 = fresh_lane() << 4;
  uint4 v[kLoadsPerHalf];
#pragma unroll
  for (int k = 0; k < kLoadsPerHalf; ++k) {
    const int off = k < kHalfRows / kWaves ? (wave + kWaves * k) * kMainStride : kRopeOff + wave * 1024;
    v[k] = *reinterpret_cast<const uint4*>(slot + off + l16);
  }
#pragma unroll
  for (int k = 0; k < kLoadsPerHalf; ++k) {
    const int off = k < kHalfRows / kWaves ? (wave + kWaves * k) * kMainStride : kRopeOff + wave * 1024;
    *reinterpret_cast<uint4*>(slot + off + l16) = bf16x8_to_f16x8(v[k]);
  }
}
// 32 raw V3.2 records -> the fp16 half tile both products read: dims < 512
// as fp16(fp32(code) * scale) (the e4m3 code widened exactly to fp32, one
// fp32 product with the record's fp32 scale of that 128-dim block, rounded
// once to fp16 (relative error below 2^-11); the hardware's scaled
// conversion uses only the scale's exponent, so the product is formed
// here), dims 512..575 converted from bf16 (exact for magnitudes in
// [2^-14, 65504]).  An all-zero record gives a zero row.  Used by the
// decode and, unchanged, by the gather test hook.
__device__ __forceinline__ uint4 codes_to_f16x8(uint32_t c0, uint32_t c1, float sc) {
  const uint32_t cw[2] = {c0, c1};
  uint32_t w[4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(cw[hh], false);
    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(cw[hh], true);
    w[2 * hh] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo * sc, f16x2_t));
    w[2 * hh + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi * sc, f16x2_t));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}
// Thread (wave w, lane l) converts chunk kk*256 + 64w + l of the half's
// 32 x 64 code chunks: record 4kk + w, codes 8l..8l+7 (block l/16), and the
// 16 bytes of RoPE dims at record 8w + l/8, chunk l%8.  The record index is
// uniform, so every address is a wave-uniform base, the lane's offset and an
// immediate.
__device__ __forceinline__ void dequant_codes(uint8_t* tile, const uint8_t* raw, int tid) {
  const int wave = uni(tid >> 6), ln = fresh_lane();  // lane id not held across the loop
  // All code and scale reads first, then the conversions and writes: the
  // compiler cannot move a read of the raw slot above a write to the tile
  // (same LDS array), so interleaved they would each wait out an LDS latency.
  constexpr int kPer = kHalfRows * 64 / kThreads;
  uint2 codes[kPer];
  float scl[kPer];
#pragma unroll
  for (int kk = 0; kk < kPer; ++kk) {
    const uint8_t* rec = raw + (kk * kWaves + wave) * kFp8TokenBytes;
    codes[kk] = *reinterpret_cast<const uint2*>(rec + ln * 8);
    scl[kk] = *reinterpret_cast<const float*>(rec + 512 + 4 * (ln >> 4));
  }
  const int rr = wave * 8 + (ln >> 3), rc = ln & 7;
  uint4 rope = *reinterpret_cast<const uint4*>(raw + rr * kFp8TokenBytes + 528 + rc * 16);
#pragma unroll
  for (int kk = 0; kk < kPer; ++kk)
    *reinterpret_cast<uint4*>(tile + (kk * kWaves + wave) * kMainStride + ln * 16) =
        codes_to_f16x8(codes[kk].x, codes[kk].y, scl[kk]);
  *reinterpret_cast<uint4*>(tile + kRopeOff + rr * kRopeStride + (rope_phys_chunk(rr, rc) << 4)) =
      bf16x8_to_f16x8(rope);
}

// The same conversion one chunk at a time, for spreading it between the
// MFMAs of another step's S^T: chunk kk < 8 is 8 codes of a record and
// their block scale (the dequant_codes loop's chunk kk), chunk 8 the 8 RoPE
// dims this thread converts.
constexpr int kV32Chunks = kHalfRows * 64 / kThreads + 1;  // 9
static_assert(4 * kV32Chunks == 36, "one V3.2 chunk per four S^T k-steps");
__device__ __forceinline__ uint4 v32_read(const uint8_t* raw, int wave, int kk) {
  const int ln = fresh_lane();
  if (kk < kV32Chunks - 1) {
    const uint8_t* rec = raw + (kk * kWaves + wave) * kFp8TokenBytes;
    const uint2 c = *reinterpret_cast<const uint2*>(rec + ln * 8);
    return make_uint4(c.x, c.y, *reinterpret_cast<const uint32_t*>(rec + 512 + 4 * (ln >> 4)), 0u);
  }
  return *reinterpret_cast<const uint4*>(raw + (wave * 8 + (ln >> 3)) * kFp8TokenBytes + 528 + (ln & 7) * 16);
}
__device__ __forceinline__ void v32_write(uint8_t* tile, int wave, int kk, uint4 ch) {
  const int ln = fresh_lane();
  if (kk < kV32Chunks - 1) {
    *reinterpret_cast<uint4*>(tile + (kk * kWaves + wave) * kMainStride + ln * 16) =
        codes_to_f16x8(ch.x, ch.y, __uint_as_float(ch.z));
  } else {
    const int r = wave * 8 + (ln >> 3), c = ln & 7;
    *reinterpret_cast<uint4*>(tile + kRopeOff + r * kRopeStride + (rope_phys_chunk(r, c) << 4)) = bf16x8_to_f16x8(ch);
  }
}

// e8m0 scale -> fp32 2^(e-127), branch-free (one v_ldexp_f32).  Codes 0..254
// are exact (0 gives the fp32 subnormal 2^-127); the NaN code 0xFF gives
// +inf, so a record with it still turns its keys non-finite.
__device__ __forceinline__ float e8m0_scale(uint32_t e) { return __builtin_ldexpf(1.0f, (int)e - 127); }

// 32 raw V4.1 records -> the bf16 half tile's 512 main dims.  Every scale
// is a power of two, 2^(e-127) (e8m0), so code * scale is a bf16 value and
// each conversion (two codes, the scale folded in) is exact; no scale is
// kept for later.  Code reads go out before any tile write, as above.
__device__ __forceinline__ void dequant_v41(uint8_t* tile, const uint8_t* raw, int tid) {
  const int wave = uni(tid >> 6), ln = fresh_lane();  // chunks as in dequant_codes
  constexpr int kPer = kHalfRows * 64 / kThreads;
  uint2 codes[kPer];
  uint32_t ebits[kPer];
#pragma unroll
  for (int kk = 0; kk < kPer; ++kk) {
    const uint8_t* rec = raw + (kk * kWaves + wave) * kFp8V41TokenBytes;
    codes[kk] = *reinterpret_cast<const uint2*>(rec + ln * 8);
    ebits[kk] = rec[512 + (ln >> 2)];  // 8 codes of dims 8l.. share scale l/4
  }
#pragma unroll
  for (int kk = 0; kk < kPer; ++kk) {
    const int r = kk * kWaves + wave, c = ln;
    const float scale = e8m0_scale(ebits[kk]);
    const uint32_t cw[2] = {codes[kk].x, codes[kk].y};
    uint32_t w[4];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      w[2 * hh] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[hh], scale, false));
      w[2 * hh + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[hh], scale, true));
    }
    *reinterpret_cast<uint4*>(tile + r * kMainStride + c * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// The same conversion one chunk at a time (chunk kk: 8 codes per thread),
// for spreading it between the MFMAs of another step's S^T.
struct V41Chunk {
  uint2 code;
  uint32_t e;
};
__device__ __forceinline__ V41Chunk v41_read(const uint8_t* raw, int wave, int kk) {
  const int ln = fresh_lane();
  const uint8_t* rec = raw + (kk * kWaves + wave) * kFp8V41TokenBytes;
  return V41Chunk{*reinterpret_cast<const uint2*>(rec + ln * 8), rec[512 + (ln >> 2)]};
}
__device__ __forceinline__ void v41_write(uint8_t* tile, int wave, int kk, const V41Chunk& ch) {
  const int ln = fresh_lane();
  const float scale = e8m0_scale(ch.e);
  const uint32_t cw[2] = {ch.code.x, ch.code.y};
  uint32_t w[4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    w[2 * hh] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[hh], scale, false));
    w[2 * hh + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[hh], scale, true));
  }
  *reinterpret_cast<uint4*>(tile + (kk * kWaves + wave) * kMainStride + ln * 16) = make_uint4(w[0], w[1], w[2], w[3]);
}

// The 32 sparse ids of half `h` of work item j of (sequence b, query token
// t) -> LDS (one LDS-DMA dword per lane; lanes past topk read 0 and are
// excluded by position, never by value).
__device__ __forceinline__ void fetch_ids_dma(int32_t* ids_lds, const int32_t* indices,
                                              int64_t row_off, int topk, int j, int h) {
  const int first = j * kPage + h * kHalfRows;
  const int32_t* base = indices + row_off + first;
  const int n = max(0, min(kHalfRows, topk - first));
  dma_buf4(lds_off(ids_lds), fresh_lane() << 2, make_rsrc(base, n * 4));  // lane id not held across the loop
}

// ---------------------------------------------------------------------------
// Fused prologue / epilogue helpers.  The RoPE angle of pair i at position
// pos is theta = pos * base^(-2i/64), the inverse frequency formed in fp64
// on the device.  Positions reach 10^4 radians, so theta is formed and
// reduced by quarter turns in fp64 (pi/2 as hi + lo); the remainder
// |r| <= pi/4 is then exact to ~1e-12 and goes to fp32, where Taylor series
// (sin to r^9, cos to r^10: truncation below 2e-9) give sin and cos to about
// 3e-7 absolute.  Light on registers, unlike a general sincosf with its
// large-argument path, and unlike the same series in fp64.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rope_cs(double pos, double inv_freq, float sign, float& c, float& s) {
  const double th = (double)sign * pos * inv_freq;
  const double q = rint(th * 0.63661977236758138);                                     // th / (pi/2)
  const float r = (float)((th - q * 1.5707963267948966) - q * 6.123233995736766e-17);  // |r| <= pi/4
  const float r2 = r * r;
  const float sp = r * (1.0f + r2 * (-1.0f / 6 + r2 * (1.0f / 120 + r2 * (-1.0f / 5040 + r2 * (1.0f / 362880)))));
  const float cp = 1.0f + r2 * (-0.5f + r2 * (1.0f / 24 + r2 * (-1.0f / 720 + r2 * (1.0f / 40320 +
                   r2 * (-1.0f / 3628800)))));
  const int qi = (int)(int64_t)q & 3;  // th = r + qi * pi/2 (mod 2 pi)
  s = qi == 0 ? sp : qi == 1 ? cp : qi == 2 ? -sp : -cp;
  c = qi == 0 ? cp : qi == 1 ? -sp : qi == 2 ? -cp : sp;
}

// RoPE angles of one wave's rows.  A lane needs pair i0 when it holds the
// low half of its row's dims and i1 for the high half.  Lane l forms the
// inverse frequency of pair l & 31 once, and the other lanes read it by
// lane index (so no lane evaluates exp2 for every pair).  When every row of
// the wave sits at one position (always with one query token per sequence),
// each of the 32 angles is computed once, pair lane & 31 on each lane, and
// read back by lane index too; otherwise each lane computes its own pairs.
struct RopeRow {
  bool shared;
  double pos;
  double inv;  // inverse frequency of pair lane & 31
  float c, s;
};
// Inverse frequency of pair i: base^(-2i/64) = 2^(-(i/32) log2(base)), in fp64.
__device__ __forceinline__ double rope_inv_freq(int i, double log2_base) { return exp2(-(double)i / 32.0 * log2_base); }
// inv: the inverse frequency of pair lane & 31 (rope_inv_freq), formed once
// per launch by the caller.
__device__ __forceinline__ RopeRow rope_row(double pos, bool row_ok, double inv, float sign) {
  RopeRow r;
  const double pos0 = __builtin_bit_cast(double, uni_u64(__builtin_bit_cast(uint64_t, pos)));
  r.shared = __builtin_amdgcn_ballot_w64(row_ok && pos != pos0) == 0;
  r.pos = pos;
  r.inv = inv;
  r.c = 0.f;
  r.s = 0.f;
  if (r.shared) rope_cs(pos0, r.inv, sign, r.c, r.s);
  return r;
}
// i0 and i1 are the same on every lane of the wave (read by lane index).
__device__ __forceinline__ void rope_pair(const RopeRow& r, float sign, int i0, int i1, bool hi, float& c,
                                          float& s) {
  if (r.shared) {
    const float c0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r.c), i0));
    const float c1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r.c), i1));
    const float s0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r.s), i0));
    const float s1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r.s), i1));
    c = hi ? c1 : c0;
    s = hi ? s1 : s0;
  } else {
    rope_cs(r.pos, __shfl(r.inv, hi ? i1 : i0, 64), sign, c, s);
  }
}
// The same where i0 and i1 may differ between lanes of the wave (readlane
// needs one lane index for the whole wave; a lane shuffle does not).
__device__ __forceinline__ void rope_pair_lanes(const RopeRow& r, float sign, int i0, int i1, bool hi, float& c,
                                                float& s) {
  const int i = hi ? i1 : i0;
  if (r.shared) {
    c = __shfl(r.c, i, 64);
    s = __shfl(r.s, i, 64);
  } else {
    rope_cs(r.pos, __shfl(r.inv, i, 64), sign, c, s);
  }
}

// ---------------------------------------------------------------------------
// Decode kernel
//
// Query fragments.  bf16 KV: all 36 k-steps stay in VGPRs (144), which
// leaves the LDS to the tile ring.  FP8 KV, whose dequantisation
// and per-tile scaling need more registers: dims 0..383 (k-steps 0..23) in
// VGPRs, dims 384..575 (k-steps 24..35) in a per-wave LDS region
// [32 rows][24 chunks] swizzled like the KV tile.
// ---------------------------------------------------------------------------
// k-steps of 16 dims in a query row: d_qk = 576, or 512 for V4.1 records
template <int KVF>
constexpr int ksteps() { return KVF == kKvFp8V41 ? 32 : 36; }
template <int KVF>
constexpr int dqk_of() { return 16 * ksteps<KVF>(); }
// The fused path (whose prologue and epilogue need the registers) keeps
// k-steps 24..35 of the query in LDS; every other path holds all of it in
// VGPRs.
template <int KVF, bool FUSED>
constexpr int q_reg_steps() { return FUSED ? 24 : ksteps<KVF>(); }
template <int KVF, bool FUSED>
constexpr int q_lds_row_bytes() { return (ksteps<KVF>() - q_reg_steps<KVF, FUSED>()) * 2 * 16; }  // 384 or 0
template <int KVF, bool FUSED>
constexpr int q_lds_wave_bytes() { return 32 * q_lds_row_bytes<KVF, FUSED>(); }                 // 12288 or 0
// FP8 records: unfused, a step dequantises the next step's records into a
// second tile between its own S^T MFMAs, and raw records go out three steps
// ahead; the fused V3.2 path (its query half in LDS leaves room for one
// tile only) dequantises each step's records before its S^T, two ahead.
template <int KVF, bool FUSED>
constexpr bool dq_ahead() { return KVF != kKvBf16 && !FUSED; }
template <int KVF, bool FUSED>
constexpr int raw_ahead() { return dq_ahead<KVF, FUSED>() ? 3 : 2; }
// Sparse id slots: ids are fetched 4 steps ahead on bf16 KV and two steps
// before the FP8 records that use them, and a slot is rewritten only after
// the step that last read it.
template <int KVF, bool FUSED>
constexpr int ids_slots() { return KVF == kKvBf16 ? 5 : raw_ahead<KVF, FUSED>() + 3; }

template <int KVF, bool SPARSE, bool FUSED>
struct DecodeLayout {
  static constexpr int kTileOff = 0;                                   // 16-bit half tiles
  static constexpr int kTiles = KVF == kKvBf16 ? kTileRing : dq_ahead<KVF, FUSED>() ? 2 : 1;
  static constexpr int kRawOff = kTiles * kHalfBytes;                  // fp8 raw slots
  static constexpr int kQOff = kRawOff + (KVF == kKvBf16 ? 0 : kRing * kRawSlotBytes);
  static constexpr int kIdsOff = kQOff + kWaves * q_lds_wave_bytes<KVF, FUSED>();
  static constexpr int kWalkOff = kIdsOff + (SPARSE ? ids_slots<KVF, FUSED>() * 256 : 0);  // 2 words per wave
  static constexpr int kWOff = kWalkOff + (KVF == kKvBf16 && !SPARSE ? kWaves * 8 : 0);  // fused: norm weight row
  static constexpr int kSmem = kWOff + (FUSED ? kDqk * 2 : 0);
  // per-step VMEM instructions issued by every wave (loads + id fetch)
  static constexpr int kVmPerStep =
      (KVF == kKvBf16 ? kLoadsPerHalf : raw_loads_per_wave<KVF>()) + (SPARSE ? 1 : 0);
};

__device__ __forceinline__ int seq_items(const DecodeArgs& a, int b) {
  if (a.topk > 0) return (a.topk + kPage - 1) / kPage;
  int L = uni(sload(a.seqlens, b));
  return L > 0 ? (L + kPage - 1) / kPage : 0;
}

// s_waitcnt with only a vmcnt limit (expcnt and lgkmcnt left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int KVF, bool SPARSE, bool FUSED>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_decode(DecodeArgs a) {
  MLA_TR_KERNEL_START
  using Lay = DecodeLayout<KVF, SPARSE, FUSED>;
  // The fused path runs both products on fp16 operands: q-hat is formed in
  // fp32 and rounded once, to fp16 (3 more bits than bf16), so QK^T meets
  // the LSE bar even on rows of a few keys; bf16 K/V and e4m3 codes convert
  // to fp16 exactly, and P keeps 3 more bits too.
  constexpr bool kF16 = FUSED || KVF == kKvFp8V32;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Lay::kSmem];

  const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
  const int half = lane >> 5, r32 = lane & 31;

  // blockIdx -> (slot, row group).  Workgroup w runs on XCD w % 8; XCD x
  // gets the consecutive slots x*S/8 .. (x+1)*S/8 - 1, and the G row groups
  // of one slot are dispatched back to back onto it.  Consecutive slots
  // mostly hold the middle splits of one sequence, which start together and
  // read the same query rows, and the row groups of a slot read the same KV:
  // both meet in that XCD's L2.  (S % 8 == 0 is required when G > 1; with
  // G == 1 and other S the slots are taken in workgroup order.)
  int slot, g;
  {
    const int G = a.groups, wg = blockIdx.x, S = a.num_slots;
    const int xcd = wg & 7, k = wg >> 3;
    if (G == 1) {
      g = 0;
      slot = (S & 7) ? wg : xcd * (S >> 3) + k;
    } else {
      g = k % G;
      slot = xcd * (S >> 3) + k / G;
    }
  }
  const int32_t* ms = a.meta + 8 * slot;
  const int b0 = uni(sload(ms, 0));
  if (b0 < 0) return;  // no work in this slot
  MLA_TR_WG_ACTIVE
  const int j0 = uni(sload(ms, 1)), b1 = uni(sload(ms, 2)), j1 = uni(sload(ms, 3)),
            nitems = uni(sload(ms, 5));
  int split_k = uni(sload(ms, 4));
  MLA_TR_FIRST(29, "s", split_k);
  const int nsteps = 2 * nitems;

  // this lane's query row within the sequence
  const int row = g * kRowsPerWg + wave * 32 + r32;
  const bool row_ok = row < a.rows;
  const int tok = row_ok ? row / a.h_q : 0;
  const int gtok = (g * kRowsPerWg) / a.h_q;   // sparse: the row group's query token

  auto item_end = [&](int b) { return b == b1 ? j1 : max(seq_items(a, b), 1); };
  // step -> (sequence, item, half) by walking forward from a known step
  auto advance = [&](int& b, int& j, int& h) {
    if (h == 0) { h = 1; return; }
    h = 0;
    ++j;
    if (j >= item_end(b)) { ++b; j = 0; }
    b = uni(b); j = uni(j);
  };
  auto ids_slot = [&](int step) {
    return reinterpret_cast<int32_t*>(smem + Lay::kIdsOff) + (step % ids_slots<KVF, FUSED>()) * 64;
  };
  auto fetch_ids = [&](int b, int j, int h, int step) {
    if constexpr (SPARSE)
      fetch_ids_dma(ids_slot(step), a.indices, ((int64_t)b * a.s_q + gtok) * a.topk, a.topk, j, h);
  };
  // Load walker: (lb, lj, lh) is the next step to stage, lL and lend the
  // length and item count of sequence lb, lphys the physical block of item
  // (lb, lj).  On the bf16 dense path the block of a new item and the length
  // of the next sequence are fetched a step before they are needed, by
  // one-lane LDS-DMA loads into two words of the wave's own, and read back by
  // land() after the step-start vmcnt(0) wait and barrier.  Neither scalar
  // loads (an SMEM load in flight turns every LDS-operand wait of the MFMA
  // loops into a full lgkmcnt(0) drain) nor vector loads into VGPRs (a
  // compiler wait on them, or on a spill of their register, also waits for
  // the KV loads it cannot see) would do.  The FP8 path, whose waits keep a
  // step of KV loads in flight, uses scalar loads when it needs the values.
  // Indices are not trusted to stay inside the pool: a block_table entry
  // outside [0, num_blocks) stages a zero page, a sparse id outside
  // [0, num_blocks * 64) is masked like -1.  Nothing is read past the pool.
  const int64_t ntok = a.num_blocks * kPage;
  auto page_in_pool = [&](int64_t phys) { return phys >= 0 && phys < a.num_blocks; };
  constexpr bool kVecWalk = KVF == kKvBf16 && !SPARSE;
  int lb = b0, lj = j0, lh = 0;
  int lL = SPARSE ? 0 : uni(sload(a.seqlens, b0));
  int lend = item_end(b0);
  int lphys = 0, lnL = 0;
  bool lany = false;
  const int32_t* walk = reinterpret_cast<const int32_t*>(smem + Lay::kWalkOff) + 2 * wave;
  const i32x4 bt_rs = make_rsrc(a.block_table, kVecWalk ? (uint32_t)((int64_t)a.batch * a.max_blocks * 4) : 0u);
  const i32x4 sl_rs = make_rsrc(a.seqlens, kVecWalk ? (uint32_t)(a.batch * 4) : 0u);
  auto fetch_word = [&](int w, const i32x4& rs, int byte_off) {
    if (lane == 0) dma_buf4(lds_off(walk + w), byte_off, rs);
  };
  // lphys = -1 when the item has no block_table entry (past the sequence,
  // or positions beyond max_blocks_per_seq pages): its page stages zeros.
  auto fetch_phys = [&]() {
    const bool any = lb <= b1 && lj * kPage < lL && lj < a.max_blocks;
    if constexpr (kVecWalk) {
      lany = any;
      if (any) fetch_word(0, bt_rs, (lb * a.max_blocks + lj) * 4);
    } else if constexpr (!SPARSE) {
      lphys = any ? uni(sload(a.block_table, (int64_t)lb * a.max_blocks + lj)) : -1;
    }
  };
  auto fetch_next_len = [&]() {
    if constexpr (kVecWalk) fetch_word(1, sl_rs, min(lb + 1, b1) * 4);
  };
  auto land = [&]() {
    if constexpr (kVecWalk) {
      lphys = lany ? uni(walk[0]) : -1;
      lnL = uni(walk[1]);
    }
  };
  auto advance_load = [&]() {
    if (lh == 0) { lh = 1; return; }
    lh = 0;
    ++lj;
    if (lj >= lend) {
      ++lb;
      lj = 0;
      const int bq = min(lb, b1);  // nothing past the slot's last sequence is staged
      if constexpr (kVecWalk) {
        lL = lnL;
        fetch_next_len();
        lend = lb == b1 ? j1 : max((lL + kPage - 1) / kPage, 1);
      } else {
        if constexpr (!SPARSE) lL = uni(sload(a.seqlens, bq));
        lend = item_end(bq);
      }
    }
    lb = uni(lb);
    lj = uni(lj);
    fetch_phys();
  };
  fetch_phys();
  fetch_next_len();
  // The plain dense decode reads its first walker words in the first
  // piece's prologue, once its query loads are out; the fused one here.
  constexpr bool kLateLand = kVecWalk && !FUSED;
  if constexpr (kVecWalk && !kLateLand) {
    __builtin_amdgcn_s_waitcnt(0);  // kernel start: nothing else is in flight yet
    lds_barrier();
  }
  if constexpr (!kLateLand) land();
  // stage the walker's step as step `step` into its ring slot
  auto issue_load = [&](int step) {
    const int rs = step % (KVF == kKvBf16 ? kTileRing : kRing);
    if constexpr (!SPARSE) {
      const bool any = lj * kPage < lL && page_in_pool(lphys);
      const int valid = any ? min(kPage, lL - lj * kPage) : 0;
      const int64_t phys = any ? lphys : 0;
      if constexpr (KVF == kKvBf16)
        load_half_bf16_dense(smem + Lay::kTileOff + rs * kHalfBytes, a.kv, phys, valid, lh, wave, lane);
      else
        load_half_fp8_dense(smem + Lay::kRawOff + rs * kRawSlotBytes, a.kv, phys, valid, lh, wave, lane);
    } else {
      const int nvalid = min(kHalfRows, a.topk - lj * kPage - lh * kHalfRows);
      if constexpr (KVF == kKvBf16)
        load_half_bf16_sparse(smem + Lay::kTileOff + rs * kHalfBytes, a.kv, ntok, ids_slot(step), nvalid,
                              wave, lane);
      else
        load_half_fp8_sparse<KVF>(smem + Lay::kRawOff + rs * kRawSlotBytes, a.kv, ntok, ids_slot(step),
                                  nvalid, wave, lane);
    }
  };

  // bf16 path: the loads of step+kDepth are captured by prepare_load() at
  // the start of step `step` and issued by emit_loads() (kLoadsPerHalf loads),
  // after the walker's and the ids' word loads of that step.  Past the
  // slot's last step the same instructions stage zeros into the free slot,
  // so every step issues exactly kLoadsPerHalf tile loads, last.  (Issuing
  // the nine loads between the MFMAs, or after S^T, was measured: no gain.)
  int pl_step = 0, pl_valid = 0, pl_h = 0, pl_nvalid = 0;
  int64_t pl_phys = 0;
  auto prepare_load = [&](int st) {
    const bool do_load = st < nsteps;
    pl_step = st;
    pl_h = lh;
    if constexpr (!SPARSE) {
      const bool any = do_load && lj * kPage < lL && page_in_pool(lphys);
      pl_valid = any ? min(kPage, lL - lj * kPage) : 0;
      pl_phys = any ? lphys : 0;
    } else {
      pl_nvalid = do_load ? min(kHalfRows, a.topk - lj * kPage - lh * kHalfRows) : 0;
    }
    if (do_load) advance_load();
  };
  auto emit_loads = [&]() {
    uint8_t* slot = smem + Lay::kTileOff + (pl_step % kTileRing) * kHalfBytes;
    if constexpr (!SPARSE) {
#pragma unroll
      for (int k = 0; k < kLoadsPerHalf; ++k) load_row_bf16_dense(slot, a.kv, pl_phys, pl_valid, pl_h, wave, k);
    } else {
      load_half_bf16_sparse(slot, a.kv, ntok, ids_slot(pl_step), pl_nvalid, wave, 0);
    }
  };

  // loads of step+2 and (sparse) ids of step+4, issued at step `step`
  int fb = b0, fj = j0, fh = 0;   // next step whose ids to fetch
  auto fetch_next_ids = [&](int step) {
    if constexpr (SPARSE) {
      if (step + 4 < nsteps) {
        fetch_ids(fb, fj, fh, step + 4);
        advance(fb, fj, fh);
      }
    }
  };
  // FP8 loads lead by kRawAhead steps, ids by kRawAhead + 2
  constexpr int kRawAhead = raw_ahead<KVF, FUSED>();
  auto issue_next = [&](int step) {
    if (step + kRawAhead < nsteps) {
      issue_load(step + kRawAhead);
      advance_load();
    }
    if constexpr (SPARSE) {
      if (step + kRawAhead + 2 < nsteps) {
        fetch_ids(fb, fj, fh, step + kRawAhead + 2);
        advance(fb, fj, fh);
      }
    }
  };

  // ---- prologue: the ids of the first steps (4 on bf16 KV, kRawAhead + 2
  // on FP8); the loads of the first kDepth (bf16) or kRawAhead (FP8) steps
  // are issued in the first piece's prologue (bf16: right after the query
  // loads)
  if constexpr (SPARSE) {
    for (int s = 0; s < min(KVF == kKvBf16 ? 4 : kRawAhead + 2, nsteps); ++s) {
      fetch_ids(fb, fj, fh, s);
      advance(fb, fj, fh);
    }
    // plain FP8 decodes wait for these ids in the first piece's prologue,
    // with its query loads in flight
    if constexpr (KVF == kKvBf16 || FUSED) __builtin_amdgcn_s_waitcnt(0);
  }
  auto issue_first_loads = [&]() {
    for (int s = 0; s < min(KVF == kKvBf16 ? kDepth : kRawAhead, nsteps); ++s) {
      issue_load(s);
      advance_load();
    }
  };
  if constexpr (KVF != kKvBf16 && FUSED) issue_first_loads();

  constexpr int kQR = q_reg_steps<KVF, FUSED>();
  uint8_t* qlds = smem + Lay::kQOff + wave * q_lds_wave_bytes<KVF, FUSED>();
  // FP8: Q rows are 384 B apart (an 8-group shift): chunk c of row r at
  // c ^ ((r >> 1) & 7) puts the 16 rows of a read phase on distinct groups
  const int x = (r32 >> 1) & 7;
  bf16x8 qf[kQR];
  f32x16 o[16];
  bool first_piece = true;

  // fused RoPE: the inverse frequency of pair lane & 31, once per launch
  // (inside the piece loop the compiler hoists the fp64 exp2 anyway, with
  // its constants spilled and each reload waiting for every load in flight)
  const double rope_inv = FUSED ? rope_inv_freq(lane & 31, a.rope_log2_base) : 0.0;

  int cb = b0, cj = j0, step = 0;
  while (step < nsteps) {
    // ======== one piece: sequence cb, items cj .. piece_end-1
    MLA_TR(1);
    const int Lb = uni(sload(a.seqlens, cb));
    const int piece_end = item_end(cb);
    float m_used = -INFINITY, lsum = 0.f;
    int vis_end = 0;  // dense: keys < vis_end are visible to this row
    if constexpr (!SPARSE) {
      int ve = Lb;
      if (a.causal) ve = min(Lb, Lb - a.s_q + tok + 1);
      vis_end = row_ok ? max(ve, 0) : 0;
    }
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) o[mt] = f32x16{};

    // ---- piece prologue: the query fragments, then a drain.  The loads of
    // the piece's first steps (and the previous piece's stores) are older
    // than the query loads, so their latencies overlap.
    // Query fragments of this piece: the bf16 q rows, or (fused) q-hat
    // formed from them below.
    const float srow = a.scale_log2;  // log2(e) * softmax scale (the fused q-hat carries its RMSNorm factor)
    {
      const uint16_t* qrow = a.q + ((int64_t)cb * a.rows + (row_ok ? row : 0)) * dqk_of<KVF>();
      const double pos = (double)Lb - (double)a.s_q + (double)tok;
      // chunk ks (dims 16ks + 8half .. +7): q-hat chunk, then its home
      auto put_q = [&](int ks, bf16x8 v) {
        if (!row_ok) v = bf16x8{};
        if (ks < kQR) {
          qf[ks] = v;
        } else {
          // the LDS address is formed here from a fresh lane index, so the
          // twelve slot addresses are not precomputed and spilled
          const int ln = fresh_lane(), lr = ln & 31;
          const int cq = 2 * (ks - kQR) + (ln >> 5);
          *reinterpret_cast<bf16x8*>(qlds + lr * q_lds_row_bytes<KVF, FUSED>() + ((cq ^ ((lr >> 1) & 7)) << 4)) = v;
        }
      };
      if constexpr (!FUSED) {
        bf16x8 vq[ksteps<KVF>()];
#pragma unroll
        for (int ks = 0; ks < ksteps<KVF>(); ++ks) vq[ks] = *reinterpret_cast<const bf16x8*>(qrow + (2 * ks + half) * 8);
        if constexpr (KVF != kKvBf16) {
          // FP8 records: the first piece's first record loads go out behind
          // the query loads, so that the two latencies overlap.  Sparse
          // record loads read their ids from LDS: the id loads went out
          // before the query loads, so waiting until only the query loads
          // may be outstanding lands them.
          if (first_piece) {
            if constexpr (SPARSE) wait_vmcnt<ksteps<KVF>()>();
            issue_first_loads();
          }
        }
#pragma unroll
        for (int ks = 0; ks < ksteps<KVF>(); ++ks) {
          const bf16x8 v = vq[ks];
          // fp16 products (the V3.2 FP8 cache): bf16 q converts exactly
          // (magnitudes in [2^-14, 65504])
          if constexpr (kF16) put_q(ks, __builtin_bit_cast(bf16x8, bf16x8_to_f16x8(__builtin_bit_cast(uint4, v))));
          else put_q(ks, v);
        }
      } else {
        // Fused prologue: q-hat = inv * RoPE(q (.) w), inv = 1/sqrt(mean(q^2)
        // + eps) over the row's 576 dims (RMSNorm, then RoPE on dims
        // 512..575 at position len - s_q + t; RoPE is linear, so the row
        // factor may come first), rounded once to fp16 for the fp16 products.
        // Pass 1 reads the row for its sum of squares (all 36 chunks in
        // flight) and leaves the chunks bound for LDS (k-steps kQR..35) raw
        // in their slots; pass 2 forms q-hat of those in place and reads the
        // register chunks again (from L2 now), with the weight row staged in
        // LDS.  Keeping the register chunks from pass 1 to pass 2 instead
        // would need 96 VGPRs beside the fragments and spills them.
        // This lane's row and query row address are formed here from a
        // fresh lane index: hoisted out of the piece loop they are spilled,
        // and each reload of a spill waits for every load in flight.
        const int fln = fresh_lane();
        const int frow = g * kRowsPerWg + wave * 32 + (fln & 31);
        const bool frow_ok = frow < a.rows;
        // chunk ks of this lane (dims 16ks + 8half ..) sits at fq + 16ks
        const uint16_t* fq = a.q + ((int64_t)cb * a.rows + (frow_ok ? frow : 0)) * dqk_of<KVF>() + (fln >> 5) * 8;
        // The first piece also reads the norm weight row beside the query
        // (stored to LDS after pass 1, for every later piece too) and issues
        // its first KV loads here, so that they land during the prologue.
        uint4 wrow = make_uint4(0, 0, 0, 0);
        if (first_piece && tid < kDqk / 8) wrow = reinterpret_cast<const uint4*>(a.norm_w)[wave * 64 + fresh_lane()];
        // LDS slot of query chunk ks >= kQR of this lane (where q-hat goes),
        // formed from a fresh lane index
        auto qslot = [&](int ks) -> bf16x8* {
          const int ln = fresh_lane(), lr = ln & 31;
          const int cq = 2 * (ks - kQR) + (ln >> 5);
          return reinterpret_cast<bf16x8*>(qlds + lr * q_lds_row_bytes<KVF, FUSED>() + ((cq ^ ((lr >> 1) & 7)) << 4));
        };
        float ss = 0.f;
        {
          bf16x8 v[ksteps<KVF>()];
#pragma unroll
          for (int ks = 0; ks < ksteps<KVF>(); ++ks) v[ks] = *reinterpret_cast<const bf16x8*>(fq + 16 * ks);
          if constexpr (KVF == kKvBf16) {
            if (first_piece) issue_first_loads();
          }

#pragma unroll
          for (int ks = 0; ks < ksteps<KVF>(); ++ks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += (float)v[ks][e] * (float)v[ks][e];
          }
          // the chunks that end in LDS are kept there raw for pass 2
#pragma unroll
          for (int ks = kQR; ks < ksteps<KVF>(); ++ks) *qslot(ks) = v[ks];
        }
        ss = row_sum2(ss);
        MLA_TR_FIRST(30, "v", ss);
        const float inv = 1.0f / sqrtf(ss / (float)kDqk + a.norm_eps);
        if (first_piece) {
          if (tid < kDqk / 8) *reinterpret_cast<uint4*>(smem + Lay::kWOff + (wave * 64 + fresh_lane()) * 16) = wrow;
          lds_barrier();
        }
        const uint16_t* wl = reinterpret_cast<const uint16_t*>(smem + Lay::kWOff);
        auto wchunk = [&](int ks) {
          return *reinterpret_cast<const bf16x8*>(wl + (2 * ks + (fresh_lane() >> 5)) * 8);
        };
        // q-hat of raw chunk v (k-step ks) with weight chunk wv; rr only for
        // the RoPE dims
        auto qhat = [&](int ks, const bf16x8& v, const bf16x8& wv, const RopeRow& rr) {
          float y[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = (float)v[e] * (float)wv[e] * inv;
          if (ks >= 32) {
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
              float cs, sn;
              rope_pair(rr, 1.0f, 8 * (ks - 32) + pp, 8 * (ks - 32) + 4 + pp, half, cs, sn);
              const float x0 = y[2 * pp], x1 = y[2 * pp + 1];
              y[2 * pp] = x0 * cs - x1 * sn;
              y[2 * pp + 1] = x0 * sn + x1 * cs;
            }
          }
          bf16x8 h;
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = to_op16<kF16>(y[e]);
          put_q(ks, h);
          return h;
        };
        // Pass 2 re-reads only the chunks that stay in registers (k-steps
        // below kQR), in groups of four, four groups ahead (two or three
        // ahead measured slower, six no faster); the first four groups'
        // reads go out first, and the LDS chunks (with the RoPE dims) are
        // turned into q-hat in place while they are in flight.  The
        // second read must not reuse the first one's registers, and its
        // window must hold: each group's reads take their offset from the
        // q-hat of the group before, so they cannot be hoisted to the top
        // (all reads at once spill, and every spill reload then waits for
        // all of them).
        int qoff = opaque(0);
        const uint16_t* qrow2 = fq + qoff;
        constexpr int kG = 4, kNG = kQR / kG, kAhead = 4;
        static_assert(kQR % kG == 0 && kNG >= kAhead && kQR <= 32, "whole groups; the RoPE dims in LDS");
        bf16x8 buf[kNG][kG];
#pragma unroll
        for (int gg = 0; gg < kAhead; ++gg)
#pragma unroll
          for (int i = 0; i < kG; ++i) buf[gg][i] = *reinterpret_cast<const bf16x8*>(qrow2 + 16 * (gg * kG + i));
        {
          // the RoPE angles are formed here, right before their use
          // (position len - s_q + t in integers, converted once: exact)
          const int r2 = g * kRowsPerWg + wave * 32 + (fresh_lane() & 31);
          const bool r2_ok = r2 < a.rows;
          const int t2 = r2_ok ? r2 / opaque_s(a.h_q) : 0;
          const RopeRow rr = rope_row((double)(Lb - a.s_q + t2), r2_ok, rope_inv, 1.0f);
          // every raw chunk and weight is read before any q-hat goes back
          // (a read after a write to LDS is not moved above it, so chunk by
          // chunk each would wait out the LDS latency)
          constexpr int kL = ksteps<KVF>() - kQR;
          bf16x8 raw[kL], wv[kL];
#pragma unroll
          for (int j = 0; j < kL; ++j) {
            raw[j] = *qslot(kQR + j);
            wv[j] = wchunk(kQR + j);
          }
#pragma unroll
          for (int j = 0; j < kL; ++j) qhat(kQR + j, raw[j], wv[j], rr);
        }

        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int g = 0; g < kNG; ++g) {
          if (g + kAhead < kNG) {
#pragma unroll
            for (int i = 0; i < kG; ++i)
              buf[g + kAhead][i] = *reinterpret_cast<const bf16x8*>(fq + qoff + 16 * ((g + kAhead) * kG + i));
          }
          uint32_t hlast = 0;
#pragma unroll
          for (int i = 0; i < kG; ++i)
            hlast = __builtin_bit_cast(uint4, qhat(g * kG + i, buf[g][i], wchunk(g * kG + i), RopeRow{})).x;
          asm volatile("" : "+v"(qoff) : "v"(hlast));
          // one group at a time: the next groups' reads are in flight, the
          // weight reads are not hoisted past it
          __builtin_amdgcn_sched_barrier(0);
        }
        MLA_TR_FIRST(31, "v", qoff);
      }
    }
    if constexpr (KVF == kKvBf16 && !FUSED) {
      // after the query loads, so that the latencies overlap; the walker
      // words went out before them, so waiting until only the query loads
      // may be outstanding lands the words (each wave reads its own)
      if (first_piece) {
        if constexpr (kLateLand) {
          wait_vmcnt<ksteps<KVF>()>();
          land();
        }
        issue_first_loads();
      }
    }
    wait_vmcnt<0>();
    lds_barrier();  // every wave's loads of the piece's first step (and Q in LDS) landed
    first_piece = false;
    MLA_TR(2);

    // ======== building blocks of one 32-key step
    auto tile_off = [&](int st) -> int {
      if constexpr (KVF == kKvBf16) return Lay::kTileOff + (st % kTileRing) * kHalfBytes;
      else if constexpr (dq_ahead<KVF, FUSED>()) return Lay::kTileOff + (st & 1) * kHalfBytes;
      else return Lay::kTileOff;
    };
    // S^T (32 keys x 32 rows) of the tile at LDS offset tb into sc, with the
    // LDS operands of k-step ks+kLa read before the MFMA of k-step ks (order
    // fixed by scheduling fences); hook(ks) runs after that MFMA is issued.
    // (bf16 and V4.1 records: the query fragments are all in VGPRs; V4.1 has
    // 32 k-steps, its 512 dims all in the main part of the tile.)
    auto qk = [&](int tb, f32x16& sc, auto&& hook) {
      constexpr int kLa = FUSED ? 3 : 4;
      const int ln = fresh_lane(), lr = ln & 31, lh = ln >> 5;
      const int lkey = key_of_row(lr), lfr = (lkey >> 1) & 7;
      const int koff = tb + lkey * kMainStride + 16 * lh;
      const int kroff = tb + kRopeOff + lkey * kRopeStride;
      auto read_k = [&](int ks) {
        if (ks < 32) return *reinterpret_cast<const bf16x8*>(smem + koff + 32 * ks);
        return *reinterpret_cast<const bf16x8*>(smem + kroff + ((((2 * (ks - 32)) | lh) ^ lfr) << 4));
      };
      constexpr int kKS = ksteps<KVF>();
      // query k-steps kQR.. sit in the wave's LDS rows (384 B, chunk c of row
      // r at c ^ ((r >> 1) & 7)), read kLa MFMAs ahead like K
      const int lx = (lr >> 1) & 7;
      const int qrow0 = Lay::kQOff + wave * q_lds_wave_bytes<KVF, FUSED>() + lr * q_lds_row_bytes<KVF, FUSED>();
      auto read_q = [&](int ks) {
        const int j = ks - kQR;
        return *reinterpret_cast<const bf16x8*>(smem + qrow0 + ((j >> 2) << 7) + ((((2 * (j & 3)) | lh) ^ lx) << 4));
      };
      bf16x8 kbuf[kLa], qbuf[kLa];
#pragma unroll
      for (int i = 0; i < kLa; ++i) kbuf[i] = read_k(i);
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const bf16x8 ka = kbuf[ks % kLa];
        const bf16x8 qb = ks < kQR ? qf[ks < kQR ? ks : 0] : qbuf[ks % kLa];
        if (ks + kLa < kKS) {
          kbuf[ks % kLa] = read_k(ks + kLa);
          if (ks + kLa >= kQR) qbuf[ks % kLa] = read_q(ks + kLa);
        }
        if (ks == 0) mfma_s_first<kF16>(sc, ka, qb);
        else mfma_s_acc<kF16>(sc, ka, qb);
        hook(ks);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_s_settle(sc);
    };
    // O^T += V^T P^T over the tile at tb (2 k-steps x 16 d-tiles): 32 MFMAs,
    // each fed by two transposed reads issued kVa MFMAs ahead.  This lane
    // supplies key row key_of_row(16kq + 8hi + 4half + j) = 16kq + 4j + 2hi +
    // half (j = (lane & 15) >> 2) and dims 32mt + 16*((lane >> 4) & 1) + 4*(lane & 3).
    auto pv = [&](int tb, const bf16x8 (&pf)[2]) {
      constexpr int kVa = 3;
      const int ln = fresh_lane();
      const int voff = tb + (4 * ((ln & 15) >> 2) + (ln >> 5)) * kMainStride + 32 * ((ln >> 4) & 1) + 8 * (ln & 3);
      auto read_v = [&](int i) {  // i = kq * 16 + mt
        const int kq = i >> 4, mt = i & 15;
        const uint8_t* p = smem + voff + kq * 16 * kMainStride + mt * 64;
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(p));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(p + 2 * kMainStride));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 vbuf[kVa];
#pragma unroll
      for (int i = 0; i < kVa; ++i) vbuf[i] = read_v(i);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const bf16x8 va = vbuf[i % kVa];
        if (i + kVa < 32) vbuf[i % kVa] = read_v(i + kVa);
        mfma_o<kF16>(o[i & 15], va, pf[i >> 4]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto key0_of = [&](int ps) { return (cj + (ps >> 1)) * kPage + (ps & 1) * kHalfRows; };
    auto has_keys = [&](int ps) {
      const int k0 = key0_of(ps);
      return SPARSE ? (k0 < a.topk) : (k0 < Lb);
    };
    // Online softmax of one tile (log2 domain), written as kSmSlices slices
    // run in order.  Register i
    // of the S^T accumulator holds key key0 + key_of_row(8*(i/4) + i%4) + half.
    //   0..3  scale, mask, max of registers 4k..4k+3
    //   4     row max over the lane pair
    //   5     lazy rescale decision
    //   6..9  p = exp2(s - m), P^T fragments, row sum of registers 4(k-6)..
    //   10    running sum
    struct SmState {
      float mx, alpha, mref, psum;
      uint32_t any_need, vmask;
      bf16x8 pf[2];
    };
    auto sm_slice = [&](int k, f32x16& sc, SmState& st, int key0, int st_step) {
      if (k < 4) {
        if (k == 0) st.mx = -INFINITY;
        // the key of register i is kc + half with kc a compile-time constant,
        // so the lane's half is folded into the limits, not into 16 keys
        if constexpr (SPARSE) {
          // valid keys of the step as one bit mask (a ballot over the ids),
          // shifted by the lane's half: key kc + half is bit kc
          if (k == 0) {
            const int ln = fresh_lane(), r = ln & 31;
            const int nvalid = min(kHalfRows, a.topk - key0);
            const uint64_t bm =
                __builtin_amdgcn_ballot_w64(ln < 32 && r < nvalid && id_in_pool(ids_slot(st_step)[r], ntok));
            st.vmask = row_ok ? (uint32_t)bm >> half : 0u;
          }
#pragma unroll
          for (int i = 4 * k; i < 4 * k + 4; ++i) {
            const int kc = key_of_row(8 * (i >> 2) + (i & 3));
            float v = sc[i] * srow;
            v = ((st.vmask >> kc) & 1u) ? v : -INFINITY;
            sc[i] = v;
            st.mx = fmaxf(st.mx, v);
          }
        } else {
          const int lim_h = vis_end - key0 - half;  // register i visible iff kc < lim_h
#pragma unroll
          for (int i = 4 * k; i < 4 * k + 4; ++i) {
            const int kc = key_of_row(8 * (i >> 2) + (i & 3));
            float v = sc[i] * srow;
            v = kc < lim_h ? v : -INFINITY;
            sc[i] = v;
            st.mx = fmaxf(st.mx, v);
          }
        }
      } else if (k == 4) {
        st.mx = row_max2(st.mx);
      } else if (k == 5) {
        const bool need = st.mx > m_used + kRescaleThreshold;
        // O is still zero while m_used is -inf: nothing to scale
        st.any_need = uni((int)(__builtin_amdgcn_ballot_w64(need && m_used != -INFINITY) != 0));
        st.alpha = need ? exp2f(m_used - st.mx) : 1.0f;  // exp2(-inf) = 0
        if (need) m_used = st.mx;
        st.mref = m_used == -INFINITY ? 0.f : m_used;
        st.psum = 0.f;
      } else if (k < 10) {
#pragma unroll
        for (int i = 4 * (k - 6); i < 4 * (k - 6) + 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(sc[i] - st.mref);
          st.psum += p;
          st.pf[i >> 3][i & 7] = to_op16<kF16>(p);
        }
      } else {
        lsum = lsum * st.alpha + st.psum;
      }
    };
    constexpr int kSmSlices = 11;
    // Rare: the running max moved by more than the threshold; scale O.
    // Rare: some row's running max moved by more than the threshold while O
    // already held keys; scale O by alpha.  The branch ends with a full vmcnt
    // wait of its own: the compiler may spill around the bulk AGPR traffic
    // here, and without that wait the reloads would leave pending loads at
    // the join that it then guards with full waits on the common path.
    auto rescale_o = [&](const SmState& st) {
      if (__builtin_expect(st.any_need != 0, 0)) {
        o_settle(o);
#pragma unroll
        for (int mt = 0; mt < 16; ++mt) {
#pragma unroll
          for (int i = 0; i < 16; ++i) o[mt][i] *= st.alpha;
          __builtin_amdgcn_sched_barrier(0);
        }
        o_settle(o);
        wait_vmcnt<0>();
      }
    };

    if constexpr (KVF == kKvBf16) {
      // ---- bf16: step ps waits for its tile (issued kDepth steps ago),
      // issues the loads of step+kDepth into the slot tile ps-1 left free,
      // then runs S^T, the online softmax and O += P V on its tile.  Within
      // one wave the softmax VALU work does not overlap the MFMAs (measured),
      // so the three phases run back to back on one resident tile.
      for (int ps = 0; ps < 2 * (piece_end - cj); ++ps, ++step) {
        MLA_ST_BEGIN;
        // Only the loads of the newest kDepth-1 steps (kLoadsPerHalf each,
        // issued after those steps' walker words) may still be in flight.
        wait_vmcnt<kLoadsPerHalf * (kDepth - 1)>();
        MLA_ST(0);
        if constexpr (FUSED) own_chunks_to_f16(smem + tile_off(step), wave);  // this wave's rows -> fp16
        lds_barrier();  // ... for every wave; tile ps-1's slot is free
        MLA_ST(1);
        land();
        prepare_load(step + kDepth);
        fetch_next_ids(step);
        emit_loads();
        MLA_ST(2);
        if (has_keys(ps)) {
          f32x16 sc;
          SmState st;
          qk(tile_off(step), sc, [](int) {});
          MLA_ST(3);
#pragma unroll
          for (int k = 0; k < kSmSlices; ++k) sm_slice(k, sc, st, key0_of(ps), step);
          rescale_o(st);
          valu_to_mfma_settle(st.pf[0], st.pf[1]);
          MLA_ST(4);
          pv(tile_off(step), st.pf);
          MLA_ST(5);
        }
        MLA_ST_STEP;
      }
    } else if constexpr (dq_ahead<KVF, FUSED>()) {
      // ---- FP8 records, two tiles.  Step s runs S^T, softmax and P.V on
      // tile s%2 and meanwhile dequantises step s+1's records into the other
      // tile, one chunk between every four MFMAs of S^T (V3.2: 9 chunks over
      // 36 k-steps; V4.1: 8 over 32); one barrier per step.  Raw records go
      // out three steps ahead (into the slot of the records dequantised a
      // step ago), ids five.
      auto dq_tile = [&](int st) { return smem + tile_off(st); };
      auto dq_raw = [&](int st) { return smem + Lay::kRawOff + (st % kRing) * kRawSlotBytes; };
      auto dequant_all = [&](int st) {
        if constexpr (KVF == kKvFp8V41) dequant_v41(dq_tile(st), dq_raw(st), tid);
        else dequant_codes(dq_tile(st), dq_raw(st), tid);
      };
      if (step == 0) {  // the first step's tile: the prologue drain landed its records
        dequant_all(0);
        lds_barrier();
      }
      for (int ps = 0; ps < 2 * (piece_end - cj); ++ps, ++step) {
        MLA_ST_BEGIN;
        if (ps > 0) {
          // The previous step issued raw(step+2) (if any) and, sparse,
          // ids(step+4) (if any), after everything this step needs:
          // raw(step+1) and ids(step+3).
          if (step + 2 >= nsteps) wait_vmcnt<0>();
          else if (SPARSE && step + 4 >= nsteps) wait_vmcnt<Lay::kVmPerStep - 1>();
          else wait_vmcnt<Lay::kVmPerStep>();
          MLA_ST(0);
          lds_barrier();  // tile step%2 staged by every wave; P.V(step-1) done with the other
          MLA_ST(1);
        }
        issue_next(step);
        MLA_ST(2);
        const bool hk = has_keys(ps);
        const bool dq = step + 1 < nsteps;
        f32x16 sc;
        SmState st;
        if (hk && dq) {
          if constexpr (KVF == kKvFp8V41) {
            V41Chunk ch;
            qk(tile_off(step), sc, [&](int ks) {
              if ((ks & 3) == 0) ch = v41_read(dq_raw(step + 1), wave, ks >> 2);
              else if ((ks & 3) == 3) v41_write(dq_tile(step + 1), wave, ks >> 2, ch);
            });
          } else {
            uint4 ch;
            qk(tile_off(step), sc, [&](int ks) {
              if ((ks & 3) == 0) ch = v32_read(dq_raw(step + 1), wave, ks >> 2);
              else if ((ks & 3) == 3) v32_write(dq_tile(step + 1), wave, ks >> 2, ch);
            });
          }
        } else if (hk) {
          qk(tile_off(step), sc, [](int) {});
        } else if (dq) {
          dequant_all(step + 1);
        }
        MLA_ST(3);
        if (hk) {
#pragma unroll
          for (int k = 0; k < kSmSlices; ++k) sm_slice(k, sc, st, key0_of(ps), step);
          rescale_o(st);
          valu_to_mfma_settle(st.pf[0], st.pf[1]);
          MLA_ST(4);
          pv(tile_off(step), st.pf);
          MLA_ST(5);
        }
        MLA_ST_STEP;
      }
    } else {
      // ---- fused FP8 V3.2: one fp16 tile (code times scale, rounded once),
      // dequantised from the raw ring each step; S^T and P.V as on bf16 KV
      for (int ps = 0; ps < 2 * (piece_end - cj); ++ps, ++step) {
        MLA_ST_BEGIN;
        if (ps > 0) {
          // This step's loads were issued two steps ago; the previous step
          // then issued the loads of step+1 (if any) and, sparse, the ids of
          // step+3 (if any).  Wait for everything older than those.
          constexpr int kLoadsPerStep = Lay::kVmPerStep - (SPARSE ? 1 : 0);
          if (step + 1 >= nsteps) wait_vmcnt<0>();
          else if (SPARSE && step + 3 >= nsteps) wait_vmcnt<kLoadsPerStep>();
          else wait_vmcnt<Lay::kVmPerStep>();
          MLA_ST(0);
          lds_barrier();  // every wave's loads of this step landed
        }
        dequant_codes(smem + Lay::kTileOff, smem + Lay::kRawOff + (step % kRing) * kRawSlotBytes, tid);
        lds_barrier();  // the tile is staged; raw slot (step+2)%3 (dequantised last step) is free
        MLA_ST(1);
        const bool hk = has_keys(ps);
        f32x16 sc;
        SmState st;
        if (hk) qk(tile_off(step), sc, [](int) {});
        MLA_ST(3);
        // The loads of step+2 go out after S^T: the register reloads inside
        // S^T wait for every older load, and would otherwise wait for these.
        issue_next(step);
        MLA_ST(2);
        if (hk) {
#pragma unroll
          for (int k = 0; k < kSmSlices; ++k) sm_slice(k, sc, st, key0_of(ps), step);
          rescale_o(st);
          valu_to_mfma_settle(st.pf[0], st.pf[1]);
          MLA_ST(4);
          pv(tile_off(step), st.pf);
          MLA_ST(5);
        }
        MLA_ST_STEP;
      }
    }

    MLA_TR(3);
    MLA_TR_ITEMS(piece_end - cj);
    // ======== finalize the piece: O / l and LSE; direct output or partial
    o_settle(o);
    {
      // this lane's row, formed again from a fresh lane index: kept from the
      // kernel start, these values would be spilled and reloaded here
      const int fln = fresh_lane();
      const int frow = g * kRowsPerWg + wave * 32 + (fln & 31);
      const bool frow_ok = frow < a.rows;
      const int fhalf = fln >> 5;
      const int ftok = frow_ok ? frow / a.h_q : 0;
      const float lt = row_sum2(lsum);
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
      const float lse2 = lt > 0.f ? m_used + __builtin_amdgcn_logf(lt) : -INFINITY;
      const int nsplit = uni(sload(a.num_splits, cb + 1) - sload(a.num_splits, cb));
      if (nsplit == 1) {
        const int64_t orow = (int64_t)cb * a.rows + frow;
        if constexpr (!FUSED) {
          if (frow_ok) {
            uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + orow * kDv;
#pragma unroll
            for (int mt = 0; mt < 16; ++mt)
#pragma unroll
              for (int qd = 0; qd < 4; ++qd) {
                const int d = 32 * mt + 8 * qd + 4 * fhalf;
                const __bf16 v0 = (__bf16)(o[mt][4 * qd] * inv), v1 = (__bf16)(o[mt][4 * qd + 1] * inv);
                const __bf16 v2 = (__bf16)(o[mt][4 * qd + 2] * inv), v3 = (__bf16)(o[mt][4 * qd + 3] * inv);
                uint2 pk;
                pk.x = (uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
                pk.y = (uint32_t)__builtin_bit_cast(uint16_t, v2) | ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
                *reinterpret_cast<uint2*>(op + d) = pk;
              }
            if (fhalf == 0) a.lse[orow] = lse2 * kLn2;
          }
        } else {
          // conjugate RoPE on dims 448..511 (d-tiles 14, 15), amax over the
          // row, e4m3 cast.  Tile by tile from the accumulators: only the 32
          // rotated values are held in VGPRs (scaling all of O at once would
          // move the 256 accumulators into VGPRs).  amax(O/l) = amax(O)/l
          // exactly, since scaling by a positive constant keeps the order.
          const double pos = (double)Lb - (double)a.s_q + (double)ftok;
          const RopeRow rr = rope_row(pos, frow_ok, rope_inv, -1.0f);
          float rot[2][16];
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd)
#pragma unroll
              for (int pp = 0; pp < 2; ++pp) {
                const int k0 = 16 * t + 4 * qd + pp;  // RoPE pair (d - 448) / 2 = k0 + 2 * fhalf
                float cs, sn;
                rope_pair(rr, -1.0f, k0, k0 + 2, fhalf, cs, sn);
                const float x0 = o[14 + t][4 * qd + 2 * pp] * inv, x1 = o[14 + t][4 * qd + 2 * pp + 1] * inv;
                rot[t][4 * qd + 2 * pp] = x0 * cs - x1 * sn;
                rot[t][4 * qd + 2 * pp + 1] = x0 * sn + x1 * cs;
              }
          float am = 0.f;
#pragma unroll
          for (int mt = 0; mt < 14; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(o[mt][i]));
          float amax = am * inv;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(rot[t][i]));
          amax = row_max2(amax);
          const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
          const float rs = amax > 0.f ? 448.0f / amax : 1.0f;
          if (frow_ok) {
            uint8_t* op = reinterpret_cast<uint8_t*>(a.out) + orow * kDv;
            auto put = [&](int mt, int qd, float v0, float v1, float v2, float v3) {
              const int d = 32 * mt + 8 * qd + 4 * fhalf;
              v0 = fminf(fmaxf(v0 * rs, -448.f), 448.f);
              v1 = fminf(fmaxf(v1 * rs, -448.f), 448.f);
              v2 = fminf(fmaxf(v2 * rs, -448.f), 448.f);
              v3 = fminf(fmaxf(v3 * rs, -448.f), 448.f);
              int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
              pk = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, pk, true);
              *reinterpret_cast<int*>(op + d) = pk;
            };
#pragma unroll
            for (int mt = 0; mt < 14; ++mt)
#pragma unroll
              for (int qd = 0; qd < 4; ++qd)
                put(mt, qd, o[mt][4 * qd] * inv, o[mt][4 * qd + 1] * inv, o[mt][4 * qd + 2] * inv,
                    o[mt][4 * qd + 3] * inv);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int qd = 0; qd < 4; ++qd)
                put(14 + t, qd, rot[t][4 * qd], rot[t][4 * qd + 1], rot[t][4 * qd + 2], rot[t][4 * qd + 3]);
            if (fhalf == 0) {
              a.lse[orow] = lse2 * kLn2;
              a.out_scale[orow] = sc;
            }
          }
        }
      } else {
        // partial of split `split_k` of sequence cb, row group g: O/l rounded
        // to bf16, stored in register order [wave][d-tile][quad pair][lane][8]
        const int64_t pidx = (int64_t)uni(sload(a.num_splits, cb) + split_k) * a.groups + g;
        const __amdgpu_buffer_rsrc_t prs = buf_rsrc(uni_ptr(a.part_o + pidx * kPartialOElems), kPartialOElems * 2);
        const int vbase = (wave * (16 * 2 * 64 * 8) + fln * 8) * 2;
#pragma unroll
        for (int mt = 0; mt < 16; ++mt)
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const __bf16 lo = (__bf16)(o[mt][8 * q2 + 2 * e] * inv), hi = (__bf16)(o[mt][8 * q2 + 2 * e + 1] * inv);
              w[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            }
            __builtin_amdgcn_raw_buffer_store_b128(w, prs, vbase + (mt * 2 + q2) * 64 * 8 * 2, 0, kPastL2);
          }
        if (fhalf == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse2 * kLn2),
                                                buf_rsrc(uni_ptr(a.part_lse + pidx * kPartialLseFloats), kPartialLseFloats * 4),
                                                (wave * 32 + (fln & 31)) * 4, 0, kPastL2);
      }
    }
    MLA_TR(4);
    MLA_TR_NEXT_PIECE
    // next piece: first item of the following sequence
    cb = uni(cb + 1);
    cj = 0;
    split_k = 0;
  }
  wait_vmcnt<0>();  // no tile load (zeros past the end) outlives the workgroup's LDS
  MLA_TR_KERNEL_END
}

// ---------------------------------------------------------------------------
// Fused combine, second launch: the epilogue of the 32 rows wt*32.. of row
// group g of sequence b, once k_combine<kCombF32, 4> has merged them.  That merge
// leaves each (32-row tile, 32-dim tile mt)'s fp32 O in the slices of the
// tile that splits s0 and s0+1 held (every lane's 16 values in the four
// 16-byte chunks it read there).  Wave `sub` (lanes `lane`) takes d-tiles
// 4*sub .. 4*sub+3; acc[4*i + qd] holds quad qd of d-tile 4*sub + i.  The
// row amax spans all 512 dims, so the four waves of the rows share it
// through LDS (amax_s: 1 KB).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float* merged_chunk(const DecodeArgs& a, int b, int g, int wt, int mt, int lane,
                                               int k) {
  // chunk k (0..3) of lane `lane`: split s0 + (k & 1), 16-byte chunk k >> 1
  const int64_t pstride = (int64_t)a.groups * kPartialOElems;
  uint16_t* pb = a.part_o + (int64_t)(a.num_splits[b] + (k & 1)) * pstride + (int64_t)g * kPartialOElems +
                 (size_t)((wt * 16 + mt) * 2 + (k >> 1)) * 64 * 8 + (size_t)lane * 8;
  return reinterpret_cast<float*>(pb);
}

__global__ void __launch_bounds__(256) k_fused_epilogue(DecodeArgs a) {
  __shared__ float amax_s[4][64];
  const int wt = blockIdx.x & 3;
  const int g = (blockIdx.x >> 2) % a.groups;
  const int b = (blockIdx.x >> 2) / a.groups;
  const int sub = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s0 = a.num_splits[b], ns = a.num_splits[b + 1] - s0;
  if (ns <= 1) return;  // the decode wrote these rows itself (uniform over the workgroup)
  const int half = lane >> 5, r32 = lane & 31;
  const int row = g * kRowsPerWg + wt * 32 + r32;
  const bool row_ok = row < a.rows;
  f32x4 acc[16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // the merge's chunk k holds its values 4k .. 4k+3, i.e. quad k of d-tile mt
      const float4 v = *reinterpret_cast<const float4*>(merged_chunk(a, b, g, wt, 4 * sub + i, lane, k));
      acc[4 * i + k] = f32x4{v.x, v.y, v.z, v.w};
    }
  const int64_t orow = (int64_t)b * a.rows + row;
  // conjugate RoPE on dims 448..511 (sub 3 holds d-tiles 12..15)
  const int Lb = a.seqlens[b];
  const int tok = row_ok ? row / a.h_q : 0;
  const double pos = (double)Lb - (double)a.s_q + (double)tok;
  const RopeRow rr = rope_row(pos, row_ok, rope_inv_freq(lane & 31, a.rope_log2_base), -1.0f);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int e = sub * 16 + k, mt = e >> 2, qd = e & 3;
    if (mt < 14) continue;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int k0 = 16 * (mt - 14) + 4 * qd + pp;  // RoPE pair (d - 448) / 2 = k0 + 2 * half
      float cs, sn;
      rope_pair(rr, -1.0f, k0, k0 + 2, half, cs, sn);
      const float x0 = acc[k][2 * pp], x1 = acc[k][2 * pp + 1];
      acc[k][2 * pp] = x0 * cs - x1 * sn;
      acc[k][2 * pp + 1] = x0 * sn + x1 * cs;
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(acc[k][e]));
  amax = row_max2(amax);
  amax_s[sub][lane] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(amax_s[0][lane], amax_s[1][lane]), fmaxf(amax_s[2][lane], amax_s[3][lane]));
  const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
  const float rs = amax > 0.f ? 448.0f / amax : 1.0f;
  if (row_ok) {
    uint8_t* op = reinterpret_cast<uint8_t*>(a.out) + orow * kDv;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int e = sub * 16 + k, mt = e >> 2, qd = e & 3;
      const int d = 32 * mt + 8 * qd + 4 * half;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = fminf(fmaxf(acc[k][i] * rs, -448.f), 448.f);
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], pk, true);
      *reinterpret_cast<int*>(op + d) = pk;
    }
    if (half == 0 && sub == 0) a.out_scale[orow] = sc;
  }
}

// Row groups (batch x groups) up to which the combine gives each tile four
// waves: fewer sequences over the same slots means more splits each.
constexpr int kCombineWideRowGroups = 8;

// The combine: one workgroup per (sequence b, row group g, 32-row tile
// wt, 32-dim tile mt), so that even one sequence with many splits spreads
// over many CUs; one wave, or (few row groups, many splits) four that
// share the tile's splits.  Lane l takes the place of the decode's
// lane l: row 32wt + l%32 and the 16 values of d-tile mt it held, two
// 16-byte chunks per split (the partials are stored in that order).
//   lse = ln sum_s e^{lse_s};  O = sum_s e^{lse_s - lse} O_s,
// splits in ascending order, -inf partials with weight 0.
// Output modes: kCombBf16 writes bf16 O.  kCombF32 (the fused path's first
// launch when few row groups have many splits) writes the merged fp32
// values over the tile's own slices of splits s0 and s0+1, which no other
// workgroup reads (lane l rewrites exactly the four chunks it read there),
// for k_fused_epilogue.  kCombEpi (the fused path otherwise) gives one
// workgroup of 8 waves to each 16-row half of a 32-row tile, and runs the
// row epilogue (conjugate RoPE, row amax through LDS, e4m3 cast) in the
// same launch: wave v merges d-tiles 2v (lanes 0..31) and 2v+1 (lanes
// 32..63) of the half's 16 rows, lane 16h + r taking the decode lane
// 32h + 16*half + r's values.  The LSE is written in every mode.
constexpr int kCombBf16 = 0, kCombF32 = 1, kCombEpi = 2;
template <int MODE, int NW>
__global__ void __launch_bounds__(MODE == kCombEpi ? 512 : 64 * NW) k_combine(DecodeArgs a) {
  static_assert(MODE != kCombEpi || NW == 1, "one wave per pair of d-tiles");
  const int lane = threadIdx.x & 63;
  int tile, mt, half, r32, lane_p;  // lane_p: the decode lane whose values this lane merges
  if constexpr (MODE == kCombEpi) {
    tile = blockIdx.x >> 1;
    mt = 2 * (int)(threadIdx.x >> 6) + (lane >> 5);
    half = (lane >> 4) & 1;
    r32 = (blockIdx.x & 1) * 16 + (lane & 15);
  } else {
    tile = blockIdx.x >> 4;
    mt = blockIdx.x & 15;
    half = lane >> 5;
    r32 = lane & 31;
  }
  lane_p = r32 + 32 * half;
  const int wt = tile & 3, g = (tile >> 2) % a.groups, b = (tile >> 2) / a.groups;
  const int s0 = a.num_splits[b], ns = a.num_splits[b + 1] - s0;
  if (ns <= 1) return;  // uniform over the workgroup
  // NW waves share the tile: wave w takes splits w, w + NW, ... and the
  // waves' LSE sums and weighted partials are added through LDS
  const int w = NW > 1 ? (int)(threadIdx.x >> 6) : 0;
  const int row = g * kRowsPerWg + wt * 32 + r32;
  const int64_t lstride = (int64_t)a.groups * kPartialLseFloats;
  const float* lsep0 = a.part_lse + (int64_t)s0 * lstride + (int64_t)g * kPartialLseFloats + wt * 32 + r32;
  const int64_t pstride = (int64_t)a.groups * kPartialOElems;
  const uint16_t* pb = a.part_o + (int64_t)s0 * pstride + (int64_t)g * kPartialOElems +
                       (size_t)((wt * 16 + mt) * 2) * 64 * 8 + (size_t)lane_p * 8;
  const int nsw = ns > w ? (ns - w + NW - 1) / NW : 0;  // this wave's splits
  const float* lsep = lsep0 + w * lstride;
  const uint16_t* pbw = pb + w * pstride;
  const int64_t lstep = lstride * NW, pstep = pstride * NW;
  // The first kInFlight of the wave's splits: LSEs and partial chunks are
  // read together (one round trip for the usual handful of splits); more
  // splits (batch 1 spreads one sequence over the machine) follow
  // kInFlight at a time.
  constexpr int kInFlight = 8;
  float l[kInFlight];
  uint4 v[kInFlight][2];
#pragma unroll
  for (int j = 0; j < kInFlight; ++j) {
    const bool ok = j < nsw;
    l[j] = ok ? lsep[j * lstep] : -INFINITY;
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2)
      v[j][q2] = ok ? *reinterpret_cast<const uint4*>(pbw + j * pstep + q2 * 64 * 8) : make_uint4(0, 0, 0, 0);
  }
  // lse = ln sum_s e^{lse_s}, kInFlight splits at a time with a running
  // maximum m and the sum tot of e^{lse_s - m}
  float m = -INFINITY, tot = 0.f;
  auto lse_group = [&](const float (&lj)[kInFlight]) {
    float mc = m;
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) mc = fmaxf(mc, lj[j]);
    if (mc != -INFINITY) {
      float t = m == -INFINITY ? 0.f : tot * expf(m - mc);
#pragma unroll
      for (int j = 0; j < kInFlight; ++j) t += lj[j] == -INFINITY ? 0.f : expf(lj[j] - mc);
      tot = t;
      m = mc;
    }
  };
  lse_group(l);
  for (int s = kInFlight; s < nsw; s += kInFlight) {
    float lx[kInFlight];
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) lx[j] = s + j < nsw ? lsep[(s + j) * lstep] : -INFINITY;
    lse_group(lx);
  }
  if constexpr (NW > 1) {
    __shared__ float red_m[NW][64], red_t[NW][64];
    red_m[w][lane] = m;
    red_t[w][lane] = tot;
    __syncthreads();
    float mm = -INFINITY;
#pragma unroll
    for (int i = 0; i < NW; ++i) mm = fmaxf(mm, red_m[i][lane]);
    float tt = 0.f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int i = 0; i < NW; ++i) tt += red_m[i][lane] == -INFINITY ? 0.f : red_t[i][lane] * expf(red_m[i][lane] - mm);
    }
    m = mm;
    tot = tt;
  }
  const float lse = m == -INFINITY ? -INFINITY : m + logf(tot);
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  auto accumulate = [&](const float (&lj)[kInFlight], const uint4 (&vj)[kInFlight][2]) {
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) {
      const float wj = lj[j] == -INFINITY ? 0.f : expf(lj[j] - lse);
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const uint32_t u[4] = {vj[j][q2].x, vj[j][q2].y, vj[j][q2].z, vj[j][q2].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[8 * q2 + 2 * e] += wj * __uint_as_float(u[e] << 16);
          acc[8 * q2 + 2 * e + 1] += wj * __uint_as_float(u[e] & 0xffff0000u);
        }
      }
    }
  };
  if (m != -INFINITY) {
    accumulate(l, v);
    for (int s = kInFlight; s < nsw; s += kInFlight) {
#pragma unroll
      for (int j = 0; j < kInFlight; ++j) {
        const bool ok = s + j < nsw;
        l[j] = ok ? lsep[(s + j) * lstep] : -INFINITY;
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
          v[j][q2] = ok ? *reinterpret_cast<const uint4*>(pbw + (s + j) * pstep + q2 * 64 * 8) : make_uint4(0, 0, 0, 0);
      }
      accumulate(l, v);
    }
  }
  if constexpr (NW > 1) {
    // waves 1.. hand their sums to wave 0, which writes the tile (after
    // this barrier no wave reads a partial any more)
    __shared__ float red_acc[NW - 1][16][64];
    if (w > 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) red_acc[w - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int k = 0; k < NW - 1; ++k)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += red_acc[k][i][lane];
  }
  if constexpr (MODE == kCombF32) {
    // chunk k (split s0 + (k & 1), 16-byte chunk k >> 1) takes values 4k .. 4k+3
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint16_t* dst = const_cast<uint16_t*>(pb) + (k & 1) * pstride + (k >> 1) * 64 * 8;
      *reinterpret_cast<float4*>(dst) = make_float4(acc[4 * k], acc[4 * k + 1], acc[4 * k + 2], acc[4 * k + 3]);
    }
    if (row < a.rows && mt == 0 && half == 0) a.lse[(int64_t)b * a.rows + row] = lse;
  } else if constexpr (MODE == kCombEpi) {
    // value i = 4qd + c sits at d = 32mt + 8qd + 4half + c, so RoPE pair
    // (d - 448) / 2 of d-tiles 14, 15 is k0 + 2half, k0 = 16(mt - 14) + 4qd + pp
    __shared__ float amax_s[16][16];
    const bool row_ok = row < a.rows;
    const int64_t orow = (int64_t)b * a.rows + row;
    if (mt >= 14) {  // conjugate RoPE on dims 448..511 (the last wave)
      const int tok = row_ok ? row / a.h_q : 0;
      const double pos = (double)a.seqlens[b] - (double)a.s_q + (double)tok;
      const RopeRow rr = rope_row(pos, row_ok, rope_inv_freq(lane & 31, a.rope_log2_base), -1.0f);
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int k0 = 16 * (mt - 14) + 4 * qd + pp;  // mt differs between the wave's halves
          float cs, sn;
          rope_pair_lanes(rr, -1.0f, k0, k0 + 2, half, cs, sn);
          const float x0 = acc[4 * qd + 2 * pp], x1 = acc[4 * qd + 2 * pp + 1];
          acc[4 * qd + 2 * pp] = x0 * cs - x1 * sn;
          acc[4 * qd + 2 * pp + 1] = x0 * sn + x1 * cs;
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(acc[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));  // the row's other half of d-tile mt
    if (half == 0) amax_s[mt][lane & 15] = amax;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, amax_s[i][lane & 15]);
    const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
    const float rs = amax > 0.f ? 448.0f / amax : 1.0f;
    if (row_ok) {
      uint8_t* op = reinterpret_cast<uint8_t*>(a.out) + orow * kDv;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = fminf(fmaxf(acc[4 * qd + c] * rs, -448.f), 448.f);
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], pk, true);
        *reinterpret_cast<int*>(op + 32 * mt + 8 * qd + 4 * half) = pk;
      }
      if (mt == 0 && half == 0) {
        a.out_scale[orow] = sc;
        a.lse[orow] = lse;
      }
    }
  } else if (row < a.rows) {
    const int64_t orow = (int64_t)b * a.rows + row;
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + orow * kDv;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {  // value i = 4qd + c sits at d = 32mt + 8qd + 4half + c
      uint2 pk;
      pk.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[4 * qd]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[4 * qd + 1]) << 16);
      pk.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[4 * qd + 2]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[4 * qd + 3]) << 16);
      *reinterpret_cast<uint2*>(op + 32 * mt + 8 * qd + 4 * half) = pk;
    }
    if (mt == 0 && half == 0) a.lse[orow] = lse;
  }
}

// ---------------------------------------------------------------------------
// Debug gather: stage both halves of one work item with the decode kernel's
// loaders (and dequantiser), copy them out un-swizzled as [64][576] 16-bit
// values: bf16, or fp16 for V3.2 FP8 records (the tile the products read).
// ---------------------------------------------------------------------------
template <int KVF, bool SPARSE>
__global__ void __launch_bounds__(kThreads) k_debug_gather(DecodeArgs a, int b, int t, int j,
                                                          uint16_t* dst) {
  constexpr int kSmem = kHalfBytes + kRawSlotBytes + 256;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmem];
  uint8_t* tile = smem;
  uint8_t* raw = smem + kHalfBytes;
  int32_t* ids = reinterpret_cast<int32_t*>(smem + kHalfBytes + kRawSlotBytes);
  const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
  for (int h = 0; h < 2; ++h) {
    __syncthreads();
    if constexpr (SPARSE) {
      fetch_ids_dma(ids, a.indices, ((int64_t)b * a.s_q + t) * a.topk, a.topk, j, h);
      __builtin_amdgcn_s_waitcnt(0);
      const int nvalid = min(kHalfRows, a.topk - j * kPage - h * kHalfRows);
      if constexpr (KVF == kKvBf16) load_half_bf16_sparse(tile, a.kv, a.num_blocks * kPage, ids, nvalid, wave, lane);
      else load_half_fp8_sparse(raw, a.kv, a.num_blocks * kPage, ids, nvalid, wave, lane);
    } else {
      const int L = a.seqlens[b];
      const bool any = j * kPage < L;
      const int64_t bt = any ? a.block_table[(int64_t)b * a.max_blocks + j] : 0;
      const bool in_pool = bt >= 0 && bt < a.num_blocks;
      const int64_t phys = in_pool ? bt : 0;
      const int valid = any && in_pool ? min(kPage, L - j * kPage) : 0;
      if constexpr (KVF == kKvBf16) load_half_bf16_dense(tile, a.kv, phys, valid, h, wave, lane);
      else load_half_fp8_dense(raw, a.kv, phys, valid, h, wave, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if constexpr (KVF != kKvBf16) {
      dequant_codes(tile, raw, tid);
      __syncthreads();
    }
    for (int k = tid; k < kHalfRows * kChunksPerRow; k += kThreads) {
      const int r = k / kChunksPerRow, c = k - r * kChunksPerRow;
      const uint8_t* src = c < 64 ? tile + r * kMainStride + c * 16
                                  : tile + kRopeOff + r * kRopeStride + (rope_phys_chunk(r, c - 64) << 4);
      *reinterpret_cast<uint4*>(dst + (h * kHalfRows + r) * kDqk + c * 8) = *reinterpret_cast<const uint4*>(src);
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_sched(const int32_t* seqlens, int batch, int piece_cost, int topk, int num_slots,
                        int32_t* meta, int32_t* num_splits, hipStream_t stream) {
  if (batch <= kSchedSmallBatch)
    hipLaunchKernelGGL((k_sched<256, kSchedSmallBatch>), dim3(1), dim3(256), 0, stream, seqlens, batch,
                       piece_cost, topk, num_slots, meta, num_splits);
  else
    hipLaunchKernelGGL((k_sched<1024, kMaxBatch>), dim3(1), dim3(1024), 0, stream, seqlens, batch, piece_cost,
                       topk, num_slots, meta, num_splits);
  return hipGetLastError();
}

template <int KVF, bool SPARSE, bool FUSED>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream, hipEvent_t start,
                                  hipEvent_t stop) {
  const int grid = a.num_slots * a.groups;
  if (start || stop)
    hipExtLaunchKernelGGL((k_decode<KVF, SPARSE, FUSED>), dim3(grid), dim3(kThreads), 0, stream, start,
                          stop, 0, a);
  else
    hipLaunchKernelGGL((k_decode<KVF, SPARSE, FUSED>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int kv_format, bool sparse, bool fused,
                         hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (kv_format == kKvBf16) {
    if (!sparse) return fused ? launch_decode_t<kKvBf16, false, true>(a, stream, start, stop)
                              : launch_decode_t<kKvBf16, false, false>(a, stream, start, stop);
    return fused ? launch_decode_t<kKvBf16, true, true>(a, stream, start, stop)
                 : launch_decode_t<kKvBf16, true, false>(a, stream, start, stop);
  }
  if (kv_format == kKvFp8V41) {  // sparse, unfused only (checked by the caller)
    if (!sparse || fused) return hipErrorInvalidValue;
    return launch_decode_t<kKvFp8V41, true, false>(a, stream, start, stop);
  }
  if (!sparse) return fused ? launch_decode_t<kKvFp8V32, false, true>(a, stream, start, stop)
                            : launch_decode_t<kKvFp8V32, false, false>(a, stream, start, stop);
  return fused ? launch_decode_t<kKvFp8V32, true, true>(a, stream, start, stop)
               : launch_decode_t<kKvFp8V32, true, false>(a, stream, start, stop);
}

hipError_t launch_combine(const DecodeArgs& a, bool fused, hipStream_t stream) {
  const int grid = a.batch * a.groups * 4;
  if (grid == 0) return hipSuccess;
  // A few sequences spread over the machine have many splits each: four
  // waves share each tile's splits.  Otherwise one wave per tile.
  // The fused path with many row groups merges and runs the row epilogue
  // in one launch (a workgroup per 16 rows); with few, the parallel fp32
  // merge and the epilogue are two launches.
  const bool wide = a.batch * a.groups <= kCombineWideRowGroups;
  if (fused) {
    if (!wide) {
      hipLaunchKernelGGL((k_combine<kCombEpi, 1>), dim3(2 * grid), dim3(512), 0, stream, a);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((k_combine<kCombF32, 4>), dim3(16 * grid), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_fused_epilogue, dim3(grid), dim3(256), 0, stream, a);
  } else {
    if (wide) hipLaunchKernelGGL((k_combine<kCombBf16, 4>), dim3(16 * grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((k_combine<kCombBf16, 1>), dim3(16 * grid), dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_debug_gather(const DecodeArgs& a, int kv_format, bool sparse, int b, int t, int j,
                               uint16_t* dst, hipStream_t stream) {
  if (kv_format == kKvBf16) {
    if (sparse) hipLaunchKernelGGL((k_debug_gather<kKvBf16, true>), dim3(1), dim3(kThreads), 0, stream, a, b, t, j, dst);
    else hipLaunchKernelGGL((k_debug_gather<kKvBf16, false>), dim3(1), dim3(kThreads), 0, stream, a, b, t, j, dst);
  } else {
    if (sparse) hipLaunchKernelGGL((k_debug_gather<kKvFp8V32, true>), dim3(1), dim3(kThreads), 0, stream, a, b, t, j, dst);
    else hipLaunchKernelGGL((k_debug_gather<kKvFp8V32, false>), dim3(1), dim3(kThreads), 0, stream, a, b, t, j, dst);
  }
  return hipGetLastError();
}

// Workspace of the allocation-free decode entry point: one copy per GPU the
// library runs on, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol); it passes the device address hipGetSymbolAddress returns for the
// current device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device; null until looked up
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace mla

#ifdef MLA_PHASE_TRACE
// Measurement library only: the phase timeline of the last decode launches
// (see the phase-timeline note at the top of this file).
extern "C" int mla_phase_trace_copy(void* times, void* items, int nwg) {
  if (nwg < 0 || nwg > mla::kTrWgs) return -1;
  if (hipMemcpyFromSymbol(times, HIP_SYMBOL(mla::g_phase_t), sizeof(uint64_t) * mla::kTrPer * nwg) != hipSuccess)
    return -2;
  if (hipMemcpyFromSymbol(items, HIP_SYMBOL(mla::g_phase_items), sizeof(int) * mla::kTrPieces * nwg) != hipSuccess)
    return -3;
  return 0;
}
extern "C" int mla_phase_trace_clear(void) {
  static uint64_t zt[mla::kTrWgs * mla::kTrPer];
  static int zi[mla::kTrWgs * mla::kTrPieces];
  if (hipMemcpyToSymbol(HIP_SYMBOL(mla::g_phase_t), zt, sizeof zt) != hipSuccess) return -1;
  return hipMemcpyToSymbol(HIP_SYMBOL(mla::g_phase_items), zi, sizeof zi) == hipSuccess ? 0 : -2;
}
#endif
