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
//  * KV blocks are staged with LDS-DMA (buffer_load ... lds, 16 B per lane)
//    into a double-buffered, XOR-swizzled [64][576] bf16 tile.  The buffer
//    resource of a block covers only its valid tokens, so rows past the
//    sequence length are written as zeros by the hardware and poisoned
//    (NaN) tail slots are never read.
//  * Lazy rescaling: the running max used for exponentiation only moves
//    when a new block max exceeds it by more than 2^8, so the 256-register
//    O accumulator is almost never rescaled ("skip scale", AI Wiki, section
//    "The Ascend kernel deep-dive"); exact up to rounding.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <cstdint>
#include <cmath>

#include "mla_internal.h"

namespace mla {

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
// Buffer accesses with cache policy sc0 sc1: they go past the CU's L1 and
// the XCD's L2 to the coherent memory side, so a store that has completed is
// seen by a load of this kind from any XCD without L2 write-back or
// invalidation.  Used for the split partials the in-kernel combine reads.
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
constexpr int kCoherent = 1 | 16;
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
// This lane's index, recomputed (mbcnt) where it is used, so per-lane LDS
// address bases live only inside a step, never across the KV loop: there the
// allocator may spill them, and each reload of a spill would cost a full
// vmcnt wait in a loop that keeps KV loads in flight.
__device__ __forceinline__ int fresh_lane() {
  return opaque(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
}

// S^T = K Q^T step on v_mfma_f32_32x32x16_bf16 with the accumulator held in
// VGPRs.  Written as inline asm because the builtin lets the compiler move
// every MFMA accumulator to AGPRs, and the 256 AGPRs are exactly the O
// accumulator of a 32-row wave tile; S then overflows and spills.  The asm is
// not volatile, so the scheduler still hoists the LDS reads feeding it.
__device__ __forceinline__ void mfma_s_first(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_acc(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// O^T += V^T P^T step with the accumulator pinned to AGPRs for its whole
// life (a builtin leaves O's register class to the allocator, which then
// shuffles the 256 accumulators between VGPRs and AGPRs inside the loop).
// Back-to-back accumulation into the same registers needs no wait states.
__device__ __forceinline__ void mfma_o(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
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
k_sched(const int32_t* __restrict__ seqlens, int B, int rows, int topk, int S,
        int32_t* __restrict__ meta, int32_t* __restrict__ num_splits) {
  constexpr int kSchedThreads = NT;
  __shared__ int32_t U[MAXB + 1];   // cost prefix: start of sequence b on the line
  __shared__ int32_t I[MAXB + 1];   // item prefix
  __shared__ int wsum[NT / 64];
  const int tid = threadIdx.x;
  const int F = [&] {
    int m = rows < kRowsPerWg ? rows : kRowsPerWg;
    int f = (m + 31) / 32;
    return f < 1 ? 1 : f;
  }();
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
  int cap = (T + 1 + S - 1) / S;
  if (cap < 2 * F) cap = 2 * F;
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
  // in-kernel combine control area: the split sequences in order, zeroed
  // counters, and the task count (4 row tiles per row group)
  {
    int32_t* ctl = num_splits + B + 1;
    const int G = (rows + kRowsPerWg - 1) / kRowsPerWg;
    auto nsplit = [&](int b) {
      int items = U[b + 1] - U[b] - F;
      items = items > 0 ? items : 1;
      int p0 = U[b] + F;
      return (p0 + items - 1) / cap - p0 / cap + 1;
    };
    int fc = 0;
    for (int b = lo; b < hi; ++b) fc += nsplit(b) > 1;
    int tot_f;
    int f0 = block_scan_exclusive<NT>(fc, wsum, &tot_f);
    for (int b = lo; b < hi; ++b)
      if (nsplit(b) > 1) ctl[3 + f0++] = b;
    for (int i = tid; i < 2 * kCtlGroups * B; i += kSchedThreads) ctl[3 + B + i] = 0;
    if (tid == 0) {
      ctl[0] = tot_f * (G <= kCtlGroups ? G : 0) * 16;  // 16 combine tasks per (sequence, row group)
      ctl[1] = 0;
      ctl[2] = 0;
    }
  }
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
// through a ring of 4 slots: two are computed on (S^T of one, P V of the
// other) while the next two are in flight.
// ---------------------------------------------------------------------------
constexpr int kHalfRows = 32;
constexpr int kMainStride = 1040;
constexpr int kRopeOff = kHalfRows * kMainStride;               // 33280
constexpr int kRopeStride = 128;
constexpr int kHalfBytes = kRopeOff + kHalfRows * kRopeStride;  // 37376
constexpr int kLoadsPerHalf = kHalfRows / kWaves + 1;           // 9 per wave: 8 rows + rope
constexpr int kTileRing = 4;  // bf16 half-tile slots
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

// Sparse bf16: row r is flat pool token ids[r] when r < nvalid and
// ids[r] >= 0, else zeros.  Same 9 loads per wave as the dense loader.
__device__ __forceinline__ void load_row_bf16_sparse(uint8_t* slot, const uint8_t* kv,
                                                     const int32_t* ids, int nvalid, int wave, int k) {
  const int l16 = fresh_lane() << 4;
  const uint32_t base = lds_off(slot);
  if (k < kHalfRows / kWaves) {
    const int r = wave + kWaves * k;
    const int id = uni(r < nvalid ? ids[r] : -1);
    const uint8_t* src = uni_ptr(id >= 0 ? kv + (int64_t)id * kRowBytes : g_zero_row);
    dma_glb16_s(base + r * kMainStride, l16, src);
  } else {
    const int rr = 8 * wave + (l16 >> 7);
    const int id = rr < nvalid ? ids[rr] : -1;
    const int cc = rope_phys_chunk(rr, (l16 >> 4) & 7);
    const uint8_t* g = id >= 0 ? kv + (int64_t)id * kRowBytes + 1024 + cc * 16 : g_zero_row + 1024 + cc * 16;
    dma_glb16(base + kRopeOff + wave * 1024, g);
  }
}
__device__ __forceinline__ void load_half_bf16_sparse(uint8_t* slot, const uint8_t* kv,
                                                      const int32_t* ids, int nvalid, int wave,
                                                      int /*lane*/) {
#pragma unroll
  for (int k = 0; k < kLoadsPerHalf; ++k) load_row_bf16_sparse(slot, kv, ids, nvalid, wave, k);
}

// FP8 V3.2 records of one half (32 x 656 B = 1312 chunks) are staged raw by
// LDS-DMA into a 24 KB slot (24 loads per half, 6 per wave; the tail of the
// slot is padding), then dequantised LDS -> LDS into a bf16 half tile.
// V4.1 records (32 x 528 B = 1056 chunks) use the same slot with 20 loads.
constexpr int kFp8ChunksPerTok = kFp8TokenBytes / 16;        // 41
constexpr int kRawHalfChunks = kHalfRows * kFp8ChunksPerTok;  // 1312
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
__device__ __forceinline__ void load_half_fp8_sparse(uint8_t* raw, const uint8_t* kv,
                                                     const int32_t* ids, int nvalid, int wave,
                                                     int lane) {
  constexpr int kTok = tok_bytes<KVF>(), kChunks = kTok / 16, kHalfChunks = kHalfRows * kChunks;
  lane = fresh_lane();
#pragma unroll
  for (int ii = 0; ii < raw_loads_per_wave<KVF>(); ++ii) {
    const int i = ii * kWaves + wave;
    const int pos_all = i * 64 + lane;
    const int r = pos_all / kChunks;
    const int c = pos_all - r * kChunks;
    const int id = (pos_all < kHalfChunks && r < nvalid) ? ids[r] : -1;
    const uint8_t* g =
        id >= 0 ? kv + (int64_t)id * kTok + c * 16 : g_zero_row + (pos_all & 63) * 16;
    dma_glb16(lds_off(raw) + i * 1024, g);
  }
}

// Scales of an FP8 half tile in LDS, in the register order of the S^T
// accumulator: [tile t][lane half h][i] holds the scale of dims 128t.. of
// key key_of_row(8*(i/4) + i%4) + h.
constexpr int kScaleBytes = 4 * 2 * 16 * 4;
__device__ __forceinline__ int scale_slot(int key) {  // key -> h*16 + i
  const int h = key & 1, kc = key - h, rem = kc & 15;
  return h * 16 + 8 * (kc >> 4) + 4 * ((rem >> 1) & 1) + (rem >> 2);
}

// 32 raw records -> the bf16 half tile with the e4m3 codes of dims < 512
// converted exactly (every e4m3 value is a bf16 value), dims 512..575
// copied, and the fp32 tile scales moved to `scl`.  The decode applies the
// scales in fp32: to each tile's partial scores in QK^T and to P in P.V, so
// no product code*scale is ever rounded to bf16.  An all-zero record gives a
// zero row with zero scales.
__device__ __forceinline__ void dequant_codes(uint8_t* tile, float* scl, const uint8_t* raw, int tid) {
  tid = (tid & ~63) | fresh_lane();  // keep the per-thread addresses out of the loop's live set
  // All code reads first, then the conversions and writes: the compiler
  // cannot move a read of the raw slot above a write to the tile (same LDS
  // array), so interleaved they would each wait out a full LDS latency.
  constexpr int kPer = kHalfRows * 64 / kThreads;
  uint2 codes[kPer];
#pragma unroll
  for (int kk = 0; kk < kPer; ++kk) {
    const int k = kk * kThreads + tid;
    codes[kk] = *reinterpret_cast<const uint2*>(raw + (k >> 6) * kFp8TokenBytes + (k & 63) * 8);
  }
  const uint4 rope = *reinterpret_cast<const uint4*>(raw + (tid >> 3) * kFp8TokenBytes + 528 + (tid & 7) * 16);
#pragma unroll
  for (int kk = 0; kk < kPer; ++kk) {
    const int k = kk * kThreads + tid;
    const int r = k >> 6, c = k & 63;
    const uint2 code = codes[kk];
    const uint32_t cw[2] = {code.x, code.y};
    uint32_t w[4];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      // two codes -> two bf16 in one instruction; with scale 1 the result is exact
      w[2 * hh] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[hh], 1.0f, false));
      w[2 * hh + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[hh], 1.0f, true));
    }
    *reinterpret_cast<uint4*>(tile + r * kMainStride + c * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  {
    const int r = tid >> 3, c = tid & 7;
    *reinterpret_cast<uint4*>(tile + kRopeOff + r * kRopeStride + (rope_phys_chunk(r, c) << 4)) = rope;
  }
  if (tid < 4 * kHalfRows) {
    const int r = tid >> 2, t = tid & 3;
    scl[t * 32 + scale_slot(r)] = *reinterpret_cast<const float*>(raw + r * kFp8TokenBytes + 512 + 4 * t);
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
  tid = (tid & ~63) | fresh_lane();
  constexpr int kPer = kHalfRows * 64 / kThreads;
  uint2 codes[kPer];
  uint32_t ebits[kPer];
#pragma unroll
  for (int kk = 0; kk < kPer; ++kk) {
    const int k = kk * kThreads + tid;
    const uint8_t* rec = raw + (k >> 6) * kFp8V41TokenBytes;
    codes[kk] = *reinterpret_cast<const uint2*>(rec + (k & 63) * 8);
    ebits[kk] = rec[512 + ((k & 63) >> 2)];  // 8 codes of dims 8c.. share scale c/4
  }
#pragma unroll
  for (int kk = 0; kk < kPer; ++kk) {
    const int k = kk * kThreads + tid;
    const int r = k >> 6, c = k & 63;
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
__device__ __forceinline__ V41Chunk v41_read(const uint8_t* raw, int wave_base, int kk) {
  const int k = kk * kThreads + (wave_base | fresh_lane());
  const uint8_t* rec = raw + (k >> 6) * kFp8V41TokenBytes;
  return V41Chunk{*reinterpret_cast<const uint2*>(rec + (k & 63) * 8), rec[512 + ((k & 63) >> 2)]};
}
__device__ __forceinline__ void v41_write(uint8_t* tile, int wave_base, int kk, const V41Chunk& ch) {
  const int k = kk * kThreads + (wave_base | fresh_lane());
  const float scale = e8m0_scale(ch.e);
  const uint32_t cw[2] = {ch.code.x, ch.code.y};
  uint32_t w[4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    w[2 * hh] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[hh], scale, false));
    w[2 * hh + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[hh], scale, true));
  }
  *reinterpret_cast<uint4*>(tile + (k >> 6) * kMainStride + (k & 63) * 16) = make_uint4(w[0], w[1], w[2], w[3]);
}

// Dequantise 32 raw records into the bf16 half tile: dims < 512 are
// e4m3 * fp32 tile scale computed in fp32 and rounded once to bf16 (RNE);
// dims 512..575 are copied.  An all-zero record gives a zero row.  (The
// staged rows as the cache defines them; the decode itself keeps the codes
// and the scales apart, see dequant_codes.)
__device__ __forceinline__ void dequant_half_scaled(uint8_t* tile, const uint8_t* raw, int tid) {
#pragma unroll
  for (int kk = 0; kk < kHalfRows * 64 / kThreads; ++kk) {
    const int k = kk * kThreads + tid;
    const int r = k >> 6, c = k & 63;
    const uint8_t* rec = raw + r * kFp8TokenBytes;
    const uint2 code = *reinterpret_cast<const uint2*>(rec + c * 8);
    const float sc = *reinterpret_cast<const float*>(rec + 512 + (c >> 4) * 4);
    const uint32_t cw[2] = {code.x, code.y};
    uint32_t w[4];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      typedef __attribute__((ext_vector_type(2))) float f2;
      f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(cw[hh], false);
      f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(cw[hh], true);
      __bf16 b0 = (__bf16)(lo[0] * sc), b1 = (__bf16)(lo[1] * sc);
      __bf16 b2 = (__bf16)(hi[0] * sc), b3 = (__bf16)(hi[1] * sc);
      w[2 * hh] = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
      w[2 * hh + 1] = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
    }
    *reinterpret_cast<uint4*>(tile + r * kMainStride + c * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  {
    const int r = tid >> 3, c = tid & 7;
    const uint4 v = *reinterpret_cast<const uint4*>(raw + r * kFp8TokenBytes + 528 + c * 16);
    *reinterpret_cast<uint4*>(tile + kRopeOff + r * kRopeStride + (rope_phys_chunk(r, c) << 4)) = v;
  }
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
// pos is theta = pos * base^(-2i/64) (the inverse frequencies come from the
// host in fp64).  Positions reach 10^4 radians, so theta is formed and
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
// low half of its row's dims and i1 for the high half.  When every row of
// the wave sits at one position (always with one query token per sequence),
// each of the 32 pairs is computed once, pair lane & 31 on each lane, and
// read back by lane index; otherwise each lane computes its own pairs.
struct RopeRow {
  bool shared;
  double pos;
  float c, s;
};
__device__ __forceinline__ RopeRow rope_row(double pos, bool row_ok, const double* inv_freq, float sign) {
  RopeRow r;
  const double pos0 = __builtin_bit_cast(double, uni_u64(__builtin_bit_cast(uint64_t, pos)));
  r.shared = __builtin_amdgcn_ballot_w64(row_ok && pos != pos0) == 0;
  r.pos = pos;
  r.c = 0.f;
  r.s = 0.f;
  if (r.shared) rope_cs(pos0, inv_freq[fresh_lane() & 31], sign, r.c, r.s);
  return r;
}
__device__ __forceinline__ void rope_pair(const RopeRow& r, const double* inv_freq, float sign, int i0, int i1,
                                          bool hi, float& c, float& s) {
  if (r.shared) {
    const float c0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r.c), i0));
    const float c1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r.c), i1));
    const float s0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r.s), i0));
    const float s1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r.s), i1));
    c = hi ? c1 : c0;
    s = hi ? s1 : s0;
  } else {
    rope_cs(r.pos, hi ? inv_freq[i1] : inv_freq[i0], sign, c, s);
  }
}

// ---------------------------------------------------------------------------
// Decode kernel
//
// Query fragments.  bf16 KV: all 36 k-steps stay in VGPRs (144), which
// leaves the LDS to the four-slot tile ring.  FP8 KV, whose dequantisation
// and per-tile scaling need more registers: dims 0..383 (k-steps 0..23) in
// VGPRs, dims 384..575 (k-steps 24..35) in a per-wave LDS region
// [32 rows][24 chunks] swizzled like the KV tile.
// ---------------------------------------------------------------------------
// k-steps of 16 dims in a query row: d_qk = 576, or 512 for V4.1 records
template <int KVF>
constexpr int ksteps() { return KVF == kKvFp8V41 ? 32 : 36; }
template <int KVF>
constexpr int dqk_of() { return 16 * ksteps<KVF>(); }
template <int KVF>
constexpr int q_reg_steps() { return KVF == kKvFp8V32 ? 24 : ksteps<KVF>(); }
template <int KVF>
constexpr int q_lds_row_bytes() { return (ksteps<KVF>() - q_reg_steps<KVF>()) * 2 * 16; }    // fp8: 384
template <int KVF>
constexpr int q_lds_wave_bytes() { return 32 * q_lds_row_bytes<KVF>(); }          // fp8: 12288
constexpr int kQRegStepsFp8 = q_reg_steps<kKvFp8V32>();
constexpr int kIdsSlots = 6;

template <int KVF, bool SPARSE>
struct DecodeLayout {
  static constexpr int kTileOff = 0;                                   // bf16 half tiles
  static constexpr int kTiles = KVF == kKvBf16 ? kTileRing : KVF == kKvFp8V41 ? 2 : 1;
  static constexpr int kRawOff = kTiles * kHalfBytes;                  // fp8 raw slots
  static constexpr int kQOff = kRawOff + (KVF == kKvBf16 ? 0 : kRing * kRawSlotBytes);
  static constexpr int kIdsOff = kQOff + kWaves * q_lds_wave_bytes<KVF>();
  static constexpr int kWalkOff = kIdsOff + (SPARSE ? kIdsSlots * 256 : 0);  // 2 words per wave
  static constexpr int kSclOff = kWalkOff + (KVF == kKvBf16 && !SPARSE ? kWaves * 8 : 0);
  static constexpr int kSmem = kSclOff + (KVF == kKvFp8V32 ? kScaleBytes : 0);
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

template <bool FUSED>
__device__ void combine_phase(const DecodeArgs& a, uint8_t* lds);

template <int KVF, bool SPARSE, bool FUSED>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_decode(DecodeArgs a) {
  using Lay = DecodeLayout<KVF, SPARSE>;
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
  if (b0 < 0) {  // no decode work: only combine tasks
    if constexpr (!FUSED) {
      if (a.ctl) combine_phase<FUSED>(a, smem);
    }
    return;
  }
  const int j0 = uni(sload(ms, 1)), b1 = uni(sload(ms, 2)), j1 = uni(sload(ms, 3)),
            nitems = uni(sload(ms, 5));
  int split_k = uni(sload(ms, 4));
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
    return reinterpret_cast<int32_t*>(smem + Lay::kIdsOff) + (step % kIdsSlots) * 64;
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
  auto fetch_phys = [&]() {
    const bool any = lb <= b1 && lj * kPage < lL;
    if constexpr (kVecWalk) {
      lany = any;
      if (any) fetch_word(0, bt_rs, (lb * a.max_blocks + lj) * 4);
    } else if constexpr (!SPARSE) {
      lphys = any ? uni(sload(a.block_table, (int64_t)lb * a.max_blocks + lj)) : 0;
    }
  };
  auto fetch_next_len = [&]() {
    if constexpr (kVecWalk) fetch_word(1, sl_rs, min(lb + 1, b1) * 4);
  };
  auto land = [&]() {
    if constexpr (kVecWalk) {
      lphys = lany ? uni(walk[0]) : 0;
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
  if constexpr (kVecWalk) {
    __builtin_amdgcn_s_waitcnt(0);  // kernel start: nothing else is in flight yet
    lds_barrier();
  }
  land();
  // stage the walker's step as step `step` into its ring slot
  auto issue_load = [&](int step) {
    const int rs = step % (KVF == kKvBf16 ? kTileRing : kRing);
    if constexpr (!SPARSE) {
      const bool any = lj * kPage < lL;
      const int valid = any ? min(kPage, lL - lj * kPage) : 0;
      if constexpr (KVF == kKvBf16)
        load_half_bf16_dense(smem + Lay::kTileOff + rs * kHalfBytes, a.kv, lphys, valid, lh, wave, lane);
      else
        load_half_fp8_dense(smem + Lay::kRawOff + rs * kRawSlotBytes, a.kv, lphys, valid, lh, wave, lane);
    } else {
      const int nvalid = min(kHalfRows, a.topk - lj * kPage - lh * kHalfRows);
      if constexpr (KVF == kKvBf16)
        load_half_bf16_sparse(smem + Lay::kTileOff + rs * kHalfBytes, a.kv, ids_slot(step), nvalid,
                              wave, lane);
      else
        load_half_fp8_sparse<KVF>(smem + Lay::kRawOff + rs * kRawSlotBytes, a.kv, ids_slot(step), nvalid,
                             wave, lane);
    }
  };

  // bf16 path: the loads of step+3 are captured by prepare_load() at the
  // start of step `step` and issued by emit_load(k), k < kLoadsPerHalf, after
  // the walker's and the ids' word loads of that step.  Past the slot's last
  // step the same instructions stage zeros into the free slot, so every step
  // issues exactly kLoadsPerHalf tile loads, last.  (Spreading the nine instructions between the MFMAs was
  // measured: no gain, the address unit's queue blocks the wave either way.)
  int pl_step = 0, pl_valid = 0, pl_h = 0, pl_nvalid = 0;
  int64_t pl_phys = 0;
  auto prepare_load = [&](int st) {
    const bool do_load = st < nsteps;
    pl_step = st;
    pl_h = lh;
    if constexpr (!SPARSE) {
      const bool any = do_load && lj * kPage < lL;
      pl_valid = any ? min(kPage, lL - lj * kPage) : 0;
      pl_phys = any ? lphys : 0;
    } else {
      pl_nvalid = do_load ? min(kHalfRows, a.topk - lj * kPage - lh * kHalfRows) : 0;
    }
    if (do_load) advance_load();
  };
  auto emit_load = [&](int k) {
    uint8_t* slot = smem + Lay::kTileOff + (pl_step % kTileRing) * kHalfBytes;
    if constexpr (!SPARSE) load_row_bf16_dense(slot, a.kv, pl_phys, pl_valid, pl_h, wave, k);
    else load_row_bf16_sparse(slot, a.kv, ids_slot(pl_step), pl_nvalid, wave, k);
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
  // FP8 loads lead by kRawAhead steps, ids by kRawAhead + 2 (V4.1, whose
  // step dequantises one step ahead, by one more)
  constexpr int kRawAhead = KVF == kKvFp8V41 ? 3 : 2;
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

  // ---- prologue: ids of steps 0..3; the loads of steps 0..2 are issued in
  // the first piece's prologue (bf16: steps 0 and 1 right after the query
  // loads, step 2 once the walker has landed the block of its item)
  if constexpr (SPARSE) {
    for (int s = 0; s < min(KVF == kKvFp8V41 ? 5 : 4, nsteps); ++s) {
      fetch_ids(fb, fj, fh, s);
      advance(fb, fj, fh);
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  auto issue_first_loads = [&]() {
    for (int s = 0; s < min(KVF == kKvFp8V41 ? 3 : 2, nsteps); ++s) {
      issue_load(s);
      advance_load();
    }
  };
  if constexpr (KVF != kKvBf16) issue_first_loads();

  constexpr int kQR = q_reg_steps<KVF>();
  uint8_t* qlds = smem + Lay::kQOff + wave * q_lds_wave_bytes<KVF>();
  // FP8: Q rows are 384 B apart (an 8-group shift): chunk c of row r at
  // c ^ ((r >> 1) & 7) puts the 16 rows of a read phase on distinct groups
  const int x = (r32 >> 1) & 7;
  bf16x8 qf[kQR];
  f32x16 o[16];
  bool first_piece = true;

  int cb = b0, cj = j0, step = 0;
  while (step < nsteps) {
    // ======== one piece: sequence cb, items cj .. piece_end-1
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
    // Query fragments of this piece.  Fused: q^ = inv * RoPE(q (.) w) with
    // inv = 1 / sqrt(mean(q^2) + eps) (RMSNorm over the row's 576 dims, then
    // RoPE on dims 512..575 at position len - s_q + t; RoPE is linear, so the
    // row factor commutes with it).  The fragments hold bf16(RoPE(q (.) w))
    // chunk by chunk and inv joins the row's softmax scale, applied to S in
    // fp32; no chunk has to wait for the whole row's statistic.
    float srow = a.scale_log2;  // log2(e) * softmax scale (* inv when fused)
    {
      const uint16_t* qrow = a.q + ((int64_t)cb * a.rows + (row_ok ? row : 0)) * dqk_of<KVF>();
      float ss = 0.f;
      const double pos = (double)Lb - (double)a.s_q + (double)tok;
      // chunk ks (dims 16ks + 8half .. +7): q-hat chunk, then its home
      auto put_q = [&](int ks, bf16x8 v) {
        if (!row_ok) v = bf16x8{};
        if (ks < kQR) {
          qf[ks] = v;
        } else {
          const int cq = 2 * (ks - kQR) + half;
          *reinterpret_cast<bf16x8*>(qlds + r32 * q_lds_row_bytes<KVF>() + ((cq ^ x) << 4)) = v;
        }
      };
      if constexpr (!FUSED) {
#pragma unroll
        for (int ks = 0; ks < ksteps<KVF>(); ++ks) put_q(ks, *reinterpret_cast<const bf16x8*>(qrow + (2 * ks + half) * 8));
      } else {
        // Six batches of 6 chunks (the RoPE chunks 32..35 first), each
        // batch's q and weight loads issued together: all 72 in flight at
        // once would not fit in the registers beside the fragments.
        constexpr int kBatch = 6;
        const RopeRow rr = rope_row(pos, row_ok, a.rope_inv_freq, 1.0f);
#pragma unroll
        for (int bt = 0; bt < 36 / kBatch; ++bt) {
          bf16x8 vb[kBatch], wb[kBatch];
#pragma unroll
          for (int i = 0; i < kBatch; ++i) {
            const int n = bt * kBatch + i, ks = n < 4 ? 32 + n : n - 4;
            vb[i] = *reinterpret_cast<const bf16x8*>(qrow + (2 * ks + half) * 8);
            wb[i] = *reinterpret_cast<const bf16x8*>(a.norm_w + (2 * ks + half) * 8);
          }
#pragma unroll
          for (int i = 0; i < kBatch; ++i) {
            const int n = bt * kBatch + i, ks = n < 4 ? 32 + n : n - 4;
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float qv = (float)vb[i][e];
              ss += qv * qv;
              y[e] = qv * (float)wb[i][e];
            }
            if (ks >= 32) {
#pragma unroll
              for (int pp = 0; pp < 4; ++pp) {
                float cs, sn;
                rope_pair(rr, a.rope_inv_freq, 1.0f, 8 * (ks - 32) + pp, 8 * (ks - 32) + 4 + pp, half, cs, sn);
                const float x0 = y[2 * pp], x1 = y[2 * pp + 1];
                y[2 * pp] = x0 * cs - x1 * sn;
                y[2 * pp + 1] = x0 * sn + x1 * cs;
              }
            }
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (__bf16)y[e];
            put_q(ks, v);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (FUSED) {
        ss = row_sum2(ss);
        srow *= 1.0f / sqrtf(ss / (float)kDqk + a.norm_eps);
      }
    }
    if constexpr (KVF == kKvBf16) {
      if (first_piece) issue_first_loads();  // after the query loads: latencies overlap
    }
    wait_vmcnt<0>();
    lds_barrier();  // every wave's loads of the piece's first step (and Q in LDS) landed
    if constexpr (KVF == kKvBf16) {
      if (first_piece) {
        // step 2: the drain above landed the walker's block of its item
        land();
        prepare_load(2);
#pragma unroll
        for (int k = 0; k < kLoadsPerHalf; ++k) emit_load(k);
      }
    }
    first_piece = false;

    // ======== building blocks of one 32-key step
    auto tile_off = [&](int st) -> int {
      if constexpr (KVF == kKvBf16) return Lay::kTileOff + (st % kTileRing) * kHalfBytes;
      else if constexpr (KVF == kKvFp8V41) return Lay::kTileOff + (st & 1) * kHalfBytes;
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
      bf16x8 kbuf[kLa];
#pragma unroll
      for (int i = 0; i < kLa; ++i) kbuf[i] = read_k(i);
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const bf16x8 ka = kbuf[ks % kLa];
        const bf16x8 qb = qf[ks < kQR ? ks : 0];
        if (ks + kLa < kKS) kbuf[ks % kLa] = read_k(ks + kLa);
        if (ks == 0) mfma_s_first(sc, ka, qb);
        else mfma_s_acc(sc, ka, qb);
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
        mfma_o(o[i & 15], va, pf[i >> 4]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // FP8: S^T from the exact codes, one 128-dim tile at a time, each tile's
    // partial scores scaled by its per-key fp32 scale before they are summed;
    // the RoPE block (bf16 in the cache) adds unscaled.
    const float* scl = reinterpret_cast<const float*>(smem + Lay::kSclOff);
    auto qk_fp8 = [&](int tb, f32x16& sc) {
      constexpr int kLa = 2;  // the tile accumulator costs 16 VGPRs: shorter lookahead
      const int ln = fresh_lane(), lr = ln & 31, lh = ln >> 5;
      const int lkey = key_of_row(lr), lfr = (lkey >> 1) & 7, lx = (lr >> 1) & 7;
      const int koff = tb + lkey * kMainStride + 16 * lh;
      const int kroff = tb + kRopeOff + lkey * kRopeStride;
      const int qb = Lay::kQOff + wave * q_lds_wave_bytes<KVF>() + lr * q_lds_row_bytes<KVF>();
      int qoff[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) qoff[e] = qb + ((((2 * e) | lh) ^ lx) << 4);
      auto read_k = [&](int ks) {
        if (ks < 32) return *reinterpret_cast<const bf16x8*>(smem + koff + 32 * ks);
        return *reinterpret_cast<const bf16x8*>(smem + kroff + ((((2 * (ks - 32)) | lh) ^ lfr) << 4));
      };
      auto read_q = [&](int ks) {
        return *reinterpret_cast<const bf16x8*>(smem + qoff[(ks - kQRegStepsFp8) & 3] +
                                                ((ks - kQRegStepsFp8) >> 2) * 128);
      };
      const f32x4* sv = reinterpret_cast<const f32x4*>(scl + lh * 16);
      bf16x8 kbuf[kLa], qbuf[kLa];
      // Two partial accumulators alternate between the 128-dim tiles: tile
      // t's fold (sc += part * scale) runs between the first MFMAs of tile
      // t+1, so the MFMA pipe does not wait for it.  Fold of tile tp: settle
      // and scale reads after MFMA 8(tp+1), quarter q after MFMA 8(tp+1)+1+q
      // (tile 3's last quarter after the loop).  The RoPE tile (ks 32..35)
      // adds unscaled at the end.
      f32x16 part[2];
      f32x4 s4[4];
      auto fold_quarter = [&](int tp, int q) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sc[4 * q + e] = (tp == 0 ? 0.f : sc[4 * q + e]) + part[tp & 1][4 * q + e] * s4[q][e];
      };
#pragma unroll
      for (int i = 0; i < kLa; ++i) kbuf[i] = read_k(i);
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        const bf16x8 ka = kbuf[ks % kLa];
        const bf16x8 qb = ks < kQR ? qf[ks < kQR ? ks : 0] : qbuf[ks % kLa];
        if (ks + kLa < 36) {
          kbuf[ks % kLa] = read_k(ks + kLa);
          if (ks + kLa >= kQRegStepsFp8) qbuf[ks % kLa] = read_q(ks + kLa);
        }
        const int t = ks >> 3, u = ks & 7;
        if (u == 0) mfma_s_first(part[t & 1], ka, qb);
        else mfma_s_acc(part[t & 1], ka, qb);
        if (t >= 1) {
          const int tp = t - 1;
          if (u == 0) {
            mfma_s_settle(part[tp & 1]);
#pragma unroll
            for (int q = 0; q < 4; ++q) s4[q] = sv[tp * 8 + q];
          } else if (u <= 4) {
            fold_quarter(tp, u - 1);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      fold_quarter(3, 3);
      mfma_s_settle(part[0]);
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] += part[0][i];
    };
    // FP8: O^T += V^T P_t^T where V holds the exact codes and P_t = p * the
    // keys' scale of tile t (d-tiles 4t..4t+3), rounded once to bf16.
    auto pv_fp8 = [&](int tb, const f32x16& p) {
      const int ln = fresh_lane(), lh = ln >> 5;
      const f32x4* sv = reinterpret_cast<const f32x4*>(scl + lh * 16);
      constexpr int kVa = 2;
      const int voff = tb + (4 * ((ln & 15) >> 2) + lh) * kMainStride + 32 * ((ln >> 4) & 1) + 8 * (ln & 3);
      auto read_v = [&](int i) {  // i = kq * 16 + mt
        const int kq = i >> 4, mt = i & 15;
        const uint8_t* pp = smem + voff + kq * 16 * kMainStride + mt * 64;
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(pp));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(pp + 2 * kMainStride));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      // mt order: the four d-tiles of one scale tile, both key halves; one
      // stream of 32 MFMAs, i = 8t + j.  The V reads run kVa MFMAs ahead
      // across tile boundaries.  Tile t+1's scaled P goes to the other half
      // of pt while tile t's MFMAs run: scale reads after MFMA j = 0, one
      // quarter after each of MFMAs 3..6 (three MFMAs after the last read of
      // that half by tile t-1), settled after MFMA 7.
      auto scale_p = [&](bf16x8 (&dst)[2], int q, const f32x4& s4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[q >> 1][4 * (q & 1) + e] = (__bf16)(p[4 * q + e] * s4[e]);
      };
      auto v_index = [](int i) { return ((i & 7) >> 2) * 16 + 4 * (i >> 3) + (i & 3); };  // kq * 16 + mt
      bf16x8 pt[2][2];
      f32x4 s4[4];
      asm volatile("" ::: "memory");
#pragma unroll
      for (int q = 0; q < 4; ++q) scale_p(pt[0], q, sv[q]);
      valu_to_mfma_settle(pt[0][0], pt[0][1]);
      bf16x8 vbuf[kVa];
#pragma unroll
      for (int i = 0; i < kVa; ++i) vbuf[i] = read_v(v_index(i));
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int t = i >> 3, j = i & 7;
        const bf16x8 va = vbuf[i % kVa];
        if (i + kVa < 32) vbuf[i % kVa] = read_v(v_index(i + kVa));
        mfma_o(o[4 * t + (j & 3)], va, pt[t & 1][j >> 2]);
        if (t + 1 < 4) {
          if (j == 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) s4[q] = sv[(t + 1) * 8 + q];
          } else if (j >= 3 && j <= 6) {
            scale_p(pt[(t + 1) & 1], j - 3, s4[j - 3]);
          } else if (j == 7) {
            valu_to_mfma_settle(pt[(t + 1) & 1][0], pt[(t + 1) & 1][1]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto key0_of = [&](int ps) { return (cj + (ps >> 1)) * kPage + (ps & 1) * kHalfRows; };
    auto has_keys = [&](int ps) {
      const int k0 = key0_of(ps);
      return SPARSE ? (k0 < a.topk) : (k0 < Lb);
    };
    // Online softmax of one tile (log2 domain) in kSmSlices slices, so that
    // it can be spread between the MFMAs of the next tile's S^T.  Register i
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
            const uint64_t bm = __builtin_amdgcn_ballot_w64(ln < 32 && r < nvalid && ids_slot(st_step)[r] >= 0);
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
          st.pf[i >> 3][i & 7] = (__bf16)p;
          if constexpr (KVF != kKvBf16) sc[i] = p;
        }
      } else {
        lsum = lsum * st.alpha + st.psum;
      }
    };
    constexpr int kSmSlices = 11;
    // k-step of the next tile's S^T after whose MFMA slice k runs
    auto slice_at = [](int k) { return k < 6 ? 2 * k : 12 + 3 * (k - 6); };
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
      // ---- bf16: step ps computes S^T of tile ps+1 with the softmax of tile
      // ps woven between its MFMAs, then O += P V of tile ps.  Tiles ps and
      // ps+1 are resident; tiles ps+2 (issued a step ago) and ps+3 (issued
      // now, into tile ps-1's slot) are in flight.
      const int n = 2 * (piece_end - cj);
      f32x16 sc_cur, sc_nxt;
      bool cur_has = has_keys(0);
      if (cur_has) qk(tile_off(step), sc_cur, [](int) {});
      for (int ps = 0; ps < n; ++ps, ++step) {
        const bool has_next = ps + 1 < n;
        const bool nxt_has = has_next && has_keys(ps + 1);
        // Tile ps+1 (issued two steps ago) and the word loads of the last step
        // landed: only that step's kLoadsPerHalf tile loads, issued after its
        // word loads, may still be in flight (vector loads complete in order).
        wait_vmcnt<kLoadsPerHalf>();
        lds_barrier();  // ... for every wave; tile ps-1's slot is free
        land();
        prepare_load(step + 3);
        fetch_next_ids(step);
#pragma unroll
        for (int k = 0; k < kLoadsPerHalf; ++k) emit_load(k);
        SmState st;
        const int key0 = key0_of(ps);
        if (nxt_has) {
          qk(tile_off(step + 1), sc_nxt, [&](int ks) {
#pragma unroll
            for (int k = 0; k < kSmSlices; ++k)
              if (ks == slice_at(k)) sm_slice(k, sc_cur, st, key0, step);
          });
        } else {
#pragma unroll
          for (int k = 0; k < kSmSlices; ++k) sm_slice(k, sc_cur, st, key0, step);
        }
        if (cur_has) {
          rescale_o(st);
          valu_to_mfma_settle(st.pf[0], st.pf[1]);
          pv(tile_off(step), st.pf);
        }
        sc_cur = sc_nxt;
        cur_has = nxt_has;
      }
    } else if constexpr (KVF == kKvFp8V41) {
      // ---- V4.1: two bf16 tiles.  Step s runs S^T, softmax and P.V on tile
      // s%2 and meanwhile dequantises step s+1's records into the other tile,
      // one chunk between every four MFMAs of S^T; one barrier per step.
      // Raw records go out three steps ahead (into the slot of the records
      // dequantised a step ago), ids five.
      const int wave_base = tid & ~63;
      auto dq_tile = [&](int st) { return smem + tile_off(st); };
      auto dq_raw = [&](int st) { return smem + Lay::kRawOff + (st % kRing) * kRawSlotBytes; };
      if (step == 0) {  // the first step's tile: the prologue drain landed its records
        dequant_v41(dq_tile(0), dq_raw(0), tid);
        lds_barrier();
      }
      for (int ps = 0; ps < 2 * (piece_end - cj); ++ps, ++step) {
        if (ps > 0) {
          // The previous step issued raw(step+2) (if any) and ids(step+4) (if
          // any), after everything this step needs: raw(step+1), ids(step+3).
          if (step + 2 >= nsteps) wait_vmcnt<0>();
          else if (step + 4 >= nsteps) wait_vmcnt<Lay::kVmPerStep - 1>();
          else wait_vmcnt<Lay::kVmPerStep>();
          lds_barrier();  // tile step%2 staged by every wave; P.V(step-1) done with the other
        }
        issue_next(step);
        const bool hk = has_keys(ps);
        const bool dq = step + 1 < nsteps;
        f32x16 sc;
        SmState st;
        if (hk && dq) {
          V41Chunk ch;
          qk(tile_off(step), sc, [&](int ks) {
            if ((ks & 3) == 0) ch = v41_read(dq_raw(step + 1), wave_base, ks >> 2);
            else if ((ks & 3) == 3) v41_write(dq_tile(step + 1), wave_base, ks >> 2, ch);
          });
        } else if (hk) {
          qk(tile_off(step), sc, [](int) {});
        } else if (dq) {
          dequant_v41(dq_tile(step + 1), dq_raw(step + 1), tid);
        }
        if (hk) {
#pragma unroll
          for (int k = 0; k < kSmSlices; ++k) sm_slice(k, sc, st, key0_of(ps), step);
          rescale_o(st);
          valu_to_mfma_settle(st.pf[0], st.pf[1]);
          pv(tile_off(step), st.pf);
        }
      }
    } else {
      // ---- FP8: one bf16 tile, dequantised from the raw ring each step
      for (int ps = 0; ps < 2 * (piece_end - cj); ++ps, ++step) {
        if (ps > 0) {
          // This step's loads were issued two steps ago; the previous step
          // then issued the loads of step+1 (if any) and, sparse, the ids of
          // step+3 (if any).  Wait for everything older than those.
          constexpr int kLoadsPerStep = Lay::kVmPerStep - (SPARSE ? 1 : 0);
          if (step + 1 >= nsteps) wait_vmcnt<0>();
          else if (SPARSE && step + 3 >= nsteps) wait_vmcnt<kLoadsPerStep>();
          else wait_vmcnt<Lay::kVmPerStep>();
          lds_barrier();  // every wave's loads of this step landed
        }
        dequant_codes(smem + Lay::kTileOff, reinterpret_cast<float*>(smem + Lay::kSclOff),
                      smem + Lay::kRawOff + (step % kRing) * kRawSlotBytes, tid);
        lds_barrier();  // the tile is staged; raw slot (step+2)%3 (dequantised last step) is free
        const bool hk = has_keys(ps);
        f32x16 sc;
        SmState st;
        if (hk) qk_fp8(tile_off(step), sc);
        // The loads of step+2 go out after S^T: the register reloads inside
        // S^T wait for every older load, and would otherwise wait for these.
        issue_next(step);
        if (hk) {
#pragma unroll
          for (int k = 0; k < kSmSlices; ++k) sm_slice(k, sc, st, key0_of(ps), step);
          rescale_o(st);
          pv_fp8(tile_off(step), sc);
        }
      }
    }

    // ======== finalize the piece: O / l and LSE; direct output or partial
    o_settle(o);
    {
      const float lt = row_sum2(lsum);
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
      const float lse2 = lt > 0.f ? m_used + __builtin_amdgcn_logf(lt) : -INFINITY;
      const int nsplit = uni(sload(a.num_splits, cb + 1) - sload(a.num_splits, cb));
      if (nsplit == 1) {
        const int64_t orow = (int64_t)cb * a.rows + row;
        if constexpr (!FUSED) {
          if (row_ok) {
            uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + orow * kDv;
#pragma unroll
            for (int mt = 0; mt < 16; ++mt)
#pragma unroll
              for (int qd = 0; qd < 4; ++qd) {
                const int d = 32 * mt + 8 * qd + 4 * half;
                const __bf16 v0 = (__bf16)(o[mt][4 * qd] * inv), v1 = (__bf16)(o[mt][4 * qd + 1] * inv);
                const __bf16 v2 = (__bf16)(o[mt][4 * qd + 2] * inv), v3 = (__bf16)(o[mt][4 * qd + 3] * inv);
                uint2 pk;
                pk.x = (uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
                pk.y = (uint32_t)__builtin_bit_cast(uint16_t, v2) | ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
                *reinterpret_cast<uint2*>(op + d) = pk;
              }
            if (half == 0) a.lse[orow] = lse2 * kLn2;
          }
        } else {
          // conjugate RoPE on dims 448..511 (d-tiles 14, 15), amax over the
          // row, e4m3 cast.  Tile by tile from the accumulators: only the 32
          // rotated values are held in VGPRs (scaling all of O at once would
          // move the 256 accumulators into VGPRs).  amax(O/l) = amax(O)/l
          // exactly, since scaling by a positive constant keeps the order.
          const double pos = (double)Lb - (double)a.s_q + (double)tok;
          const RopeRow rr = rope_row(pos, row_ok, a.rope_inv_freq, -1.0f);
          float rot[2][16];
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd)
#pragma unroll
              for (int pp = 0; pp < 2; ++pp) {
                const int k0 = 16 * t + 4 * qd + pp;  // RoPE pair (d - 448) / 2 = k0 + 2 * half
                float cs, sn;
                rope_pair(rr, a.rope_inv_freq, -1.0f, k0, k0 + 2, half, cs, sn);
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
          if (row_ok) {
            uint8_t* op = reinterpret_cast<uint8_t*>(a.out) + orow * kDv;
            auto put = [&](int mt, int qd, float v0, float v1, float v2, float v3) {
              const int d = 32 * mt + 8 * qd + 4 * half;
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
            if (half == 0) {
              a.lse[orow] = lse2 * kLn2;
              a.out_scale[orow] = sc;
            }
          }
        }
      } else {
        // partial of split `split_k` of sequence cb, row group g: O/l rounded
        // to bf16, stored in register order [wave][d-tile][quad pair][lane][8]
        // (coherent stores: the in-kernel combine may read them from another XCD)
        const int64_t pidx = (int64_t)uni(sload(a.num_splits, cb) + split_k) * a.groups + g;
        const __amdgpu_buffer_rsrc_t prs = buf_rsrc(uni_ptr(a.part_o + pidx * kPartialOElems), kPartialOElems * 2);
        const int vbase = (wave * (16 * 2 * 64 * 8) + lane * 8) * 2;
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
            __builtin_amdgcn_raw_buffer_store_b128(w, prs, vbase + (mt * 2 + q2) * 64 * 8 * 2, 0, kCoherent);
          }
        if (half == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse2 * kLn2),
                                                buf_rsrc(uni_ptr(a.part_lse + pidx * kPartialLseFloats), kPartialLseFloats * 4),
                                                (wave * 32 + r32) * 4, 0, kCoherent);
        if (!FUSED && a.ctl) {
          // every wave's stores completed (and are visible device-wide);
          // then the piece counts itself in
          wait_vmcnt<0>();
          __syncthreads();
          if (tid == 0) __hip_atomic_fetch_add(&a.ctl[3 + a.batch + 2 * cb + g], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    // next piece: first item of the following sequence
    cb = uni(cb + 1);
    cj = 0;
    split_k = 0;
  }
  wait_vmcnt<0>();  // no tile load (zeros past the end) outlives the workgroup's LDS
  // (the fused decode merges in a separate launch: its main loop has no
  // registers to spare for the merge code)
  if constexpr (!FUSED) {
    if (a.ctl) combine_phase<FUSED>(a, smem);
  }
}

// ---------------------------------------------------------------------------
// LSE combine of the 32 rows wt*32.. of row group g of sequence b: wave
// `sub` (lanes `lane`) merges d-tiles 4*sub .. 4*sub+3; thread (sub, lane)
// holds lane's row and 16 of the 64 (d-tile, quad) float4s.  Plain output
// needs one wave per sub; fused output needs all four subs of the rows in
// one workgroup (amax_s: 1 KB of LDS for the row amax across them).
// ---------------------------------------------------------------------------
template <bool FUSED, bool COHERENT>
__device__ void combine_rows(const DecodeArgs& a, int b, int g, int wt, int sub, int lane,
                             float (*amax_s)[64]) {
  const int s0 = a.num_splits[b], ns = a.num_splits[b + 1] - s0;
  if (ns <= 1) return;
  const int half = lane >> 5, r32 = lane & 31;
  const int row = g * kRowsPerWg + wt * 32 + r32;
  const bool row_ok = row < a.rows;

  // this lane's LSE of split s: lsep[s * lstride]
  const int64_t lstride = (int64_t)a.groups * kPartialLseFloats;
  const float* lsep = a.part_lse + (int64_t)s0 * lstride + (int64_t)g * kPartialLseFloats + wt * 32 + r32;
  // COHERENT (in-kernel combine): partials read past L1 and L2, as stored
  auto lse_of = [&](int s) -> float {
    if constexpr (COHERENT)
      return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          buf_rsrc(uni_ptr(a.part_lse + ((int64_t)(s0 + s) * a.groups + g) * kPartialLseFloats), kPartialLseFloats * 4),
          (wt * 32 + r32) * 4, 0, kCoherent));
    else
      return lsep[s * lstride];
  };
  auto load_split = [&](int s, uint4 (&v)[8]) {
    if constexpr (COHERENT) {
      const __amdgpu_buffer_rsrc_t rs = buf_rsrc(
          uni_ptr(a.part_o + ((int64_t)(s0 + s) * a.groups + g) * kPartialOElems), kPartialOElems * 2);
      const int vb = (wt * (16 * 2 * 64 * 8) + ((sub * 8) * 64 + lane) * 8) * 2;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rs, vb + k * 64 * 8 * 2, 0, kCoherent);
        v[k] = make_uint4(t[0], t[1], t[2], t[3]);
      }
    } else {
      const uint16_t* pb = a.part_o + ((int64_t)(s0 + s) * a.groups + g) * kPartialOElems +
                           (size_t)wt * (16 * 2 * 64 * 8) + (size_t)((sub * 8) * 64 + lane) * 8;
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const uint4*>(pb + k * 64 * 8);
    }
  };
  // LSE = log sum_s exp(lse_s): running max and rescaled sum, eight splits'
  // loads in flight at a time
  // The first eight splits' LSEs and the first four splits' partials are
  // loaded together (one round trip for the common case ns <= 4).
  float l8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) l8[i] = i < ns ? lse_of(i) : -INFINITY;
  uint4 v[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (j < ns) load_split(j, v[j]);
  float m = -INFINITY, tot = 0.f;
  for (int s = 0; s < ns; s += 8) {
    float l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) l[i] = s == 0 ? l8[i] : (s + i < ns ? lse_of(s + i) : -INFINITY);
    float mc = m;
#pragma unroll
    for (int i = 0; i < 8; ++i) mc = fmaxf(mc, l[i]);
    if (mc != -INFINITY) {
      float t = m == -INFINITY ? 0.f : tot * expf(m - mc);
#pragma unroll
      for (int i = 0; i < 8; ++i) t += l[i] == -INFINITY ? 0.f : expf(l[i] - mc);
      tot = t;
      m = mc;
    }
  }
  const float lse = m == -INFINITY ? -INFINITY : m + logf(tot);
  // thread (sub, lane) owns d-tiles 4*sub .. 4*sub+3 of its row: acc[4*i + qd]
  // holds quad qd of d-tile 4*sub + i (8 stored quad pairs)
  f32x4 acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = f32x4{};
  // O = sum_s exp(lse_s - LSE) O_s, four splits' partials in flight at a
  // time (a split without keys for the row has lse_s = -inf and weight 0)
  auto add_split = [&](const uint4 (&v)[8], float w) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t u[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
      // load k = (d-tile 4*sub + k/2, quad pair k%2); u[e] holds elements
      // 2e, 2e+1 of the pair, i.e. quad 2*(k%2) + e/2, lanes (2e)%4, (2e+1)%4
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f32x4& t = acc[4 * (k >> 1) + 2 * (k & 1) + (e >> 1)];
        t[(2 * e) & 3] += w * __uint_as_float(u[e] << 16);
        t[(2 * e + 1) & 3] += w * __uint_as_float(u[e] & 0xffff0000u);
      }
    }
  };
  auto weight = [&](float l) { return l == -INFINITY ? 0.f : expf(l - lse); };
  if (m != -INFINITY) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < ns) add_split(v[j], weight(l8[j]));
    for (int s = 4; s < ns; s += 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (s + j < ns) load_split(s + j, v[j]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (s + j < ns) add_split(v[j], weight(s + j < 8 ? l8[s + j] : lse_of(s + j)));
    }
  }
  const int64_t orow = (int64_t)b * a.rows + row;
  if constexpr (!FUSED) {
    if (row_ok) {
      uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + orow * kDv;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int e = sub * 16 + k, mt = e >> 2, qd = e & 3;
        const int d = 32 * mt + 8 * qd + 4 * half;
        uint2 pk;
        pk.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[k][0]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[k][1]) << 16);
        pk.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[k][2]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[k][3]) << 16);
        *reinterpret_cast<uint2*>(op + d) = pk;
      }
      if (half == 0 && sub == 0) a.lse[orow] = lse;
    }
  } else {
    // conjugate RoPE on dims 448..511 (sub 3 holds d-tiles 12..15)
    const int Lb = a.seqlens[b];
    const int tok = row_ok ? row / a.h_q : 0;
    const double pos = (double)Lb - (double)a.s_q + (double)tok;
    const RopeRow rr = rope_row(pos, row_ok, a.rope_inv_freq, -1.0f);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int e = sub * 16 + k, mt = e >> 2, qd = e & 3;
      if (mt < 14) continue;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int k0 = 16 * (mt - 14) + 4 * qd + pp;  // RoPE pair (d - 448) / 2 = k0 + 2 * half
        float cs, sn;
        rope_pair(rr, a.rope_inv_freq, -1.0f, k0, k0 + 2, half, cs, sn);
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
      if (half == 0 && sub == 0) {
        a.lse[orow] = lse;
        a.out_scale[orow] = sc;
      }
    }
  }
}

// The combine as its own launch, per (sequence, row group, 32-row tile).
// Plain output: the tile's four d-tile quarters go to two workgroups of two
// waves each (twice the workgroups in flight on a streaming kernel).  Fused:
// one workgroup of four waves, which share the row amax.
template <bool FUSED>
__global__ void __launch_bounds__(FUSED ? 256 : 128) k_combine(DecodeArgs a) {
  __shared__ float amax_s[4][64];
  if constexpr (FUSED) {
    const int wt = blockIdx.x & 3;
    const int g = (blockIdx.x >> 2) % a.groups;
    const int b = (blockIdx.x >> 2) / a.groups;
    combine_rows<FUSED, false>(a, b, g, wt, threadIdx.x >> 6, threadIdx.x & 63, amax_s);
  } else {
    const int u = blockIdx.x >> 1;
    const int wt = u & 3;
    const int g = (u >> 2) % a.groups;
    const int b = (u >> 2) / a.groups;
    combine_rows<FUSED, false>(a, b, g, wt, 2 * (blockIdx.x & 1) + (threadIdx.x >> 6), threadIdx.x & 63,
                               amax_s);
  }
}

// ---------------------------------------------------------------------------
// In-kernel combine (decode launched cooperatively, so every workgroup is
// resident; plain output only).  Each split piece, once its partial is
// stored (coherently) and complete, counts itself in arrived[b][g].  A wave
// out of decode work claims combine tasks (b, g, 32-row tile, d-quarter) in
// sequence order from one counter, 16 per (b, g) -- as many as the waves of
// the launch for 64 split sequences, so a task seldom waits for a claimer --
// and waits until every piece of (b, g) has arrived.  The last of the 16
// tasks of (b, g) clears its counters and the last claim clears the claim
// counter, so the metadata is ready for the next decode call.  The wait is
// bounded in time: past it the task is skipped and an error word is set.
// Control area ctl (after the split prefix, written by the scheduler):
//   [0] tasks T   [1] claim counter   [2] error word
//   [3 .. 3+B) split sequences in order   then arrived[B][2], done[B][2]
// ---------------------------------------------------------------------------
constexpr int kCombineTasksPerGroup = 16;
template <bool FUSED>
__device__ void combine_phase(const DecodeArgs& a, uint8_t* /*lds*/) {
  static_assert(!FUSED, "the fused output merges in its own launch");
  int32_t* ctl = a.ctl;
  const int B = a.batch, G = a.groups;
  int32_t* list = ctl + 3;
  int32_t* arrived = ctl + 3 + B;
  int32_t* done = arrived + 2 * B;
  const int lane = fresh_lane();
  const int T = uni(ctl[0]);
  const int claimers = (int)gridDim.x * kWaves;
  for (;;) {
    int t = 0;
    if (lane == 0) t = atomicAdd(&ctl[1], 1);
    t = uni(t);
    if (t >= T) {
      if (lane == 0 && t == T + claimers - 1)
        __hip_atomic_store(&ctl[1], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    const int i = t / (kCombineTasksPerGroup * G), g = (t / kCombineTasksPerGroup) % G;
    const int wt = (t >> 2) & 3, sub = t & 3;
    const int b = uni(list[i]);
    const int ns = uni(a.num_splits[b + 1] - a.num_splits[b]);
    int ok = 1;
    if (lane == 0) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__hip_atomic_load(&arrived[2 * b + g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < ns) {
        __builtin_amdgcn_s_sleep(32);  // ~2k cycles between polls: a thousand waiting waves stay light on memory
        if (__builtin_amdgcn_s_memrealtime() - t0 > 100000000ull) {  // 1 s at 100 MHz
          ok = 0;
          __hip_atomic_store(&ctl[2], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    if (uni(ok)) combine_rows<false, true>(a, b, g, wt, sub, lane, nullptr);
    wait_vmcnt<0>();  // this task's output is written before it counts as done
    if (lane == 0 && atomicAdd(&done[2 * b + g], 1) == kCombineTasksPerGroup - 1) {
      __hip_atomic_store(&arrived[2 * b + g], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&done[2 * b + g], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// Debug gather: stage both halves of one work item with the decode kernel's
// loaders (and dequantiser), copy them out un-swizzled as [64][576] bf16.
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
      if constexpr (KVF == kKvBf16) load_half_bf16_sparse(tile, a.kv, ids, nvalid, wave, lane);
      else load_half_fp8_sparse(raw, a.kv, ids, nvalid, wave, lane);
    } else {
      const int L = a.seqlens[b];
      const bool any = j * kPage < L;
      const int64_t phys = any ? a.block_table[(int64_t)b * a.max_blocks + j] : 0;
      const int valid = any ? min(kPage, L - j * kPage) : 0;
      if constexpr (KVF == kKvBf16) load_half_bf16_dense(tile, a.kv, phys, valid, h, wave, lane);
      else load_half_fp8_dense(raw, a.kv, phys, valid, h, wave, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if constexpr (KVF != kKvBf16) {
      dequant_half_scaled(tile, raw, tid);
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
hipError_t launch_sched(const int32_t* seqlens, int batch, int rows, int topk, int num_slots,
                        int32_t* meta, int32_t* num_splits, hipStream_t stream) {
  if (batch <= kSchedSmallBatch)
    hipLaunchKernelGGL((k_sched<256, kSchedSmallBatch>), dim3(1), dim3(256), 0, stream, seqlens, batch, rows,
                       topk, num_slots, meta, num_splits);
  else
    hipLaunchKernelGGL((k_sched<1024, kMaxBatch>), dim3(1), dim3(1024), 0, stream, seqlens, batch, rows,
                       topk, num_slots, meta, num_splits);
  return hipGetLastError();
}

template <int KVF, bool SPARSE, bool FUSED>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream, hipEvent_t start,
                                  hipEvent_t stop) {
  const int grid = a.num_slots * a.groups;
  if (a.ctl) {
    // every workgroup must be resident: the combine tasks wait on other
    // workgroups' pieces
    if (start) {
      const hipError_t e = hipEventRecord(start, stream);
      if (e != hipSuccess) return e;
    }
    DecodeArgs ac = a;
    void* args[] = {&ac};
    const hipError_t e = hipLaunchCooperativeKernel((const void*)k_decode<KVF, SPARSE, FUSED>, dim3(grid),
                                                    dim3(kThreads), args, 0, stream);
    if (e != hipSuccess) {
      (void)hipGetLastError();  // clear it: the caller falls back to the separate combine
      return e;
    }
    return stop ? hipEventRecord(stop, stream) : hipSuccess;
  }
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
  if (fused) hipLaunchKernelGGL(k_combine<true>, dim3(grid), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(k_combine<false>, dim3(2 * grid), dim3(128), 0, stream, a);
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

}  // namespace mla
