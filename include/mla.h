/*
 * mla.h -- C ABI of libmla.so: paged Multi-head Latent Attention decoding
 * on AMD Instinct MI355X (gfx950).
 *
 * The operation.  For every sequence b, query token t and head h, one query
 * row of d_qk = 576 dims (512 latent + 64 decoupled-RoPE dims) attends to a
 * single shared latent KV head stored in a paged cache of 64-token blocks;
 * V is the first d_v = 512 dims of K.  The result is the softmax-weighted
 * sum O (d_v dims) and the log-sum-exp of the scaled scores.
 *   - "FlashMLA" (AI Wiki), section "How is FlashMLA designed?": fused,
 *     tiled attention with an online softmax over KV streamed through
 *     on-chip memory; a paged KV cache of fixed-size blocks (64 tokens,
 *     section "What is FlashMLA?") and variable-length sequences.
 *   - "FlashMLA" Ampere-adaptation README (gitlite), section "Usage": a
 *     scheduling-metadata call made once per decoding step, taking
 *     cache_seqlens, s_q*h_q/h_kv and h_kv, whose results feed every
 *     per-layer decode call; the decode call takes q, the paged cache,
 *     block_table, cache_seqlens, dv, the metadata and a causal flag and
 *     returns (o, lse).
 *   - "FlashMLA" (AI Wiki), section "Interfaces": sparse decoding takes an
 *     indices tensor (batch, s_q, topk) whose entries encode the page block
 *     and the offset (here: flat token id = block*64 + offset), -1 marking
 *     an invalid entry, with block_table then ignored.
 *   - Same page, section "The FP8 and FP4 KV cache": the V3.2 token record,
 *     512 e4m3 values + four fp32 scales (one per 128 dims) + 64 bf16 RoPE
 *     values, 656 bytes, data before scales.
 *   - "FlashMLA fused norm-RoPE-attention-RoPE-cast kernel" card, section
 *     "Arithmetic intensity": optional Q-RMSNorm and Q-RoPE before
 *     attention and conjugate O-RoPE plus an FP8 cast after it, fused.
 *
 * Conventions.  Every pointer is DEVICE memory unless marked [host].  All
 * calls that take a `stream` (a hipStream_t; NULL = the null stream) are
 * asynchronous on it and never synchronise the host.  The caller allocates
 * and owns every buffer, including metadata and workspace; the library
 * keeps only a per-device cache of device properties.  Validation reads
 * scalar arguments only (never device memory).  Errors are returned, never
 * thrown; mla_last_error() gives a thread-local message for the last
 * non-OK status.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad alignment, bad struct_size */
  MLA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (shape outside the supported set) */
  MLA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than mla_workspace_bytes()   */
  MLA_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed                */
} mla_status;

typedef enum {
  MLA_KV_BF16 = 0,     /* [num_blocks][64][576] bf16, 1152 B per token                  */
  MLA_KV_FP8_V32 = 1,  /* [num_blocks][64][656] bytes: 512 e4m3 | 4 fp32 LE | 64 bf16    */
  /* [num_blocks][64][528] bytes: 512 e4m3 codes of all dims, then 16 e8m0
   * scales, scale j (value 2^(e-127); 0xFF is NaN) for dims 32j..32j+31.  The
   * head dim of this format is 512 (AI Wiki, The FP8 and FP4 KV cache, the
   * V4.1 row): d_qk = d_v = 512, V = K, q is [b][s_q][h_q][512].  Sparse
   * (indices) and unfused only. */
  MLA_KV_FP8_V41 = 2
} mla_kv_format;

#define MLA_PAGE_SIZE 64
#define MLA_D_QK 576
#define MLA_D_QK_V41 512
#define MLA_D_V 512
#define MLA_MAX_BATCH 16384
/* Piece cost (in 64-key items) that suits the fused decode, whose query
 * prologue (RMSNorm, RoPE, q-hat) costs about four items: mla_get_metadata's
 * piece_cost for metadata that fused decode calls will use. */
#define MLA_PIECE_COST_FUSED 4
#define MLA_MAX_PIECE_COST 64

/* [host] Number of scheduler slots S to use on `device` for decode calls
 * with `rows_per_kv_head` = s_q*h_q/h_kv query rows: one slot per compute
 * unit per 128-row group.  Returns a value >= 1, or 0 on error. */
int32_t mla_num_sched_slots(int32_t device, int32_t rows_per_kv_head);

/* [host] int32 element counts of the two metadata arrays. */
size_t mla_sched_meta_ints(int32_t num_slots);  /* = 8 * num_slots  */
size_t mla_num_splits_ints(int32_t batch);      /* = batch + 1      */

/* Split-KV scheduling metadata (once per decoding step; reusable by every
 * decode call with the same cache_seqlens contents, rows and topk).
 *   cache_seqlens     int32 [batch], each >= 0 (read on the device)
 *   rows_per_kv_head  s_q*h_q/h_kv (>= 1)
 *   h_kv              must be 1
 *   topk              0 = dense; > 0: sparse with topk indices per query row
 *   num_slots         S, normally mla_num_sched_slots()
 *   piece_cost        F below, in 64-key items: 0 = the default
 *                     max(1, ceil(min(rows,128)/64)) (about two for 128 rows,
 *                     a plain piece's query load, pipeline fill and
 *                     finalize), else 1..MLA_MAX_PIECE_COST
 *                     (MLA_PIECE_COST_FUSED for the fused decode)
 *   sched_meta        int32 [S][8] out: per slot {b0, j0, b1, j1_end, k0, items, 0, 0}
 *   num_splits        int32 [mla_num_splits_ints(batch)] out: [0..batch] prefix
 *                     offsets of per-sequence splits (sequence b has
 *                     num_splits[b+1] - num_splits[b] of them)
 * The split rule: a sequence has n_b = ceil(len/64) work items (ceil(topk/64)
 * when sparse; an empty sequence keeps one item with no KV); with F the
 * piece cost (a piece's fixed cost in items), the items are laid on a line
 * where
 * sequence b starts at U_b = sum_{b'<b}(F + n_b') and its item j sits at
 * U_b + F + j; with cap = ceil((U_batch+1)/S), slot s takes the items at
 * positions [s*cap, (s+1)*cap).  A small total (U_batch < S) thus gives
 * every item a slot of its own, so even one sequence spreads over the
 * machine.  Errors: INVALID_ARG for null pointers, bad sizes or a piece
 * cost outside [0, MLA_MAX_PIECE_COST],
 * UNSUPPORTED for h_kv != 1 or batch > MLA_MAX_BATCH. */
mla_status mla_get_metadata(const int32_t* cache_seqlens, int32_t batch,
                            int32_t rows_per_kv_head, int32_t h_kv, int32_t topk,
                            int32_t num_slots, int32_t piece_cost, int32_t* sched_meta,
                            int32_t* num_splits, void* stream);

/* [host] Workspace bytes a decode call needs: split partials, O in bf16
 * (128 rows x 512 per row group) and LSE in fp32 (128 per row group). */
size_t mla_workspace_bytes(int32_t batch, int32_t s_q, int32_t h_q, int32_t num_slots);

typedef struct mla_decode_params {
  uint32_t struct_size;        /* sizeof(mla_decode_params)                                */
  int32_t batch, s_q, h_q, h_kv, d_qk, d_v;  /* h_kv == 1, d_qk == 576, d_v == 512          */
  const void* q;               /* bf16 [batch][s_q][h_q][576], 16-byte aligned              */
  const void* kv;              /* paged cache, format below, 16-byte aligned                */
  int32_t kv_format;           /* mla_kv_format                                            */
  int32_t page_size;           /* must be 64                                               */
  int64_t num_blocks;          /* blocks in the pool                                       */
  const int32_t* block_table;  /* int32 [batch][max_blocks_per_seq]; may be NULL if sparse  */
  int32_t max_blocks_per_seq;
  const int32_t* cache_seqlens;/* int32 [batch]                                            */
  float softmax_scale;         /* applied to q.K (typically 576^-0.5); positive and finite */
  int32_t causal;              /* bottom-right aligned: token t sees keys j <= len-s_q+t    */
  const int32_t* indices;      /* NULL = dense; else int32 [batch][s_q][topk] flat token ids, -1 = masked */
  int32_t topk;
  const int32_t* sched_meta;   /* from mla_get_metadata with the same rows and topk         */
  const int32_t* num_splits;   /* from mla_get_metadata; read only                        */
  int32_t num_slots;
  void* workspace;             /* >= mla_workspace_bytes(), 256-byte aligned                */
  size_t workspace_bytes;
  void* out;                   /* bf16 [batch][s_q][h_q][512]; fused: e4m3 bytes, same shape */
  float* lse;                  /* fp32 [batch][s_q][h_q], natural log of sum exp(scaled scores); -inf for an empty row */
  int32_t fused;               /* 1 = RMSNorm+RoPE on q, conjugate RoPE + FP8 cast on O      */
  const void* norm_weight;     /* fused: bf16 [576]                                        */
  float norm_eps;              /* fused: RMSNorm epsilon                                   */
  float rope_base;             /* fused: RoPE base (positions are len - s_q + t)           */
  float* out_scale;            /* fused: fp32 [batch][s_q][h_q], O = codes * scale          */
  uint32_t flags;              /* MLA_FLAG_* bits; 0 = decode and merge in one call         */
} mla_decode_params;

/* mla_decode leaves split partials in the workspace for a later
 * mla_combine call on the same stream (e.g. to time or overlap it).  Any
 * other flag bit is rejected (MLA_ERR_INVALID_ARG). */
#define MLA_FLAG_DEFER_COMBINE 1u

/* Paged MLA decode: O and LSE for every query row (see the file comment).
 * A row that sees no key gets O = 0 and LSE = -inf.  Sequences whose work
 * the schedule splits write partials (O in bf16, LSE in fp32) to the
 * workspace and a combine launch merges them by LSE; others write their
 * output directly.  The metadata is read only, so any number of decode calls
 * (one per layer) may reuse it; calls that share a workspace must be ordered
 * on one stream.
 * Supported: h_kv = 1, d_qk = 576 (512 with MLA_KV_FP8_V41), d_v = 512,
 * page 64, s_q*h_q <= 65536;
 * sparse needs causal = 0 and (s_q == 1 or h_q % 128 == 0); MLA_KV_FP8_V32
 * works paged or sparse, fused or not; MLA_KV_FP8_V41 needs indices and
 * fused = 0; fused needs s_q*h_q of whole heads as above.
 * batch = 0 is a no-op that launches nothing; q, kv, block_table,
 * cache_seqlens, out and lse may then be NULL (sched_meta, num_splits and
 * the workspace may not).
 * Pool bounds: nothing outside the pool [0, num_blocks) is ever read.  A
 * sparse id outside [0, num_blocks*64) is masked like -1.  A block_table
 * entry outside [0, num_blocks) names no page: its 64 positions stay
 * visible and read as all-zero keys (score 0), and so do positions past
 * max_blocks_per_seq pages.  Entries past ceil(len/64) are never read.
 * 16-bit arithmetic: the fused path and every decode over a V3.2 FP8 cache
 * run both products on fp16 operands.  Fused: q-hat is rounded once to
 * fp16, bf16 KV converts exactly.  V3.2 FP8: each key value is
 * fp16(fp32(code) * fp32 scale), rounded once; q converts exactly.  These
 * paths need |q|, |q-hat| and |K| below 65504; magnitudes under 2^-14
 * keep 2^-24 absolute resolution.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP (launch failure). */
mla_status mla_decode(const mla_decode_params* params, void* stream);

/* Measurement hook: mla_decode whose decode-kernel launch also records
 * `start_event` and `stop_event` (hipEvent_t created with timing enabled;
 * either may be NULL) at the kernel's own start and end on the stream, so
 * hipEventElapsedTime gives the kernel's execution time without the gaps
 * that events recorded around the launch add.  Same arguments and errors as
 * mla_decode. */
mla_status mla_decode_timed(const mla_decode_params* params, void* stream, void* start_event,
                            void* stop_event);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): mla_decode without a
 * workspace.  The split partials go to a static device array of
 * MLA_NOALLOC_SCRATCH_BYTES per GPU (allocated with the library's code
 * object on each device it runs on, held until the process ends); its
 * device address is looked up on the first call on a device, which must be
 * the current device.  params->workspace and workspace_bytes are ignored;
 * flags must be 0 (decode and merge in one call).  Every call on a GPU
 * shares that GPU's array, so calls that overlap on one GPU (on different
 * streams, or from several threads without ordering) race; calls ordered on
 * one stream do not.  Nothing in the array needs to start at zero: the
 * combine reads only partials the decode launch of the same call wrote.
 * Calls no hipMalloc, hipFree or allocating routine.  Errors as mla_decode;
 * MLA_ERR_WORKSPACE when mla_workspace_bytes() for the call exceeds
 * MLA_NOALLOC_SCRATCH_BYTES. */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
mla_status mla_decode_noalloc(const mla_decode_params* params, void* stream);

/* The LSE merge of split partials ("FlashMLA" Ampere-adaptation README,
 * section "Usage": the decode returns (o, lse) over the whole KV length).
 * For every sequence the schedule split, every row: lse = ln sum_s e^{lse_s},
 * O = sum_s e^{lse_s - lse} O_s (splits in ascending order; -inf partials
 * weigh 0), then the bf16 (or fused FP8) output and LSE are written.  Only
 * needed after mla_decode with MLA_FLAG_DEFER_COMBINE; same params, same
 * stream.  Errors as mla_decode. */
mla_status mla_combine(const mla_decode_params* params, void* stream);

/* Test hook: the 64 x 576 tile of 16-bit values the KV loader stages for
 * work item j of sequence b (query token t when sparse), written
 * un-swizzled to dst [64][576]: the bf16 rows of a bf16 cache; for a V3.2
 * FP8 cache the fp16 rows both products read, fp16(fp32(code) * fp32
 * scale) for dims < 512 and the bf16 RoPE dims in fp16; zero rows past the
 * sequence or for -1 indices.  Not available for MLA_KV_FP8_V41
 * (MLA_ERR_UNSUPPORTED). */
mla_status mla_debug_gather(const mla_decode_params* params, int32_t b, int32_t t, int32_t j,
                            void* dst, void* stream);

const char* mla_status_string(mla_status s);
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H_ */
