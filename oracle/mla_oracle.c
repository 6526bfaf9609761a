/*
 * mla_oracle.c -- the CPU oracle for paged MLA decoding.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library.  It
 * shares no code, header, table or constant generator with the HIP kernels
 * and includes nothing from them.
 *
 * Everything is computed in IEEE double precision with plain loops, in the
 * order the method is defined, with no blocking, no online softmax and no
 * fusion.  Built without -ffast-math.
 *
 * What it computes (sources are the pages' titles and sections):
 *  - "FlashMLA" (AI Wiki), section "How is FlashMLA designed?": attention
 *    over keys streamed from a paged cache is ordinary softmax attention;
 *    the tiled/online formulation only reorders it.  So the oracle is the
 *    definition: s_j = scale * <q, K_j>, LSE = max + ln sum exp(s - max),
 *    O = sum_j softmax_j * V_j.
 *  - Same page, sections "How is FlashMLA designed?" and "What is
 *    FlashMLA?" (day-one release): a paged KV cache with fixed blocks of 64
 *    tokens and per-sequence lengths.
 *  - "FlashMLA" Ampere-adaptation README (gitlite), section "Usage": the
 *    decode call takes q, the paged cache, block_table, cache_seqlens, dv
 *    and a causal flag and returns (o, lse); V is the first dv dims of K.
 *  - "FlashMLA" (AI Wiki), section "Interfaces": sparse decoding takes
 *    indices of shape (batch, s_q, topk) whose entries already hold the
 *    page block and the offset; -1 marks an invalid entry; block_table is
 *    then ignored.
 *  - Same page, section "The FP8 and FP4 KV cache": the V3.2 record is 512
 *    float8_e4m3 values with one float32 scale per 128 values, then 64 RoPE
 *    values kept in bfloat16, 656 bytes per token, data before scales.
 *  - "FlashMLA fused norm-RoPE-attention-RoPE-cast kernel" (inference-
 *    research card), section "Arithmetic intensity": the fused kernel runs
 *    Q-norm, Q-RoPE, attention, conjugate O-RoPE and the cast to FP8 in
 *    that order without changing the attention arithmetic.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - LSE is the natural log of the sum of exp of the *scaled* scores.
 *  - Causal with s_q > 1 is bottom-right aligned: query token t of a
 *    sequence of length L sees keys j <= L - s_q + t.
 *  - A row with no visible key has O = 0 and LSE = -inf.
 *  - Sparse ids are flat token ids into the pool (block * 64 + offset);
 *    duplicates count as separate keys; -1 entries are skipped, and so is
 *    any id outside the pool [0, num_blocks * 64).
 *  - A block_table entry outside [0, num_blocks) names no page: its 64
 *    positions read as all-zero keys (they stay visible, as positions);
 *    so do positions past max_blocks_per_seq pages, which have no entry.
 *  - e4m3 is OCP E4M3FN (bias 7, no infinities, S.1111.111 is NaN, max
 *    448); encoding rounds to nearest, ties to even, saturating to +-448.
 *  - RMSNorm runs over all 576 dims of a head with a 576-entry weight;
 *    RoPE rotates adjacent pairs (512+2i, 513+2i) of q by pos*base^(-2i/64)
 *    with pos = L - s_q + t; the conjugate rotation uses -theta on O's
 *    pairs (448+2i, 449+2i); the FP8 cast uses scale = amax/448 (1 if amax
 *    is 0) over the 512 dims of the post-RoPE fp64 O.
 *  - The split-KV schedule follows the written rule in orc_sched_plan.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_PAGE 64
#define ORC_FP8_TOKEN_BYTES 656
#define ORC_FP8V41_TOKEN_BYTES 528

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* bfloat16 is the top half of an IEEE binary32; widening is exact. */
double orc_bf16_to_f64(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP E4M3FN decode from the bit fields: sign, 4-bit exponent (bias 7),
 * 3-bit mantissa; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN. */
double orc_e4m3_decode(uint8_t code) {
  int s = (code >> 7) & 1;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* OCP E8M0 (a scale): an 8-bit biased exponent, value 2^(e - 127); the
 * all-ones code is NaN.  No sign, no mantissa. */
double orc_e8m0_decode(uint8_t code) {
  if (code == 0xFF) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/* OCP E4M3FN encode: round to nearest, ties to even mantissa, finite
 * overflow and infinities saturate to +-448, NaN maps to 0x7F/0xFF. */
uint8_t orc_e4m3_encode_rne(double x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs(x);
  if (isnan(x)) return (uint8_t)(sign | 0x7F);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  if (a < ldexp(1.0, -6)) {
    /* subnormal range, quantum 2^-9; q == 8 is the smallest normal 0x08 */
    double q = nearbyint(a / ldexp(1.0, -9)); /* default mode: ties to even */
    return (uint8_t)(sign | (uint8_t)q);
  }
  int e2;
  (void)frexp(a, &e2);        /* a = f * 2^e2, f in [0.5, 1) */
  int e = e2 - 1;              /* a in [2^e, 2^(e+1)) */
  double q = nearbyint(a / ldexp(1.0, e - 3)); /* in [8, 16] */
  if (q >= 16.0) { e += 1; q = 8.0; }
  int code = ((e + 7) << 3) | ((int)q - 8);
  if (code > 0x7E) code = 0x7E; /* only reachable at a >= 464, handled above */
  return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------ */
/* Problem description                                                 */
/* ------------------------------------------------------------------ */

typedef struct {
  int32_t batch, s_q, h_q, d_qk, d_v;
  int32_t kv_format;       /* 0: bf16 [nblk][64][d_qk]; 1: V3.2 fp8 [nblk][64][656];
                              2: V4.1 fp8 [nblk][64][528] (d_qk = 512) */
  int64_t num_blocks;
  const uint16_t* q;       /* bf16 bits [batch][s_q][h_q][d_qk] */
  const void* kv;
  const int32_t* block_table; /* [batch][max_blocks] (dense only) */
  int32_t max_blocks;
  const int32_t* seqlens;  /* [batch] */
  int32_t causal;
  const int32_t* indices;  /* [batch][s_q][topk] flat token ids, -1 invalid; NULL = dense */
  int32_t topk;
  double scale;            /* softmax scale applied to q.K */
  int32_t fused;           /* 1: RMSNorm + RoPE on q, conjugate RoPE + FP8 cast on O */
  const uint16_t* norm_w;  /* bf16 bits [d_qk] */
  double eps;
  double rope_base;
} orc_problem;

/* Fetch key vector (all d_qk dims) of flat token id `tok` as fp64; a token
 * outside the pool reads as the zero vector. */
static void fetch_token(const orc_problem* p, int64_t tok, double* k) {
  if (tok < 0 || tok >= p->num_blocks * ORC_PAGE) {
    for (int d = 0; d < p->d_qk; ++d) k[d] = 0.0;
    return;
  }
  if (p->kv_format == 0) {
    const uint16_t* src = (const uint16_t*)p->kv + tok * (int64_t)p->d_qk;
    for (int d = 0; d < p->d_qk; ++d) k[d] = orc_bf16_to_f64(src[d]);
  } else if (p->kv_format == 2) {
    /* V4.1 record (AI Wiki, The FP8 and FP4 KV cache): [0,512) e4m3 codes
     * of all 512 dims, then 16 e8m0 scales, scale j for dims 32j..32j+31. */
    const uint8_t* rec = (const uint8_t*)p->kv + tok * (int64_t)ORC_FP8V41_TOKEN_BYTES;
    for (int d = 0; d < 512; ++d) k[d] = orc_e4m3_decode(rec[d]) * orc_e8m0_decode(rec[512 + d / 32]);
  } else {
    /* V3.2 record: [0,512) e4m3 codes, [512,528) four little-endian fp32
     * tile scales (one per 128 dims), [528,656) 64 bf16 RoPE values. */
    const uint8_t* rec = (const uint8_t*)p->kv + tok * (int64_t)ORC_FP8_TOKEN_BYTES;
    float sc[4];
    memcpy(sc, rec + 512, sizeof sc);
    for (int d = 0; d < 512; ++d) k[d] = orc_e4m3_decode(rec[d]) * (double)sc[d / 128];
    for (int r = 0; r < 64; ++r) {
      uint16_t bits;
      memcpy(&bits, rec + 528 + 2 * r, 2);
      k[512 + r] = orc_bf16_to_f64(bits);
    }
  }
}

/* Flat token id of logical position j of sequence b (dense paging); -1
 * when the block_table entry names no page of the pool. */
static int64_t dense_token(const orc_problem* p, int b, int64_t j) {
  if (j / ORC_PAGE >= p->max_blocks) return -1; /* no block_table entry */
  int32_t blk = p->block_table[(int64_t)b * p->max_blocks + j / ORC_PAGE];
  if (blk < 0 || blk >= p->num_blocks) return -1;
  return (int64_t)blk * ORC_PAGE + (j % ORC_PAGE);
}

/* RMSNorm over all d dims: y = x * w / sqrt(mean(x^2) + eps). */
void orc_rmsnorm(const double* x, const double* w, int d, double eps, double* y) {
  double ss = 0.0;
  for (int i = 0; i < d; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / (double)d + eps);
  for (int i = 0; i < d; ++i) y[i] = x[i] * w[i] * inv;
}

/* Rotary embedding on `npairs` adjacent pairs starting at x[0]:
 * pair i = (x[2i], x[2i+1]) rotates by sign * pos * base^(-2i/(2*npairs)). */
void orc_rope(double* x, int npairs, double pos, double base, double sign) {
  for (int i = 0; i < npairs; ++i) {
    double theta = sign * pos * pow(base, -2.0 * (double)i / (double)(2 * npairs));
    double c = cos(theta), s = sin(theta);
    double a = x[2 * i], b = x[2 * i + 1];
    x[2 * i] = a * c - b * s;
    x[2 * i + 1] = a * s + b * c;
  }
}

/* Softmax attention of one query row over n explicit keys (each d_qk dims,
 * row-major).  V_j = K_j[0:d_v].  Empty key set: O = 0, LSE = -inf. */
void orc_attend(const double* q, int64_t n, const double* keys, int d_qk, int d_v,
                double scale, double* o, double* lse) {
  for (int e = 0; e < d_v; ++e) o[e] = 0.0;
  if (n == 0) { *lse = -INFINITY; return; }
  double* s = (double*)malloc(sizeof(double) * (size_t)n);
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j) {
    const double* k = keys + j * (int64_t)d_qk;
    double acc = 0.0;
    for (int d = 0; d < d_qk; ++d) acc += q[d] * k[d];
    s[j] = scale * acc;
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < n; ++j) l += exp(s[j] - m);
  for (int64_t j = 0; j < n; ++j) {
    double pj = exp(s[j] - m) / l;
    const double* k = keys + j * (int64_t)d_qk;
    for (int e = 0; e < d_v; ++e) o[e] += pj * k[e];
  }
  *lse = m + log(l);
  free(s);
}

/* Merge partial results of disjoint key sets by their LSEs:
 * lse = ln sum_s exp(lse_s); O = sum_s exp(lse_s - lse) O_s.
 * Parts with lse_s = -inf carry weight 0; if all are -inf the result is
 * O = 0, LSE = -inf. */
void orc_combine(int nparts, const double* lse_parts, const double* o_parts, int d_v,
                 double* o, double* lse) {
  double m = -INFINITY;
  for (int s = 0; s < nparts; ++s)
    if (lse_parts[s] > m) m = lse_parts[s];
  for (int e = 0; e < d_v; ++e) o[e] = 0.0;
  if (m == -INFINITY) { *lse = -INFINITY; return; }
  double tot = 0.0;
  for (int s = 0; s < nparts; ++s)
    if (lse_parts[s] != -INFINITY) tot += exp(lse_parts[s] - m);
  double L = m + log(tot);
  for (int s = 0; s < nparts; ++s) {
    if (lse_parts[s] == -INFINITY) continue;
    double w = exp(lse_parts[s] - L);
    for (int e = 0; e < d_v; ++e) o[e] += w * o_parts[(int64_t)s * d_v + e];
  }
  *lse = L;
}

/* Key list visible to query token t of sequence b, as flat token ids.
 * Returns the count; ids must hold room for the maximum count. */
static int64_t visible_tokens(const orc_problem* p, int b, int t, int64_t* ids) {
  int64_t n = 0;
  if (p->indices) {
    const int32_t* row = p->indices + ((int64_t)b * p->s_q + t) * p->topk;
    for (int k = 0; k < p->topk; ++k)
      if (row[k] >= 0 && row[k] < p->num_blocks * ORC_PAGE) ids[n++] = row[k];
    return n;
  }
  int64_t L = p->seqlens[b];
  int64_t last = p->causal ? (L - p->s_q + t) : (L - 1); /* inclusive */
  if (last > L - 1) last = L - 1;
  for (int64_t j = 0; j <= last; ++j) ids[n++] = dense_token(p, b, j);
  return n;
}

/* Query row (b, t, h) after the optional fused prologue, in fp64. */
static void query_row(const orc_problem* p, int b, int t, int h, double* q) {
  const uint16_t* src = p->q + (((int64_t)b * p->s_q + t) * p->h_q + h) * p->d_qk;
  for (int d = 0; d < p->d_qk; ++d) q[d] = orc_bf16_to_f64(src[d]);
  if (p->fused) {
    double w[1024], y[1024];
    for (int d = 0; d < p->d_qk; ++d) w[d] = orc_bf16_to_f64(p->norm_w[d]);
    orc_rmsnorm(q, w, p->d_qk, p->eps, y);
    for (int d = 0; d < p->d_qk; ++d) q[d] = y[d];
    double pos = (double)p->seqlens[b] - (double)p->s_q + (double)t;
    orc_rope(q + 512, (p->d_qk - 512) / 2, pos, p->rope_base, +1.0);
  }
}

/* Fused epilogue of one output row (query token t of sequence b): the
 * conjugate RoPE on the last 64 dims of o, then the per-row scale
 * amax/448 (1 for an all-zero row) and the e4m3 codes of o/scale. */
static void fused_epilogue(const orc_problem* p, int b, int t, double* orow, uint8_t* crow,
                           double* oscale) {
  double pos = (double)p->seqlens[b] - (double)p->s_q + (double)t;
  orc_rope(orow + (p->d_v - 64), 32, pos, p->rope_base, -1.0);
  double amax = 0.0;
  for (int e = 0; e < p->d_v; ++e)
    if (fabs(orow[e]) > amax) amax = fabs(orow[e]);
  double sc = amax > 0.0 ? amax / 448.0 : 1.0;
  *oscale = sc;
  for (int e = 0; e < p->d_v; ++e) crow[e] = orc_e4m3_encode_rne(orow[e] / sc);
}

/* Full decode.  o: [batch][s_q][h_q][d_v] fp64; lse: [batch][s_q][h_q].
 * In fused mode o holds the post-RoPE fp64 O, codes the e4m3 bytes
 * [batch][s_q][h_q][d_v] and oscale the per-row fp64 scale. */
int orc_decode(const orc_problem* p, double* o, double* lse, uint8_t* codes, double* oscale,
               int nthreads) {
  if (p->d_qk > 1024 || p->d_v > p->d_qk) return 1;
  if (p->fused && (p->d_v != 512 || p->d_qk != 576)) return 1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  for (int b = 0; b < p->batch; ++b) {
    for (int t = 0; t < p->s_q; ++t) {
      int64_t cap = p->indices ? p->topk : (p->seqlens[b] > 0 ? p->seqlens[b] : 0);
      int64_t* ids = (int64_t*)malloc(sizeof(int64_t) * (size_t)(cap > 0 ? cap : 1));
      int64_t n = visible_tokens(p, b, t, ids);
      double* keys = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * p->d_qk);
#pragma omp parallel for schedule(static)
      for (int64_t j = 0; j < n; ++j) fetch_token(p, ids[j], keys + j * p->d_qk);
#pragma omp parallel for schedule(dynamic, 1)
      for (int h = 0; h < p->h_q; ++h) {
        double q[1024];
        int64_t row = ((int64_t)b * p->s_q + t) * p->h_q + h;
        query_row(p, b, t, h, q);
        double* orow = o + row * p->d_v;
        orc_attend(q, n, keys, p->d_qk, p->d_v, p->scale, orow, &lse[row]);
        if (p->fused) fused_epilogue(p, b, t, orow, codes + row * p->d_v, &oscale[row]);
      }
      free(keys);
      free(ids);
    }
  }
  return 0;
}

/* One output row (b, t, h) over every key it sees, as orc_decode computes
 * it (fused epilogue included); for checking sampled rows of workloads too
 * large for a full oracle run. */
int orc_decode_row(const orc_problem* p, int b, int t, int h, double* o, double* lse, uint8_t* codes,
                   double* oscale) {
  if (p->d_qk > 1024 || p->d_v > p->d_qk) return 1;
  if (p->fused && (p->d_v != 512 || p->d_qk != 576)) return 1;
  int64_t cap = p->indices ? p->topk : (p->seqlens[b] > 0 ? p->seqlens[b] : 0);
  int64_t* ids = (int64_t*)malloc(sizeof(int64_t) * (size_t)(cap > 0 ? cap : 1));
  int64_t n = visible_tokens(p, b, t, ids);
  double* keys = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * p->d_qk);
  for (int64_t j = 0; j < n; ++j) fetch_token(p, ids[j], keys + j * p->d_qk);
  double q[1024];
  query_row(p, b, t, h, q);
  orc_attend(q, n, keys, p->d_qk, p->d_v, p->scale, o, lse);
  if (p->fused) fused_epilogue(p, b, t, o, codes, oscale);
  free(keys);
  free(ids);
  return 0;
}

/* One row over an explicit subset of its keys (split-mode self-check).
 * key_pos holds logical positions (dense) or flat token ids (sparse). */
int orc_decode_row_subset(const orc_problem* p, int b, int t, int h, int64_t n,
                          const int64_t* key_pos, double* o, double* lse) {
  double q[1024];
  double* keys = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * p->d_qk);
  for (int64_t j = 0; j < n; ++j) {
    int64_t tok = p->indices ? key_pos[j] : dense_token(p, b, key_pos[j]);
    fetch_token(p, tok, keys + j * p->d_qk);
  }
  query_row(p, b, t, h, q);
  orc_attend(q, n, keys, p->d_qk, p->d_v, p->scale, o, lse);
  free(keys);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Split-KV schedule (the written rule both sides implement)           */
/* ------------------------------------------------------------------ */
/*
 * n_b   = ceil(topk/64) if topk > 0 else ceil(seqlens[b]/64)   (work items)
 * F     = piece_cost if > 0, else max(1, ceil(min(M,128)/64))     (piece cost)
 * U_0 = 0, U_{b+1} = U_b + F + n_b, T = U_B
 * cap   = ceil((T+1)/S)
 * Batch b has max(n_b,1) items; item j sits at P(b,j) = U_b + F + j and
 * belongs to slot floor(P/cap).  (An empty batch has one item, no KV.)
 * splits_b = floor(P(b,last)/cap) - floor(P(b,0)/cap) + 1
 * num_splits[0] = 0, num_splits[b+1] = num_splits[b] + splits_b
 * meta[s] = {b0, j0, b1, j1+1, k0, items, 0, 0} for the first (b0,j0) and
 * last (b1,j1) item of slot s, k0 = s - floor(P(b0,0)/cap) being the split
 * index of batch b0 that slot s computes; an empty slot is {-1,0,-1,0,0,0,0,0}.
 */
int orc_sched_plan(const int32_t* seqlens, int B, int M, int topk, int S, int piece_cost,
                   int32_t* meta, int32_t* num_splits) {
  if (B < 0 || S < 1 || M < 1 || piece_cost < 0) return 1;
  int mm = M < 128 ? M : 128;
  int64_t F = piece_cost > 0 ? piece_cost : (mm + 63) / 64;
  if (F < 1) F = 1;
  int64_t* U = (int64_t*)malloc(sizeof(int64_t) * (size_t)(B + 1));
  int64_t* nb = (int64_t*)malloc(sizeof(int64_t) * (size_t)(B > 0 ? B : 1));
  U[0] = 0;
  for (int b = 0; b < B; ++b) {
    int64_t L = seqlens[b] > 0 ? seqlens[b] : 0;
    nb[b] = topk > 0 ? (topk + ORC_PAGE - 1) / ORC_PAGE : (L + ORC_PAGE - 1) / ORC_PAGE;
    U[b + 1] = U[b] + F + nb[b];
  }
  int64_t T = U[B];
  int64_t cap = (T + 1 + S - 1) / S;
  for (int s = 0; s < S; ++s) {
    int32_t* ms = meta + 8 * (int64_t)s;
    ms[0] = -1; ms[1] = 0; ms[2] = -1; ms[3] = 0; ms[4] = 0; ms[5] = 0; ms[6] = 0; ms[7] = 0;
  }
  num_splits[0] = 0;
  for (int b = 0; b < B; ++b) {
    int64_t items = nb[b] > 0 ? nb[b] : 1;
    int64_t first_slot = (U[b] + F) / cap;
    num_splits[b + 1] = num_splits[b] + (int32_t)((U[b] + F + items - 1) / cap - first_slot + 1);
    for (int64_t j = 0; j < items; ++j) {
      int64_t s = (U[b] + F + j) / cap;
      int32_t* ms = meta + 8 * s;
      if (ms[0] < 0) { /* first item of slot s */
        ms[0] = b; ms[1] = (int32_t)j; ms[4] = (int32_t)(s - first_slot);
      }
      ms[2] = b; ms[3] = (int32_t)(j + 1); ms[5] += 1;
    }
  }
  free(U);
  free(nb);
  return 0;
}
