/*
 * lsa_oracle.c -- CPU oracle for indexer-driven sparse attention.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. This is the plain, slow and
 * obviously correct reference that the GPU library is checked against. Only
 * the test suite, the package's smoke check and the benchmark's CPU-baseline
 * leg may load it. It shares no code, header, table or helper with the GPU
 * library, and the GPU library never calls it.
 *
 * What it computes (sources are the public pages this project follows):
 *   - "Joint Subspace Sparse Attention for Efficient Long-Context Decoding"
 *     (JSSA), Fig. 1: for one KV head at one decoding step, the mean of the
 *     head's query heads, projected into a low-dimensional subspace, scores a
 *     projected-key cache; the top-B token positions are kept; every query
 *     head of the group attends only to those positions (Key contributions:
 *     distinct per-KV-head selections under the standard GQA KV-cache layout).
 *   - "LongCat Sparse Attention: Taming the Lightning via Streaming-aware
 *     Hierarchical Cross-Layer Indexing", abstract: the indexer's O(L^2)
 *     causal prefill scoring, and hierarchical coarse-to-fine scoring that
 *     narrows the candidate set before the fine pass.
 *
 * Conventions that the pages leave open, and the reading taken here:
 *   - every product and sum is taken in double precision; bf16 inputs are
 *     decoded exactly (their 16 bits are the top half of an IEEE binary32);
 *     a value is rounded only where the method stores it (the projected-key
 *     cache and the block centroids), with round-to-nearest-even taken
 *     directly from the double (no intermediate float);
 *   - query head h belongs to KV head h / G (G = Hq / Hkv): consecutive query
 *     heads share a KV head, the standard GQA layout;
 *   - the indexer score is the plain dot product of the projected mean query
 *     and the projected key (no scale, no activation);
 *   - selection order: higher score first; equal scores (+0 and -0 equal)
 *     go to the lower token position; NaN ranks below every number; the
 *     selected positions are written in ascending order and padded with -1;
 *   - attention scale 1/sqrt(d); the softmax runs over the selected set only;
 *     an empty set gives o = 0 and lse = -inf.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC lsa_oracle.c -o liblsa_oracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { REF_F32 = 0, REF_BF16 = 1, REF_FP8 = 2 };

/* ------------------------------------------------------------------------ */
/* Element access                                                           */
/* ------------------------------------------------------------------------ */

/* OCP 8-bit float E4M3 (the "FN" variant: no infinities): sign, 4
 * exponent bits with bias 7, 3 mantissa bits. Exponent field 0 holds the
 * subnormals m * 2^-9; exponent 15 with mantissa 7 is NaN; the largest
 * finite magnitude is 1.75 * 2^8 = 448. (The pages name FP8 projected-key
 * caches -- JSSA Fig. 10 -- but not the format; this is the reading.) */
static double fp8_decode(uint8_t b) {
  int e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return (b & 0x80) ? -v : v;
}

/* Round a double to the nearest E4M3 value, ties to even, straight from the
 * double; beyond the largest finite value the result saturates to +-448
 * (the format has no infinity); NaN stays NaN. With x = f * 2^e,
 * 0.5 <= |f| < 1, a normal E4M3 value keeps 4 significant bits, so the
 * spacing is 2^(e-4); below the smallest normal (2^-6) it stays 2^-9. */
static uint8_t f64_to_fp8(double x) {
  if (isnan(x)) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs(x);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  if (e < -5) e = -5;
  double q = ldexp(1.0, e - 4);
  double y = nearbyint(a / q) * q; /* exact: the quotient is below 2^5 */
  if (y > 448.0) y = 448.0;
  if (y < ldexp(1.0, -6)) return sign | (uint8_t)(y / ldexp(1.0, -9)); /* subnormal (or 0) */
  int E;
  double f = frexp(y, &E); /* y = f * 2^E exactly, f in [0.5, 1) */
  int field = E - 1 + 7;
  int mant = (int)((2.0 * f - 1.0) * 8.0);
  return sign | (uint8_t)(field << 3) | (uint8_t)mant;
}

/* Exact decode of one stored element to double. */
static double elem(const void* p, int dtype, int64_t i) {
  if (dtype == REF_F32) return (double)((const float*)p)[i];
  if (dtype == REF_FP8) return fp8_decode(((const uint8_t*)p)[i]);
  uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Round a double to the nearest bf16 (ties to even), straight from the
 * double: with x = m * 2^e, 0.5 <= |m| < 1, a normal bf16 keeps 8
 * significant bits, so the spacing is 2^(e-8); below the smallest normal
 * (2^-126) the spacing stays 2^-133. */
static uint16_t f64_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
  if (isinf(x)) return signbit(x) ? 0xFF80 : 0x7F80;
  int e;
  frexp(x, &e);
  if (e < -125) e = -125;
  double q = ldexp(1.0, e - 8);
  double y = nearbyint(x / q) * q; /* exact: the quotient is below 2^9 */
  float f = (float)y;              /* exact when |y| fits; overflows to inf */
  if (fabs(y) > 3.3895313892515355e38) f = signbit(y) ? -INFINITY : INFINITY;
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  return (uint16_t)(bits >> 16);
}

static void st(void* p, int dtype, int64_t i, double x) {
  if (dtype == REF_F32)
    ((float*)p)[i] = (float)x;
  else if (dtype == REF_FP8)
    ((uint8_t*)p)[i] = f64_to_fp8(x);
  else
    ((uint16_t*)p)[i] = f64_to_bf16(x);
}

/* Exposed so the tests can pin the rounding rules on their own. */
uint16_t lsa_ref_round_bf16(double x) { return f64_to_bf16(x); }
uint8_t lsa_ref_round_fp8(double x) { return f64_to_fp8(x); }
double lsa_ref_decode_fp8(uint8_t b) { return fp8_decode(b); }

void lsa_ref_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int lsa_ref_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Setup: the projected-key cache and its block centroids                   */
/* ------------------------------------------------------------------------ */

/* k_idx[n,g,t,:] = K[n,t,g,:] . W  (JSSA Fig. 1: the projected-key cache
 * holds every cached key mapped into the shared r-dimensional subspace).
 * K is addressed by element strides (sequence, token, head), innermost d
 * contiguous. W is [d,r] (shared) or [Hkv,d,r] (per KV head), fp32.
 * out is [N,Hkv,T,r] contiguous, stored as out_dtype. */
int lsa_ref_project_keys(const void* K, int k_dtype, int64_t s_seq,
                         int64_t s_tok, int64_t s_head, int N, int T, int Hkv,
                         int d, const float* W, int w_per_head, int r,
                         void* out, int out_dtype) {
  int64_t total = (int64_t)N * Hkv * T;
#pragma omp parallel for schedule(static)
  for (int64_t key = 0; key < total; ++key) {
    int t = (int)(key % T);
    int g = (int)((key / T) % Hkv);
    int n = (int)(key / ((int64_t)T * Hkv));
    int64_t kb = n * s_seq + (int64_t)t * s_tok + (int64_t)g * s_head;
    const float* Wg = W + (w_per_head ? (int64_t)g * d * r : 0);
    for (int j = 0; j < r; ++j) {
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += elem(K, k_dtype, kb + c) * (double)Wg[(int64_t)c * r + j];
      st(out, out_dtype, key * r + j, acc);
    }
  }
  return 0;
}

/* Block centroid = mean of the block's stored projected keys (the coarse
 * level of hierarchical indexing, LongCat Sparse Attention abstract item 3;
 * the summaries are the mean projected key of each block of `block` tokens).
 * A partial last block is averaged over its valid tokens. in is
 * [N,Hkv,T,r] contiguous, out is [N,Hkv,ceil(T/block),r] contiguous, both in
 * `dtype`. */
int lsa_ref_centroids(const void* k_idx, int dtype, int N, int Hkv, int T,
                      int r, int block, void* out) {
  int nb = (T + block - 1) / block;
  int64_t total = (int64_t)N * Hkv * nb;
#pragma omp parallel for schedule(static)
  for (int64_t cb = 0; cb < total; ++cb) {
    int b = (int)(cb % nb);
    int64_t head = cb / nb; /* n * Hkv + g */
    int t0 = b * block;
    int t1 = t0 + block < T ? t0 + block : T;
    for (int j = 0; j < r; ++j) {
      double s = 0.0;
      for (int t = t0; t < t1; ++t) s += elem(k_idx, dtype, (head * T + t) * r + j);
      st(out, dtype, cb * r + j, s / (double)(t1 - t0));
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Scoring preparation (JSSA Fig. 1; Fig. 9 "scoring preparation")          */
/* ------------------------------------------------------------------------ */

/* q_idx[n,g,:] = ( (1/G) sum_{i<G} Q[n, g*G+i, :] ) . W
 * Q is [N,Hq,d] contiguous; out q_idx is [N,Hkv,r] double. */
int lsa_ref_query_prep(const void* Q, int q_dtype, int N, int Hq, int Hkv,
                       int d, const float* W, int w_per_head, int r,
                       double* q_idx) {
  if (Hkv <= 0 || Hq % Hkv != 0) return -1;
  int G = Hq / Hkv;
  double* mean = (double*)malloc(sizeof(double) * (size_t)d);
  for (int n = 0; n < N; ++n)
    for (int g = 0; g < Hkv; ++g) {
      for (int c = 0; c < d; ++c) {
        double s = 0.0;
        for (int i = 0; i < G; ++i) s += elem(Q, q_dtype, ((int64_t)n * Hq + g * G + i) * d + c);
        mean[c] = s / (double)G;
      }
      const float* Wg = W + (w_per_head ? (int64_t)g * d * r : 0);
      for (int j = 0; j < r; ++j) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += mean[c] * (double)Wg[(int64_t)c * r + j];
        q_idx[((int64_t)n * Hkv + g) * r + j] = acc;
      }
    }
  free(mean);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Indexer scoring of the projected-key cache (JSSA Fig. 1; Fig. 9)         */
/* ------------------------------------------------------------------------ */

/* Position of candidate slot s of one row, or -1 when the slot is not a
 * real token. Without a candidate list the slot is the position itself. */
static int64_t slot_pos(const int32_t* cand_row, int cand_block, int64_t s,
                        int n_positions) {
  if (!cand_row) return s < n_positions ? s : -1;
  int32_t c = cand_row[s / cand_block];
  if (c < 0) return -1;
  int64_t p = (int64_t)c * cand_block + s % cand_block;
  return p < n_positions ? p : -1;
}

/* scores[row, s] = q_idx[row] . k_idx[n, g, pos(s)] for row = n*Hkv + g.
 * Without candidates s runs over the T cached positions; with candidates it
 * runs over n_cand * cand_block slots (cand_block = 1: cand holds token
 * positions; cand_block > 1: cand holds block ids, slot s covers token
 * cand[s / cand_block] * cand_block + s % cand_block, the fine level of
 * hierarchical indexing). A slot that maps to no token scores -inf.
 * k_idx is addressed by element strides (sequence, head, token), innermost
 * r contiguous. */
int lsa_ref_scores(const double* q_idx, int N, int Hkv, int r,
                   const void* k_idx, int k_dtype, int64_t ks_seq,
                   int64_t ks_head, int64_t ks_tok, int T,
                   const int32_t* cand, int n_cand, int cand_block,
                   int64_t cand_ld, double* scores, int64_t scores_ld) {
  int rows = N * Hkv;
  int64_t n_out = cand ? (int64_t)n_cand * cand_block : T;
#pragma omp parallel for schedule(dynamic, 1)
  for (int row = 0; row < rows; ++row) {
    int n = row / Hkv, g = row % Hkv;
    const int32_t* cr = cand ? cand + (int64_t)row * cand_ld : NULL;
    const double* q = q_idx + (int64_t)row * r;
    for (int64_t s = 0; s < n_out; ++s) {
      int64_t p = slot_pos(cr, cand_block, s, T);
      double acc;
      if (p < 0) {
        acc = -INFINITY;
      } else {
        int64_t kb = n * ks_seq + g * ks_head + p * ks_tok;
        acc = 0.0;
        for (int j = 0; j < r; ++j) acc += q[j] * elem(k_idx, k_dtype, kb + j);
      }
      scores[(int64_t)row * scores_ld + s] = acc;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Exact top-B selection (JSSA Fig. 1; Fig. 9 "top-B selection")            */
/* ------------------------------------------------------------------------ */

typedef struct {
  double score;
  int64_t pos;
} cand_t;

/* Selection order: higher score first, NaN last, equal scores (including
 * +0 == -0) to the lower position. */
static int order_cmp(const void* a_, const void* b_) {
  const cand_t* a = (const cand_t*)a_;
  const cand_t* b = (const cand_t*)b_;
  int na = isnan(a->score), nb = isnan(b->score);
  if (na != nb) return na ? 1 : -1;
  if (!na && a->score != b->score) return a->score > b->score ? -1 : 1;
  return (a->pos > b->pos) - (a->pos < b->pos);
}

static int pos_cmp(const void* a_, const void* b_) {
  const cand_t* a = (const cand_t*)a_;
  const cand_t* b = (const cand_t*)b_;
  return (a->pos > b->pos) - (a->pos < b->pos);
}

/* One row: keep the first min(B, valid) slots of the selection order,
 * write their positions ascending, pad with -1. Returns the count. */
static int select_row(const double* sc, int64_t n_slots, const int32_t* cand_row,
                      int cand_block, int n_positions, int B, cand_t* buf,
                      int32_t* out_idx, double* out_score) {
  int64_t m = 0;
  for (int64_t s = 0; s < n_slots; ++s) {
    int64_t p = slot_pos(cand_row, cand_block, s, n_positions);
    if (p < 0) continue;
    buf[m].score = sc[s];
    buf[m].pos = p;
    ++m;
  }
  qsort(buf, (size_t)m, sizeof(cand_t), order_cmp);
  int k = m < B ? (int)m : B;
  qsort(buf, (size_t)k, sizeof(cand_t), pos_cmp);
  for (int i = 0; i < B; ++i) {
    out_idx[i] = i < k ? (int32_t)buf[i].pos : -1;
    if (out_score) out_score[i] = i < k ? buf[i].score : -INFINITY;
  }
  return k;
}

/* Per row: the top-B valid slots (JSSA Fig. 1: the top-B token positions
 * per KV head). Valid slots of row `row` are s < n_valid[row] (or all n
 * slots when n_valid is NULL; or s < row / causal_group + 1 when
 * causal_group > 0, the causal prefix of query row / causal_group) whose
 * position is a real token (see slot_pos; n_positions bounds the positions,
 * pass n when there is no candidate list). */
int lsa_ref_topk(const double* scores, int rows, int n, int64_t ld,
                 const int32_t* n_valid, int causal_group, const int32_t* cand,
                 int cand_block, int64_t cand_ld, int n_positions, int B,
                 int32_t* out_idx, double* out_score, int32_t* out_count) {
  if (B < 1) return -1;
#pragma omp parallel
  {
    cand_t* buf = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
#pragma omp for schedule(dynamic, 1)
    for (int row = 0; row < rows; ++row) {
      int64_t nv = n;
      if (n_valid) nv = n_valid[row] < n ? n_valid[row] : n;
      if (causal_group > 0) {
        int64_t c = row / causal_group + 1;
        nv = c < n ? c : n;
      }
      if (nv < 0) nv = 0;
      const int32_t* cr = cand ? cand + (int64_t)row * cand_ld : NULL;
      int cnt = select_row(scores + (int64_t)row * ld, nv, cr, cand_block,
                           cand ? n_positions : (int)nv, B, buf,
                           out_idx + (int64_t)row * B,
                           out_score ? out_score + (int64_t)row * B : NULL);
      if (out_count) out_count[row] = cnt;
    }
    free(buf);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Causal prefill indexer (LongCat Sparse Attention abstract: the indexer's */
/* O(L^2) scoring; per query token, top-B over its causal prefix)           */
/* ------------------------------------------------------------------------ */

/* For query rows i in [row_begin, row_end) and KV head g: scores
 * S[i,j] = q_idx[i,g] . k_idx[j,g] for j <= i, then the top-B of that
 * prefix in the selection order. q_idx and k_idx are [L,Hkv,r]
 * contiguous. out_idx / out_score are [(row_end-row_begin), Hkv, B]. */
int lsa_ref_prefill_topk(const void* q_idx, const void* k_idx, int dtype,
                         int L, int Hkv, int r, int row_begin, int row_end,
                         int B, int32_t* out_idx, double* out_score) {
  if (B < 1) return -1;
  int64_t tasks = (int64_t)(row_end - row_begin) * Hkv;
#pragma omp parallel
  {
    cand_t* buf = (cand_t*)malloc(sizeof(cand_t) * (size_t)L);
    double* sc = (double*)malloc(sizeof(double) * (size_t)L);
    double* q = (double*)malloc(sizeof(double) * (size_t)r);
#pragma omp for schedule(dynamic, 1)
    for (int64_t task = 0; task < tasks; ++task) {
      int i = row_begin + (int)(task / Hkv);
      int g = (int)(task % Hkv);
      for (int j = 0; j < r; ++j) q[j] = elem(q_idx, dtype, ((int64_t)i * Hkv + g) * r + j);
      for (int t = 0; t <= i; ++t) {
        double acc = 0.0;
        for (int j = 0; j < r; ++j) acc += q[j] * elem(k_idx, dtype, ((int64_t)t * Hkv + g) * r + j);
        sc[t] = acc;
      }
      select_row(sc, i + 1, NULL, 1, i + 1, B, buf, out_idx + task * B,
                 out_score ? out_score + task * B : NULL);
    }
    free(buf);
    free(sc);
    free(q);
  }
  return 0;
}

/* Query-block-shared prefill selection (the query_block_size option of
 * LSA-L's sparse-attention call, "Their 42x decode speedup never compiled
 * on my GPU", section "The failure that decided the verdict"; the page
 * names the option only, so this is a reading). The L query tokens form
 * blocks of qb consecutive tokens; block b covers tokens [b*qb,
 * min(L,(b+1)*qb)). One selection serves the whole block:
 *   qbar[b,g]  = mean of q_idx[i,g] over the block's tokens, stored in the
 *                q_idx dtype (the same head-mean reduction the decode
 *                prep applies to a GQA group, here over tokens);
 *   S[b,g,j]   = qbar[b,g] . k_idx[j,g] for j < min(L,(b+1)*qb), the keys
 *                visible to the block's last token;
 *   then the top-B of that prefix in the selection order.
 * Each token of the block later attends to the selection's positions
 * j <= its own (lsa_ref_attention's query_block). out_idx / out_score are
 * [ceil(L/qb), Hkv, B]. qb = 1 is lsa_ref_prefill_topk. */
static void block_query(const void* q_idx, int dtype, int L, int Hkv, int r, int qb, int b,
                        int g, double* q) {
  int i0 = b * qb, i1 = (b + 1) * qb < L ? (b + 1) * qb : L;
  for (int c = 0; c < r; ++c) {
    double s = 0.0;
    for (int i = i0; i < i1; ++i) s += elem(q_idx, dtype, ((int64_t)i * Hkv + g) * r + c);
    double mean = s / (double)(i1 - i0);
    if (dtype == REF_BF16) {
      uint16_t bits = f64_to_bf16(mean);
      q[c] = elem(&bits, REF_BF16, 0);
    } else {
      q[c] = (double)(float)mean;
    }
  }
}

int lsa_ref_prefill_block_topk(const void* q_idx, const void* k_idx, int dtype, int L, int Hkv,
                               int r, int qb, int B, int32_t* out_idx, double* out_score,
                               double* scores, int64_t ld) {
  if (B < 0 || qb < 1 || (B == 0 && !scores)) return -1;
  int nbk = (L + qb - 1) / qb;
  int64_t tasks = (int64_t)nbk * Hkv;
#pragma omp parallel
  {
    cand_t* buf = (cand_t*)malloc(sizeof(cand_t) * (size_t)L);
    double* sc = (double*)malloc(sizeof(double) * (size_t)L);
    double* q = (double*)malloc(sizeof(double) * (size_t)r);
#pragma omp for schedule(dynamic, 1)
    for (int64_t task = 0; task < tasks; ++task) {
      int b = (int)(task / Hkv), g = (int)(task % Hkv);
      block_query(q_idx, dtype, L, Hkv, r, qb, b, g, q);
      int nv = (b + 1) * qb < L ? (b + 1) * qb : L;
      for (int t = 0; t < L; ++t) {
        double acc = -INFINITY;
        if (t < nv) {
          acc = 0.0;
          for (int j = 0; j < r; ++j) acc += q[j] * elem(k_idx, dtype, ((int64_t)t * Hkv + g) * r + j);
        }
        sc[t] = acc;
        if (scores) scores[task * ld + t] = acc;
      }
      if (B > 0)
        select_row(sc, nv, NULL, 1, nv, B, buf, out_idx + task * B,
                   out_score ? out_score + task * B : NULL);
    }
    free(buf);
    free(sc);
    free(q);
  }
  return 0;
}

/* Full causal score matrix for small L: scores[(i*Hkv+g)*ld + j] =
 * q_idx[i,g] . k_idx[j,g] for j <= i and -inf for j > i. */
int lsa_ref_prefill_scores(const void* q_idx, const void* k_idx, int dtype,
                           int L, int Hkv, int r, double* scores, int64_t ld) {
  int64_t tasks = (int64_t)L * Hkv;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t task = 0; task < tasks; ++task) {
    int i = (int)(task / Hkv), g = (int)(task % Hkv);
    for (int t = 0; t < L; ++t) {
      double acc = -INFINITY;
      if (t <= i) {
        acc = 0.0;
        for (int j = 0; j < r; ++j)
          acc += elem(q_idx, dtype, task * r + j) * elem(k_idx, dtype, ((int64_t)t * Hkv + g) * r + j);
      }
      scores[task * ld + t] = acc;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Indexed attention over the selected positions (JSSA Fig. 1; Key         */
/* contributions: per-KV-head index sets read in place from the standard    */
/* GQA KV-cache layout)                                                     */
/* ------------------------------------------------------------------------ */

/* For each row and query head h (KV head g = h / G):
 *   z_t = scale * q[row,h] . K[seq, t, g]      for t in idx[row, g, :], t >= 0
 *   o   = sum_t softmax(z)_t V[seq, t, g],  lse = log sum_t exp(z_t)
 * mode 0 (decode): row is the sequence; mode 1 (prefill): every row is a
 * query token of sequence 0, and causal: positions after the row's own token
 * are skipped. q is [rows,Hq,d] contiguous; K and V share the element
 * strides (sequence, token, head), innermost d contiguous; idx is
 * [ceil(rows/qb),Hkv,B]: row `row` reads index row row/qb (qb = 1: one
 * index row per row; qb > 1, prefill only: a selection shared by a block of
 * qb query tokens); entries outside [0,T) are skipped. scale <= 0 means
 * 1/sqrt(d). */
int lsa_ref_attention(int mode, int rows, int Hq, int Hkv, int d, int B,
                      const void* q, int q_dtype, const void* Kc,
                      const void* Vc, int kv_dtype, int64_t s_seq,
                      int64_t s_tok, int64_t s_head, int T,
                      const int32_t* idx, int qb, double scale, double* out,
                      double* lse) {
  if (Hkv <= 0 || Hq % Hkv != 0 || qb < 1 || (qb > 1 && mode != 1)) return -1;
  int G = Hq / Hkv;
  if (!(scale > 0.0)) scale = 1.0 / sqrt((double)d);
  int64_t tasks = (int64_t)rows * Hq;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)(B > 0 ? B : 1));
#pragma omp for schedule(dynamic, 4)
    for (int64_t task = 0; task < tasks; ++task) {
      int row = (int)(task / Hq), h = (int)(task % Hq), g = h / G;
      int64_t seq = mode == 0 ? row : 0;
      int64_t tmax = mode == 1 ? (row < T - 1 ? row : T - 1) : T - 1;  /* last visible position */
      const int32_t* I = idx + ((int64_t)(row / qb) * Hkv + g) * B;
      int64_t q_off = task * d;   /* this (row, head)'s query vector */
      double m = -INFINITY;
      for (int b = 0; b < B; ++b) {
        int64_t t = I[b];
        if (t < 0 || t > tmax) continue;
        int64_t kb = seq * s_seq + t * s_tok + (int64_t)g * s_head;
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += elem(q, q_dtype, q_off + c) * elem(Kc, kv_dtype, kb + c);
        z[b] = acc * scale;
        if (z[b] > m) m = z[b];
      }
      double* o = out + task * d;
      for (int c = 0; c < d; ++c) o[c] = 0.0;
      if (m == -INFINITY) {
        if (lse) lse[task] = -INFINITY;
        continue;
      }
      double l = 0.0;
      for (int b = 0; b < B; ++b) {
        int64_t t = I[b];
        if (t < 0 || t > tmax) continue;
        double p = exp(z[b] - m);
        l += p;
        int64_t vb = seq * s_seq + t * s_tok + (int64_t)g * s_head;
        for (int c = 0; c < d; ++c) o[c] += p * elem(Vc, kv_dtype, vb + c);
      }
      for (int c = 0; c < d; ++c) o[c] /= l;
      if (lse) lse[task] = m + log(l);
    }
    free(z);
  }
  return 0;
}
