/*
 * dsa_oracle.c -- plain, slow CPU reference for the DeepSeek Sparse Attention
 * (DSA) hot path: Lightning-Indexer scores, top-k selection, and sparse GQA
 * attention over the selected positions.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may link, load
 * or call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * What it follows (page 5, "Kwai Keye-VL-2.0 technical report" summary,
 * section 1 on long-video cost):
 *   - a lightweight scout module (the Lightning Indexer) scores every
 *     position of the context for the current query token;
 *   - the scout keeps ONE shared key per position (an MQA design: "one set
 *     of eyes"), used by all of its heads;
 *   - for each query token the k = 2048 most relevant positions are kept,
 *     and attention runs only over them, turning O(L^2) into O(L k);
 *   - the base model is GQA (the same section, paragraph on the GQA/DSA
 *     adaptation): one index set per token serves every query head.
 * The indexer score itself is not printed on the pages; this file uses the
 * plain weighted-ReLU form  I[t,s] = sum_h w[t,h] * max(0, qI[t,h] . kI[s]).
 * Page 5 section 8 (training-side engineering) asks for a deterministic
 * top-k; ties are broken towards the lower position here.
 *
 * Every floating-point step is done in IEEE double, on the exact values of
 * the bf16 / fp32 inputs, in the textbook order of the definition.
 *
 * Varlen convention: sequence b owns packed query rows [cu_q[b], cu_q[b+1])
 * and packed key rows [cu_k[b], cu_k[b+1]).  Local query i of sequence b sits
 * at position p = Lk_b - Lq_b + i and may see local keys 0..p (self
 * included).  Indices are sequence-local positions.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the upper half of an IEEE binary32; the conversion is exact. */
static double bf16_to_double(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Locate the sequence that owns packed query row r; returns its index or -1. */
static int find_seq(int batch, const int32_t* cu_q, int64_t r) {
  for (int b = 0; b < batch; ++b)
    if (r >= cu_q[b] && r < cu_q[b + 1]) return b;
  return -1;
}

/* Causal position of packed query row r inside its sequence. */
static int64_t row_position(const int32_t* cu_q, const int32_t* cu_k, int b, int64_t r) {
  int64_t lq = cu_q[b + 1] - cu_q[b];
  int64_t lk = cu_k[b + 1] - cu_k[b];
  return lk - lq + (r - cu_q[b]);
}

/*
 * Number of visible keys (p + 1) for each requested row; -1 for a row that
 * belongs to no sequence or whose position is negative (Lq > Lk).
 */
int oracle_visible_counts(int batch, const int32_t* cu_q, const int32_t* cu_k,
                          int64_t n_rows, const int64_t* rows, int64_t* counts) {
  int bad = 0;
  for (int64_t i = 0; i < n_rows; ++i) {
    int b = find_seq(batch, cu_q, rows[i]);
    if (b < 0) { counts[i] = -1; bad = 1; continue; }
    int64_t p = row_position(cu_q, cu_k, b, rows[i]);
    if (p < 0) { counts[i] = -1; bad = 1; continue; }
    counts[i] = p + 1;
  }
  return bad;
}

/*
 * Indexer scores for the requested packed query rows.
 *   qI : bf16 [total_q, n_heads, d]      w : fp32 [total_q, n_heads]
 *   kI : bf16 [total_k, d]  (one key per position, shared by every head)
 *   scores : double [n_rows, ld]; column s <= p receives I[row, s], columns
 *            beyond p are set to NaN so that any use of them shows.
 * Returns 0, or 1 if a row is outside every sequence.
 */
int oracle_index_scores(int batch, const int32_t* cu_q, const int32_t* cu_k,
                        const uint16_t* qI, const uint16_t* kI, const float* w,
                        int n_heads, int d, int64_t n_rows, const int64_t* rows,
                        double* scores, int64_t ld) {
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t r = rows[i];
    double* out = scores + i * ld;
    for (int64_t s = 0; s < ld; ++s) out[s] = NAN;
    int b = find_seq(batch, cu_q, r);
    if (b < 0) { bad = 1; continue; }
    int64_t p = row_position(cu_q, cu_k, b, r);
    if (p < 0 || p >= ld) { bad = 1; continue; }
    double* q = (double*)malloc(sizeof(double) * (size_t)n_heads * (size_t)d);
    double* wr = (double*)malloc(sizeof(double) * (size_t)n_heads);
    for (int h = 0; h < n_heads; ++h) {
      wr[h] = (double)w[r * n_heads + h];
      for (int j = 0; j < d; ++j)
        q[h * d + j] = bf16_to_double(qI[(r * n_heads + h) * d + j]);
    }
    for (int64_t s = 0; s <= p; ++s) {
      const uint16_t* key = kI + (cu_k[b] + s) * d;
      double total = 0.0;
      for (int h = 0; h < n_heads; ++h) {
        double dot = 0.0;
        for (int j = 0; j < d; ++j) dot += q[h * d + j] * bf16_to_double(key[j]);
        double relu = dot > 0.0 ? dot : 0.0;
        total += wr[h] * relu;
      }
      out[s] = total + 0.0; /* -0.0 becomes +0.0 */
    }
    free(q);
    free(wr);
  }
  return bad;
}

typedef struct {
  double score;
  int32_t pos;
} scored_pos;

/* Larger score first; on equal scores the lower position first. */
static int by_score_then_pos(const void* a, const void* b) {
  const scored_pos* x = (const scored_pos*)a;
  const scored_pos* y = (const scored_pos*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

static int ascending_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/*
 * Top-k per row.  counts[i] = p + 1 visible positions of row i; scores row i
 * holds valid values in columns 0..counts[i]-1 (any finite double; -0.0 and
 * +0.0 compare equal, as IEEE comparison makes them).  The n = min(k,
 * counts[i]) best positions by (score descending, position ascending) are
 * written to idx[i, 0..n-1] in ascending position order; idx[i, n..k-1] = -1.
 */
int oracle_topk(int64_t n_rows, const int64_t* counts, const double* scores, int64_t ld,
                int k, int32_t* idx) {
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t i = 0; i < n_rows; ++i) {
    int32_t* out = idx + i * (int64_t)k;
    for (int j = 0; j < k; ++j) out[j] = -1;
    int64_t cnt = counts[i];
    if (cnt <= 0 || cnt > ld) { bad = 1; continue; }
    scored_pos* all = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)cnt);
    for (int64_t s = 0; s < cnt; ++s) {
      all[s].score = scores[i * ld + s];
      all[s].pos = (int32_t)s;
    }
    qsort(all, (size_t)cnt, sizeof(scored_pos), by_score_then_pos);
    int64_t n = cnt < k ? cnt : k;
    for (int64_t j = 0; j < n; ++j) out[j] = all[j].pos;
    qsort(out, (size_t)n, sizeof(int32_t), ascending_i32);
    free(all);
  }
  return bad;
}

/*
 * Sparse GQA attention for the requested rows over their selected positions.
 *   Q : bf16 [total_q, n_heads_q, d]   K, V : bf16 [total_k, n_heads_kv, d]
 *   idx : int32 [n_rows, topk] sequence-local positions, -1 = unused slot
 *   out : double [n_rows, n_heads_q, d]    lse : double [n_rows, n_heads_q]
 * Query head h reads KV head g = h / (n_heads_q / n_heads_kv).
 *   z_s = scale * Q[h] . K[s, g],  O = sum_s e^{z_s - m} V[s, g] / sum_s e^{z_s - m},
 *   lse = m + ln sum_s e^{z_s - m},  m = max_s z_s.
 * A row with no valid index gets O = 0 and lse = -inf.
 * Returns 0, or 1 on an invalid row or an index outside 0..p.
 */
int oracle_sparse_attn(int batch, const int32_t* cu_q, const int32_t* cu_k,
                       const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                       int n_heads_q, int n_heads_kv, int d, double scale,
                       int64_t n_rows, const int64_t* rows, const int32_t* idx, int topk,
                       double* out, double* lse) {
  int bad = 0;
  int group = n_heads_q / n_heads_kv;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t r = rows[i];
    int b = find_seq(batch, cu_q, r);
    double* o = out + i * (int64_t)n_heads_q * d;
    for (int64_t e = 0; e < (int64_t)n_heads_q * d; ++e) o[e] = 0.0;
    for (int h = 0; h < n_heads_q; ++h) lse[i * n_heads_q + h] = -INFINITY;
    if (b < 0) { bad = 1; continue; }
    int64_t p = row_position(cu_q, cu_k, b, r);
    const int32_t* sel = idx + i * (int64_t)topk;
    int n = 0;
    for (int j = 0; j < topk; ++j) {
      if (sel[j] < 0) continue;
      if (sel[j] > p) bad = 1;
      ++n;
    }
    if (n == 0) continue;
    double* z = (double*)malloc(sizeof(double) * (size_t)topk);
    for (int h = 0; h < n_heads_q; ++h) {
      int g = h / group;
      const uint16_t* q = Q + (r * n_heads_q + h) * (int64_t)d;
      double m = -INFINITY;
      for (int j = 0; j < topk; ++j) {
        if (sel[j] < 0 || sel[j] > p) { z[j] = -INFINITY; continue; }
        const uint16_t* key = K + ((cu_k[b] + sel[j]) * (int64_t)n_heads_kv + g) * d;
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += bf16_to_double(q[c]) * bf16_to_double(key[c]);
        z[j] = scale * dot;
        if (z[j] > m) m = z[j];
      }
      double denom = 0.0;
      for (int j = 0; j < topk; ++j) {
        if (z[j] == -INFINITY) continue;
        double e = exp(z[j] - m);
        denom += e;
        const uint16_t* val = V + ((cu_k[b] + sel[j]) * (int64_t)n_heads_kv + g) * d;
        for (int c = 0; c < d; ++c) o[h * d + c] += e * bf16_to_double(val[c]);
      }
      for (int c = 0; c < d; ++c) o[h * d + c] /= denom;
      lse[i * n_heads_q + h] = m + log(denom);
    }
    free(z);
  }
  return bad;
}

/* ------------------------------------------------------------------------
 * FP8 indexer inputs (a declared input transform, not on the pages: they
 * give no indexer precision).  Format: OCP 8-bit floating point, E4M3 variant
 * ("e4m3fn"): sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent field 0 encodes subnormals m/8 * 2^-6; no infinities; S.1111.111
 * is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
 *
 * Quantisation of one vector x of d values (one indexer key, or one head of
 * one indexer query), with every step an IEEE binary32 operation:
 *   amax  = max_j |x_j|
 *   inv   = 448 / amax            (binary32 division)
 *   c_j   = e4m3(x_j * inv)       (binary32 product, then round to nearest,
 *                                  ties to even, saturating at +-448)
 *   scale = amax / 448            (binary32 division)
 * and x_j is represented by scale * value(c_j).  A vector of zeros gets codes
 * 0 and scale 0.  The fp8 indexer score is the weighted-ReLU score of these
 * represented values.
 * ------------------------------------------------------------------------ */

/* Value of an e4m3fn code (NaN for the two NaN codes). */
double oracle_e4m3_value(uint8_t code) {
  int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double v = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
  return sign ? -v : v;
}

/* Nearest e4m3fn code to a finite y: round to nearest, ties to the even
   mantissa, magnitudes beyond 448 saturate to 448; the sign is kept (so -0.0
   gives the negative-zero code). */
uint8_t oracle_e4m3_encode(double y) {
  uint8_t sign = signbit(y) ? 0x80 : 0;
  double a = fabs(y);
  /* Spacing of representable values around a: 2^(e-3) for a in [2^e, 2^(e+1))
     with e >= -6; subnormals (a < 2^-6) are spaced 2^-9. */
  int e = a < ldexp(1.0, -6) ? -6 : ilogb(a);
  double quantum = ldexp(1.0, e - 3);
  double n = nearbyint(a / quantum); /* a / quantum is exact; default rounding is to even */
  double v = n * quantum;
  if (v > 448.0) v = 448.0;
  /* Code of the representable magnitude v. */
  uint8_t mag;
  if (v < ldexp(1.0, -6)) {
    mag = (uint8_t)(v / ldexp(1.0, -9));
  } else {
    int ev = ilogb(v);
    mag = (uint8_t)(((ev + 7) << 3) | (int)(v / ldexp(1.0, ev) * 8.0 - 8.0));
  }
  return sign | mag;
}

/*
 * Quantise rows of a bf16 matrix x [rows, d] to codes [rows, d] and scales
 * [rows] as stated above.  Returns 0, or 1 if an input is not finite.
 */
int oracle_quantize_fp8(const uint16_t* x, int64_t rows, int d, uint8_t* codes,
                        float* scales) {
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t r = 0; r < rows; ++r) {
    float amax = 0.0f;
    for (int j = 0; j < d; ++j) {
      float v = (float)bf16_to_double(x[r * d + j]);
      if (!isfinite(v)) bad = 1;
      if (fabsf(v) > amax) amax = fabsf(v);
    }
    if (amax == 0.0f) {
      for (int j = 0; j < d; ++j) codes[r * d + j] = 0;
      scales[r] = 0.0f;
      continue;
    }
    volatile float inv = 448.0f / amax;
    for (int j = 0; j < d; ++j) {
      volatile float y = (float)bf16_to_double(x[r * d + j]) * inv;
      codes[r * d + j] = oracle_e4m3_encode((double)y);
    }
    volatile float scale = amax / 448.0f;
    scales[r] = scale;
  }
  return bad;
}

/* Represented values scale[r] * value(codes[r, j]) as doubles (exact). */
void oracle_dequantize_fp8(const uint8_t* codes, const float* scales, int64_t rows, int d,
                           double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int j = 0; j < d; ++j)
      out[r * d + j] = (double)scales[r] * oracle_e4m3_value(codes[r * d + j]);
}

/*
 * Indexer scores from real-valued (double) queries and keys, same definition
 * and conventions as oracle_index_scores:
 *   q_rows : double [n_rows, n_heads, d]  the queries of the requested rows
 *   kI     : double [total_k, d]          w : fp32 [total_q, n_heads]
 */
int oracle_index_scores_f64(int batch, const int32_t* cu_q, const int32_t* cu_k,
                            const double* q_rows, const double* kI, const float* w,
                            int n_heads, int d, int64_t n_rows, const int64_t* rows,
                            double* scores, int64_t ld) {
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t r = rows[i];
    double* out = scores + i * ld;
    for (int64_t s = 0; s < ld; ++s) out[s] = NAN;
    int b = find_seq(batch, cu_q, r);
    if (b < 0) { bad = 1; continue; }
    int64_t p = row_position(cu_q, cu_k, b, r);
    if (p < 0 || p >= ld) { bad = 1; continue; }
    const double* q = q_rows + i * (int64_t)n_heads * d;
    for (int64_t s = 0; s <= p; ++s) {
      const double* key = kI + (cu_k[b] + s) * d;
      double total = 0.0;
      for (int h = 0; h < n_heads; ++h) {
        double dot = 0.0;
        for (int j = 0; j < d; ++j) dot += q[h * d + j] * key[j];
        double relu = dot > 0.0 ? dot : 0.0;
        total += (double)w[r * n_heads + h] * relu;
      }
      out[s] = total + 0.0;
    }
  }
  return bad;
}

/* ------------------------------------------------------------------------
 * Indexer warm-up loss (page 5 section 1, the paragraph on the two training
 * stages: in the dense warm-up the rest of the model is frozen and only the
 * indexer is trained, so that its judgement of which positions matter comes
 * close to the full attention's distribution, the gap measured by the KL
 * divergence).  The pages print no formula.  Read plainly, for query row t
 * at position p (keys s = 0..p):
 *   z_h[s]  = scale * Q[t,h] . K[s, h / G]                  (G = Hq / Hkv)
 *   A_h[s]  = exp(z_h[s]) / sum_{s'} exp(z_h[s'])           (dense attention, head h)
 *   P[s]    = (1/Hq) sum_h A_h[s]                           (the target: heads averaged)
 *   Pi[s]   = exp(I[t,s]) / sum_{s'} exp(I[t,s'])           (the indexer's distribution)
 *   loss[t] = sum_s P[s] (ln P[s] - ln Pi[s])               (KL(P || Pi); P[s] = 0 adds 0)
 *   grad[t,s] = Pi[s] - P[s]                                (d loss[t] / d I[t,s]; P is a
 *                                                            fixed target)
 * scores holds I for the listed rows (row i at scores + i ld, columns 0..p);
 * grad, when not NULL, receives columns 0..p of each row in the same layout.
 * ------------------------------------------------------------------------ */
int oracle_indexer_kl(int batch, const int32_t* cu_q, const int32_t* cu_k,
                      const uint16_t* Q, const uint16_t* K, int n_heads_q, int n_heads_kv,
                      int d, double scale, int64_t n_rows, const int64_t* rows,
                      const double* scores, int64_t ld, double* loss, double* grad) {
  int bad = 0;
  int group = n_heads_q / n_heads_kv;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t r = rows[i];
    int b = find_seq(batch, cu_q, r);
    loss[i] = 0.0;
    if (b < 0) { bad = 1; continue; }
    int64_t p = row_position(cu_q, cu_k, b, r);
    if (p + 1 > ld) { bad = 1; continue; }
    int64_t n = p + 1;
    const double* I = scores + i * ld;
    double* P = (double*)calloc((size_t)n, sizeof(double));
    double* z = (double*)malloc(sizeof(double) * (size_t)n);
    /* P: the per-head softmax over all visible keys, averaged over heads. */
    for (int h = 0; h < n_heads_q; ++h) {
      int g = h / group;
      const uint16_t* q = Q + (r * n_heads_q + h) * (int64_t)d;
      double m = -INFINITY;
      for (int64_t s = 0; s < n; ++s) {
        const uint16_t* key = K + ((cu_k[b] + s) * (int64_t)n_heads_kv + g) * d;
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += bf16_to_double(q[c]) * bf16_to_double(key[c]);
        z[s] = scale * dot;
        if (z[s] > m) m = z[s];
      }
      double denom = 0.0;
      for (int64_t s = 0; s < n; ++s) denom += exp(z[s] - m);
      for (int64_t s = 0; s < n; ++s) P[s] += exp(z[s] - m) / denom / n_heads_q;
    }
    /* ln Pi[s] = I[s] - (mI + ln sum exp(I - mI)). */
    double mI = -INFINITY;
    for (int64_t s = 0; s < n; ++s)
      if (I[s] > mI) mI = I[s];
    double lI = 0.0;
    for (int64_t s = 0; s < n; ++s) lI += exp(I[s] - mI);
    double log_norm = mI + log(lI);
    double kl = 0.0;
    for (int64_t s = 0; s < n; ++s) {
      double log_pi = I[s] - log_norm;
      if (P[s] > 0.0) kl += P[s] * (log(P[s]) - log_pi);
      if (grad) grad[i * ld + s] = exp(log_pi) - P[s];
    }
    loss[i] = kl;
    free(P);
    free(z);
  }
  return bad;
}

/* ------------------------------------------------------------------------
 * Backward of the indexer score (page 5 section 1, the two training stages:
 * the dense warm-up trains only the indexer, so the warm-up loss's gradient
 * must reach the indexer's own inputs).  With G[i, s] = d L / d I[t, s] for
 * listed row i (packed row t at position p; columns 0..p), x = qI[t,h] . kI[s]
 * and the ReLU's derivative read as 1 for x > 0 and 0 otherwise:
 *   dq[i, h, :] = sum_{s <= p} G[i,s] w[t,h] [x > 0] kI[s, :]
 *   dw[i, h]    = sum_{s <= p} G[i,s] max(0, x)
 *   dk[c, :]   += sum_i sum_h G[i, s] w[t,h] [x > 0] qI[t,h,:]  (c = packed key of
 *                                                               position s of t's sequence)
 * Inputs as in oracle_index_scores_f64 (double queries of the listed rows,
 * double keys); dk [total_k, d] is accumulated (the caller clears it).
 * Columns of G beyond a row's position are never read.
 * Returns 0, or 1 if a row is outside every sequence or p >= ld.
 * ------------------------------------------------------------------------ */
int oracle_index_scores_backward(int batch, const int32_t* cu_q, const int32_t* cu_k,
                                 const double* q_rows, const double* kI, const float* w,
                                 int n_heads, int d, int64_t n_rows, const int64_t* rows,
                                 const double* G, int64_t ld, double* dq, double* dw,
                                 double* dk) {
  int bad = 0;
  int* seq = (int*)malloc(sizeof(int) * (size_t)(n_rows > 0 ? n_rows : 1));
  int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_rows > 0 ? n_rows : 1));
  for (int64_t i = 0; i < n_rows; ++i) {
    seq[i] = find_seq(batch, cu_q, rows[i]);
    pos[i] = seq[i] < 0 ? -1 : row_position(cu_q, cu_k, seq[i], rows[i]);
    if (seq[i] < 0 || pos[i] < 0 || pos[i] >= ld) bad = 1;
  }
  if (bad) {
    free(seq);
    free(pos);
    return 1;
  }
  /* dq and dw: one listed row at a time. */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_rows; ++i) {
    const int64_t t = rows[i];
    const double* q = q_rows + i * (int64_t)n_heads * d;
    double* dqi = dq + i * (int64_t)n_heads * d;
    for (int64_t e = 0; e < (int64_t)n_heads * d; ++e) dqi[e] = 0.0;
    for (int h = 0; h < n_heads; ++h) dw[i * n_heads + h] = 0.0;
    for (int64_t s = 0; s <= pos[i]; ++s) {
      const double g = G[i * ld + s];
      const double* key = kI + (cu_k[seq[i]] + s) * d;
      for (int h = 0; h < n_heads; ++h) {
        double x = 0.0;
        for (int j = 0; j < d; ++j) x += q[h * d + j] * key[j];
        if (x > 0.0) {
          const double coef = g * (double)w[t * n_heads + h];
          for (int j = 0; j < d; ++j) dqi[h * d + j] += coef * key[j];
          dw[i * n_heads + h] += g * x;
        }
      }
    }
  }
  /* dk: one packed key at a time, over the listed rows that see it. */
  const int64_t total_k = cu_k[batch];
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t c = 0; c < total_k; ++c) {
    int b = 0;
    while (b + 1 < batch && cu_k[b + 1] <= c) ++b;
    const int64_t s = c - cu_k[b];
    const double* key = kI + c * d;
    for (int64_t i = 0; i < n_rows; ++i) {
      if (seq[i] != b || s > pos[i]) continue;
      const int64_t t = rows[i];
      const double g = G[i * ld + s];
      const double* q = q_rows + i * (int64_t)n_heads * d;
      for (int h = 0; h < n_heads; ++h) {
        double x = 0.0;
        for (int j = 0; j < d; ++j) x += q[h * d + j] * key[j];
        if (x > 0.0) {
          const double coef = g * (double)w[t * n_heads + h];
          for (int j = 0; j < d; ++j) dk[c * d + j] += coef * q[h * d + j];
        }
      }
    }
  }
  free(seq);
  free(pos);
  return 0;
}

/* dk of the indexer backward for listed packed keys only: dk[c] = sum over
 * the listed rows i that see key keys[c] (same sequence, local position at
 * most the row's) and every head h with x = qI[i,h] . kI[key] > 0 of
 * Gk[i, c] * w[row_i, h] * qI[i, h, :].  Gk [n_rows, n_keys] holds dL/dI at
 * (row i, key c).  The sum is the key's column of the dense backward above,
 * without touching the keys nobody asked for.  Returns 1 on an invalid row
 * or key. */
int oracle_index_scores_backward_keys(int batch, const int32_t* cu_q, const int32_t* cu_k,
                                      const double* q_rows, const double* kI, const float* w,
                                      int n_heads, int d, int64_t n_rows, const int64_t* rows,
                                      const double* Gk, int64_t n_keys, const int64_t* keys,
                                      double* dk) {
  int bad = 0;
  int* seq = (int*)malloc(sizeof(int) * (size_t)(n_rows > 0 ? n_rows : 1));
  int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_rows > 0 ? n_rows : 1));
  for (int64_t i = 0; i < n_rows; ++i) {
    seq[i] = find_seq(batch, cu_q, rows[i]);
    pos[i] = seq[i] < 0 ? -1 : row_position(cu_q, cu_k, seq[i], rows[i]);
    if (seq[i] < 0 || pos[i] < 0) bad = 1;
  }
  for (int64_t c = 0; c < n_keys; ++c)
    if (keys[c] < 0 || keys[c] >= cu_k[batch]) bad = 1;
  if (bad) {
    free(seq);
    free(pos);
    return 1;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t c = 0; c < n_keys; ++c) {
    int b = 0;
    while (b + 1 < batch && cu_k[b + 1] <= keys[c]) ++b;
    const int64_t s = keys[c] - cu_k[b];
    const double* key = kI + keys[c] * d;
    double* out = dk + c * d;
    for (int j = 0; j < d; ++j) out[j] = 0.0;
    for (int64_t i = 0; i < n_rows; ++i) {
      if (seq[i] != b || s > pos[i]) continue;
      const double g = Gk[i * n_keys + c];
      const double* q = q_rows + i * (int64_t)n_heads * d;
      for (int h = 0; h < n_heads; ++h) {
        double x = 0.0;
        for (int j = 0; j < d; ++j) x += q[h * d + j] * key[j];
        if (x > 0.0) {
          const double coef = g * (double)w[rows[i] * n_heads + h];
          for (int j = 0; j < d; ++j) out[j] += coef * q[h * d + j];
        }
      }
    }
  }
  free(seq);
  free(pos);
  return 0;
}
