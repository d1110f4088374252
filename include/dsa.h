/*
 * dsa.h -- C ABI of libdsa.so: the DeepSeek Sparse Attention (DSA) hot path
 * on AMD Instinct MI355X (gfx950).
 *
 * Method (Kwai Keye-VL-2.0 technical-report summary, page 5, section 1, the
 * paragraphs on the Lightning Indexer and on the GQA adaptation):
 *   1. a lightweight indexer scores every visible position of the context for
 *      the current query token, using ONE key per position shared by all of
 *      its heads (an MQA design);
 *   2. the k best positions (k = 2048 on the pages) are kept for that token;
 *   3. attention runs only over the kept positions, so its cost is O(L k)
 *      instead of O(L^2); one index set serves every GQA query head.
 * Page 5 section 8 requires the top-k to be deterministic, so training and
 * inference select the same positions.  Page 1 (the launch article) states
 * the DSA kernels run in variable-length (packed) mode; every call here takes
 * a packed batch.
 *
 * Indexer score used here (the pages print no formula):
 *   I[t, s] = sum_h w[t, h] * max(0, qI[t, h, :] . kI[s, :]).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers into caller-owned, contiguous,
 *     row-major buffers.  The library never allocates, frees, copies or
 *     synchronises; it only enqueues kernels on `stream`.  The one
 *     exception is the opt-in device-side checking described below.
 *   - bf16 tensors are IEEE binary32 values truncated to their upper 16 bits
 *     (torch.bfloat16), passed as `const void*`, 16-byte aligned.
 *   - Calls are stateless and may be made from any host thread.
 *   - Return value: DSA_OK when all work was enqueued; otherwise an error
 *     code and nothing was enqueued.  dsa_last_error() gives a message for
 *     the calling thread's most recent failure.  Faults during execution
 *     surface as HIP errors on the caller's next synchronisation.
 *   - Validation is host-side (pointers, sizes, shapes).  Device-resident
 *     metadata (cu_seqlens, index values, scores) is a precondition, not
 *     checked by default: cu_seqlens must start at 0, be non-decreasing with
 *     Lq_b <= Lk_b, stay within max_seqlen_q / max_seqlen_k and end at
 *     total_q / total_k; scores must be finite; an index list holds each
 *     position at most once.  Indices outside 0..p are treated as empty
 *     slots by the attention kernels.
 *   - Device-side checking (opt-in): with the environment variable DSA_CHECK
 *     set to anything but "" or "0" (read at every call), each entry point
 *     first runs the matching dsa_check_* call below on its own inputs and
 *     returns its status without enqueueing the real work when it fails.
 *     Checked calls wait for `stream` (so they cannot be captured into a
 *     graph), and the first one on a device allocates a 256-byte report
 *     buffer that lives until the process ends.  Checks share that buffer,
 *     so checked calls from several host threads run one after another.
 *     The attention entry points check their index lists with their own
 *     reading (an entry outside 0..p is an empty slot; a position listed
 *     twice is an error), so a call that is valid unchecked stays valid
 *     checked.
 *
 * Varlen layout (dsa_varlen)
 *   Sequence b owns packed query rows [cu_seqlens_q[b], cu_seqlens_q[b+1])
 *   and packed key rows [cu_seqlens_k[b], cu_seqlens_k[b+1]).  Local query
 *   i of sequence b sits at position p = Lk_b - Lq_b + i and sees local keys
 *   0..p (itself included).  Prefill has Lq_b = Lk_b; decode has Lq_b = 1 and
 *   p = Lk_b - 1 (the new token's key is already in the caches).  Indices are
 *   int32 sequence-local positions.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size or window */
  DSA_ERR_UNSUPPORTED = 2,      /* a shape outside the supported set below   */
  DSA_ERR_WORKSPACE = 3,        /* workspace missing or too small             */
  DSA_ERR_HIP = 4               /* a HIP launch call failed                   */
} dsa_status;

/* softmax_scale value that selects the default scale 1 / sqrt(head_dim) in
   the attention and warm-up-loss entry points (a scale of exactly zero has no
   use: it would make every selected position equally likely). */
#define DSA_SCALE_DEFAULT 0.0f

/* Static text for a status code. */
const char* dsa_status_string(int status);
/* Message describing the calling thread's most recent failed call ("" if none). */
const char* dsa_last_error(void);

/* Packed (varlen) batch description.  The two cu_seqlens arrays live on the
   device; the scalar fields are host copies the caller keeps consistent. */
typedef struct {
  int32_t batch;                /* number of sequences B >= 1                 */
  const int32_t* cu_seqlens_q;  /* device int32 [B+1], cu_seqlens_q[0] == 0   */
  const int32_t* cu_seqlens_k;  /* device int32 [B+1], cu_seqlens_k[0] == 0   */
  int64_t total_q;              /* == cu_seqlens_q[B]                         */
  int64_t total_k;              /* == cu_seqlens_k[B]                         */
  int32_t max_seqlen_q;         /* max_b Lq_b                                 */
  int32_t max_seqlen_k;         /* max_b Lk_b                                 */
} dsa_varlen;

/*
 * dsa_index_scores -- Lightning-Indexer scores for a window of query rows
 * (page 5 section 1: the scout scores every position; one MQA key per
 * position serves all indexer heads).
 *
 *   q_idx  bf16 [total_q, n_heads_idx, d_idx]   indexer queries
 *   k_idx  bf16 [total_k, d_idx]                one indexer key per position
 *   w      fp32 [total_q, n_heads_idx]          per-head weights (any sign)
 *   rows   packed query rows row_begin .. row_begin + row_count - 1
 *   scores fp32 [row_count, ld_scores]: scores[i, s] = I[row_begin + i, s] for
 *          s = 0..p of that row; columns beyond p are left untouched.
 *
 * Arithmetic: bf16 x bf16 products accumulated in fp32 (MFMA), the ReLU,
 * weighting and head sum in fp32.  Integer-valued inputs whose partial sums
 * stay below 2^24 give exact scores.
 * Supported: d_idx in {64, 128}; 1 <= n_heads_idx <= 64; one sequence's keys
 * at most 2 GiB (max_seqlen_k * d_idx * 2 < 2^31).
 * Invalid: null pointers, misaligned bf16 pointers, scores not 16-byte
 * aligned, ld_scores < max_seqlen_k or not a multiple of 4, a window outside
 * [0, total_q).  row_count == 0 is a no-op.
 */
int dsa_index_scores(const dsa_varlen* vl, const void* q_idx, const void* k_idx, const float* w,
                     int32_t n_heads_idx, int32_t d_idx, int64_t row_begin, int64_t row_count,
                     float* scores, int64_t ld_scores, hipStream_t stream);

/*
 * FP8 indexer inputs.  The pages state no indexer precision; this optional
 * variant holds indexer queries and keys as 8-bit floats (OCP E4M3,
 * "e4m3fn": bias 7, 3 mantissa bits, largest magnitude 448, no infinities)
 * with one binary32 scale per vector of d_idx values:
 *   x_j  ~  scale * value(c_j),   scale = amax / 448,   amax = max_j |x_j|.
 *
 * dsa_quantize_fp8 -- x bf16 [rows, dim] -> codes uint8 [rows, dim] and
 *   scales fp32 [rows]; every step binary32: inv = 448 / amax (correctly
 *   rounded), c_j = value x_j * inv rounded to the nearest e4m3 value, ties to
 *   even, saturating at +-448; scale = amax / 448.  A row of zeros gets codes 0
 *   and scale 0.  Inputs must be finite.  Supported: dim in {64, 128}.
 *   Invalid: null pointers, x not 16-byte aligned, codes not 16-byte aligned,
 *   rows < 0.  Queries are quantised per head: x = q_idx viewed as
 *   [total_q * n_heads_idx, d_idx].
 *
 * dsa_index_scores_fp8 -- the indexer score of dsa_index_scores on the values
 *   the codes represent:
 *     q_codes uint8 [total_q, n_heads_idx, d_idx],  q_scales fp32 [total_q, n_heads_idx]
 *     k_codes uint8 [total_k, d_idx],               k_scales fp32 [total_k]
 *     I[t, s] = k_scale[s] * sum_h (w[t,h] q_scale[t,h]) max(0, codes_q[t,h] . codes_k[s])
 *   (equal to the plain definition because scales are non-negative).  Code
 *   products are exact; the MFMA sums them in fp32; the weighting and head
 *   sum are fp32.  Window, scores layout, support and errors as
 *   dsa_index_scores, with code pointers 16-byte aligned and scale pointers
 *   4-byte aligned; one sequence's key codes at most 2 GiB.
 */
int dsa_quantize_fp8(const void* x, int64_t rows, int32_t dim, uint8_t* codes, float* scales,
                     hipStream_t stream);
int dsa_index_scores_fp8(const dsa_varlen* vl, const uint8_t* q_codes, const float* q_scales,
                         const uint8_t* k_codes, const float* k_scales, const float* w,
                         int32_t n_heads_idx, int32_t d_idx, int64_t row_begin, int64_t row_count,
                         float* scores, int64_t ld_scores, hipStream_t stream);

/* Workspace bytes dsa_topk needs for this call shape (0: it needs none). */
int dsa_topk_workspace_size(const dsa_varlen* vl, int64_t row_count, int32_t k, size_t* bytes);

/*
 * dsa_topk -- deterministic per-row top-k of indexer scores (page 5 section 1:
 * the k most relevant positions per query token; section 8: deterministic).
 *
 *   scores  fp32 [row_count, ld_scores] as written by dsa_index_scores; only
 *           columns 0..p of each row are read.  Values must be finite;
 *           -0.0 and +0.0 are equal.
 *   indices int32 [row_count, k]: the n = min(k, p + 1) positions with the
 *           largest score, ties broken towards the LOWER position, written in
 *           ascending position order; slots n..k-1 are -1.
 *
 * The result is a pure function of the inputs (bitwise repeatable).
 * Supported: 1 <= k <= 2048.
 * Invalid: null pointers, scores not 16-byte aligned, ld_scores <
 * max_seqlen_k or not a multiple of 4, a window outside [0, total_q).
 * workspace may be NULL when dsa_topk_workspace_size reports 0 (it always
 * does today; the argument keeps room for call shapes that will need one).
 */
int dsa_topk(const dsa_varlen* vl, const float* scores, int64_t ld_scores, int64_t row_begin,
             int64_t row_count, int32_t k, int32_t* indices, void* workspace,
             size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes dsa_index_topk needs for a window of row_count rows. */
int dsa_index_topk_workspace_size(const dsa_varlen* vl, int64_t row_count, int32_t k,
                                  size_t* bytes);

/*
 * dsa_index_topk -- dsa_index_scores followed by dsa_topk, fused: the k best
 * positions of every window row by indexer score (page 5 section 1: the
 * scout scores every position and the k best are kept; section 8: the
 * selection is deterministic) without writing the row's scores out.
 *
 *   q_idx, k_idx, w, n_heads_idx, d_idx, row window: as dsa_index_scores
 *   indices   int32 [row_count, k]: exactly what dsa_index_scores ->
 *             dsa_topk write for the same inputs (bitwise: the scores are
 *             computed by the same kernel arithmetic and the same tie rule
 *             selects among them).
 *   workspace device buffer of at least dsa_index_topk_workspace_size bytes,
 *             256-byte aligned, contents clobbered; calls sharing it must be
 *             ordered.  After the call, its first row_count uint32 words are
 *             the rows' candidate counts, and row_count words starting at
 *             byte offset 256 * ceil(4 * row_count / 256) are 1 for rows
 *             that took the exact fallback below, else 0 (diagnostics).
 *
 * How: a sample pass scores every S-th key of each row (S = 64, or more for
 * rows beyond 262144 keys) and reads off a per-row threshold that about
 * 5120 scores of the row are expected to reach; the indexer then keeps only
 * the scores at or above it, as (score, position) candidates, and an exact
 * top-k runs over those.  When a row has fewer than k candidates, or more
 * than its list holds (10240), its scores are recomputed and selected the
 * unfused way, so the result never depends on the estimate.  Rows of at most
 * 10240 positions keep every score as a candidate.
 * Supported / invalid: as dsa_index_scores and dsa_topk (1 <= k <= 2048).
 */
int dsa_index_topk(const dsa_varlen* vl, const void* q_idx, const void* k_idx, const float* w,
                   int32_t n_heads_idx, int32_t d_idx, int64_t row_begin, int64_t row_count,
                   int32_t k, int32_t* indices, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * dsa_sparse_attn_prefill -- GQA softmax attention of each query row over its
 * selected positions only (page 5 section 1: attention among the chosen
 * positions, O(L k); GQA adaptation: one index set per token for all heads).
 *
 *   q       bf16 [total_q, n_heads_q, head_dim]
 *   k, v    bf16 [total_k, n_heads_kv, head_dim]
 *   indices int32 [row_count, topk]: row i belongs to packed query row
 *           row_begin + i; entries outside 0..p are empty slots.
 *   out     bf16 [total_q, n_heads_q, head_dim]; rows of the window written.
 *   lse     fp32 [total_q, n_heads_q] natural-log log-sum-exp of the scaled
 *           logits, or NULL.  A row with no valid index gets out = 0 and
 *           lse = -inf.
 * Query head h reads KV head h / (n_heads_q / n_heads_kv).
 *   O[h] = sum_s softmax_s(softmax_scale * q[h] . k[s, g]) v[s, g].
 * softmax_scale: DSA_SCALE_DEFAULT (0) selects 1 / sqrt(head_dim).
 * Arithmetic: bf16 MFMA with fp32 accumulation, fp32 softmax, probabilities
 * rounded to bf16 for the value product, bf16 output (round to nearest even).
 * Supported: head_dim in {64, 128}; n_heads_q / n_heads_kv in 1..16;
 * n_heads_kv in 1..8; 1 <= topk <= 4096; one sequence's K (and V) rows at
 * most 2 GiB, i.e. max_seqlen_k * n_heads_kv * head_dim * 2 < 2^31 (the
 * kernels address a sequence with 32-bit byte offsets).
 * Invalid: null pointers, misaligned bf16 pointers, n_heads_q % n_heads_kv,
 * a window outside [0, total_q), non-finite softmax_scale.
 */
int dsa_sparse_attn_prefill(const dsa_varlen* vl, const void* q, const void* k, const void* v,
                            const int32_t* indices, int32_t topk, int64_t row_begin,
                            int64_t row_count, int32_t n_heads_q, int32_t n_heads_kv,
                            int32_t head_dim, float softmax_scale, void* out, float* lse,
                            hipStream_t stream);

/*
 * dsa_indexer_kl -- the indexer's warm-up loss and its gradient with respect
 * to the indexer scores (page 5 section 1, the two training stages: in the
 * dense warm-up only the indexer is trained, so that its distribution over
 * positions approaches the full attention's, the gap measured by KL
 * divergence).  For window row t at position p, keys s = 0..p, G = Hq / Hkv:
 *   A_h[s]    = softmax_s(softmax_scale * q[t,h] . k[s, h / G])  dense attention of head h
 *   P[s]      = (1 / n_heads_q) sum_h A_h[s]                    the target, heads averaged
 *   Pi[s]     = softmax_s(scores[t, s])                         the indexer's distribution
 *   loss[t]   = sum_s P[s] (ln P[s] - ln Pi[s])                 KL(P || Pi), natural log
 *   grad[t,s] = Pi[s] - P[s]                                    d loss[t] / d scores[t, s]
 *
 *   q       bf16 [total_q, n_heads_q, head_dim]; k bf16 [total_k, n_heads_kv, head_dim]
 *   scores  fp32 [row_count, ld_scores]: the window's indexer scores as
 *           dsa_index_scores writes them (columns 0..p read), 16-byte aligned
 *   loss    fp32 [row_count], one value per window row (caller sums or averages)
 *   grad    fp32 [row_count, ld_grad] or NULL; columns 0..p written, others
 *           untouched.  grad == scores (with ld_grad == ld_scores) overwrites
 *           the scores in place.
 * Arithmetic: bf16 products with fp32 accumulation (MFMA), fp32 softmax
 * statistics; every dense logit is computed twice (statistics, then P).
 * softmax_scale: DSA_SCALE_DEFAULT (0) selects 1 / sqrt(head_dim).
 * Supported: head_dim in {64, 128}, n_heads_q in {1, 2, 4, ..., 64},
 * n_heads_kv <= 8 dividing it, softmax_scale > 0 (after the default is
 * applied), one sequence's K rows within 2 GiB.
 * Invalid: null q, k, scores or loss, misaligned pointers, ld_scores or
 * ld_grad < max_seqlen_k, ld_scores not a multiple of 4, a window outside
 * [0, total_q), grad == scores with ld_grad != ld_scores, non-finite scale.
 * Under DSA_CHECK the scores of the window are checked to be finite first.
 */
int dsa_indexer_kl(const dsa_varlen* vl, const void* q, const void* k, const float* scores,
                   int64_t ld_scores, int64_t row_begin, int64_t row_count, int32_t n_heads_q,
                   int32_t n_heads_kv, int32_t head_dim, float softmax_scale, float* loss,
                   float* grad, int64_t ld_grad, hipStream_t stream);

/*
 * dsa_index_scores_backward -- gradient of the indexer score with respect to
 * the indexer's own inputs (page 5 section 1, the two training stages: in
 * the dense warm-up only the indexer is trained, so the warm-up loss's
 * gradient has to reach its queries, keys and head weights).  For window
 * row t at position p, keys s = 0..p, x[t,h,s] = q_idx[t,h,:] . k_idx[s,:]
 * and G = grad = d loss / d I (as dsa_indexer_kl writes it, or any other
 * upstream gradient), taking the ReLU's derivative as 1 for x > 0 and 0
 * otherwise:
 *   dw[t,h]       = sum_s G[t,s] max(0, x[t,h,s])                   written
 *   dq_idx[t,h,:] = w[t,h] sum_{s: x > 0} G[t,s] k_idx[s,:]          written
 *   dk_idx[s,:]  += sum_t sum_{h: x > 0} G[t,s] w[t,h] q_idx[t,h,:]   added
 *
 *   q_idx, k_idx, w, n_heads_idx, d_idx, window: as dsa_index_scores
 *   grad    fp32 [row_count, ld_grad]; columns 0..p of each row read
 *   dq_idx  fp32 [row_count, n_heads_idx, d_idx], or NULL together with dw
 *   dw      fp32 [row_count, n_heads_idx], or NULL together with dq_idx
 *   dk_idx  fp32 [total_k, d_idx] or NULL: the window's contribution is
 *           added, so the windows of one pass sum into it (the caller zeroes
 *           it first; calls adding to one dk_idx must run in stream order)
 *   workspace  device memory of dsa_index_scores_backward_workspace_size
 *           bytes (for the outputs requested), 256-byte aligned; it holds the
 *           transposed keys (dq) and the window's weighted, transposed
 *           queries (dk) and is free again when the call's work is done.
 * Arithmetic: x recomputed as dsa_index_scores computes it (bf16 MFMA, fp32
 * accumulation); the dq and dk products take G [x > 0] and, for dk,
 * w q_idx rounded to bf16 (nearest even) as MFMA operands with fp32
 * accumulation; dw is q_idx[t,h,:] dotted (fp32) with the dq sum before the
 * weight, which equals sum_s G relu(x) since relu(x) = [x > 0] x.
 * Supported: as dsa_index_scores, and one sequence's dk_idx rows within
 * 2 GiB (max_seqlen_k * d_idx * 4 < 2^31).
 * Invalid: null inputs, misaligned pointers (bf16 inputs 16-byte, fp32
 * 4-byte), ld_grad < max_seqlen_k, dq_idx without dw or the reverse, no
 * output at all, a window outside [0, total_q); a missing, short or
 * misaligned workspace gives DSA_ERR_WORKSPACE.  row_count == 0 is a no-op.
 */
int dsa_index_scores_backward_workspace_size(const dsa_varlen* vl, int32_t n_heads_idx,
                                             int32_t d_idx, int64_t row_count, int want_dq,
                                             int want_dk, size_t* bytes);
int dsa_index_scores_backward(const dsa_varlen* vl, const void* q_idx, const void* k_idx,
                              const float* w, int32_t n_heads_idx, int32_t d_idx,
                              int64_t row_begin, int64_t row_count, const float* grad,
                              int64_t ld_grad, float* dq_idx, float* dw, float* dk_idx,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes dsa_sparse_attn_prefill_grouped needs for a window of
   row_count rows (the unions of up to ceil(row_count / 16) groups). */
int dsa_sparse_attn_prefill_grouped_workspace_size(const dsa_varlen* vl, int64_t row_count,
                                                   int32_t topk, size_t* bytes);

/*
 * dsa_sparse_attn_prefill_grouped -- the attention of dsa_sparse_attn_prefill
 * computed for groups of 16 adjacent query rows at once (page 5 section 8:
 * adjacent queries select largely the same positions, so the 16 index sets
 * are de-duplicated before attention).  Rows row_begin + 16 j .. + 15 form
 * group j; the union of their index rows is gathered once per group and a
 * per-(row, position) mask keeps every query to its own set, so the result
 * is that of dsa_sparse_attn_prefill on the same indices (same arithmetic per
 * query; the group may span sequences).  Pays off when the sets overlap: the
 * K/V rows gathered per group are the union's, and the union is ordered so
 * that each 32-entry tile is computed only for the query heads of the rows
 * that own one of its entries.
 *
 *   q, k, v, out, lse, softmax_scale, window: as dsa_sparse_attn_prefill.
 *   indices int32 [row_count, topk]: every row's selected positions in any
 *           order, no position twice in a row; entries outside 0..p (-1
 *           padding included) are skipped, as in dsa_sparse_attn_prefill.
 *   workspace  device buffer of at least
 *              dsa_sparse_attn_prefill_grouped_workspace_size bytes for this
 *              row_count and topk, 256-byte aligned, contents clobbered; calls
 *              sharing it must be ordered.
 * Supported: as dsa_sparse_attn_prefill with n_heads_q / n_heads_kv in
 * {1, 2, 4, 8}, plus all K (and V) rows at most 2 GiB
 * (total_k * n_heads_kv * head_dim * 2 < 2^31).
 */
int dsa_sparse_attn_prefill_grouped(const dsa_varlen* vl, const void* q, const void* k,
                                    const void* v, const int32_t* indices, int32_t topk,
                                    int64_t row_begin, int64_t row_count, int32_t n_heads_q,
                                    int32_t n_heads_kv, int32_t head_dim, float softmax_scale,
                                    void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes dsa_sparse_attn_decode needs for a window of row_count
   queries (partial results of the split over the index list). */
int dsa_sparse_attn_decode_workspace_size(const dsa_varlen* vl, int64_t row_count,
                                          int32_t n_heads_q, int32_t head_dim, int32_t topk,
                                          size_t* bytes);

/*
 * dsa_sparse_attn_decode -- the same attention for one new token per
 * sequence (Lq_b == 1, p = Lk_b - 1) reading bf16 KV caches (page 5 section 8
 * names a DSA-specific decode optimisation without describing it; here the
 * index list of each query is split across workgroups and the partial results
 * are merged in a fixed order, so the output is bitwise repeatable).
 *
 *   q        bf16 [batch, n_heads_q, head_dim]
 *   k_cache, v_cache  bf16 [total_k, n_heads_kv, head_dim]
 *   rows     queries row_begin .. row_begin + row_count - 1 of the batch
 *   indices  int32 [row_count, topk]: row i belongs to query row_begin + i
 *   out      bf16 [batch, n_heads_q, head_dim];  lse fp32 [batch, n_heads_q] or
 *            NULL; rows of the window written.
 *   workspace  device buffer of at least dsa_sparse_attn_decode_workspace_size
 *              bytes for this row_count, 256-byte aligned; its contents need
 *              not be initialised and are clobbered.  Calls sharing one
 *              workspace must be ordered; calls on disjoint windows with
 *              disjoint workspaces may run concurrently on different streams.
 * Supported / invalid: as dsa_sparse_attn_prefill, plus total_q == batch.
 */
int dsa_sparse_attn_decode(const dsa_varlen* vl, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* indices, int32_t topk,
                           int64_t row_begin, int64_t row_count, int32_t n_heads_q,
                           int32_t n_heads_kv, int32_t head_dim, float softmax_scale, void* out,
                           float* lse, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * dsa_sparse_attn_decode_noalloc -- dsa_sparse_attn_decode without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under graph capture, serving loops or harnesses that forbid hipMalloc).
 * The split partials live in a fixed 16 MiB device array inside the library
 * (one per GPU, held until the process ends; its address is looked up on the
 * first call on each device).  The call allocates nothing and is otherwise
 * identical to dsa_sparse_attn_decode: same kernels, same split of the index
 * list, bitwise the same results.
 *
 * Limit: the partials, row_count * splits * n_heads_q * (head_dim + 2) * 4
 * bytes, must fit the 16 MiB (every shape with n_heads_q * (head_dim + 2) <=
 * 8192, i.e. up to 63 query heads at head_dim 128); larger calls return
 * DSA_ERR_UNSUPPORTED before enqueueing anything.
 * Every call on one GPU shares that GPU's array and leaves its partials in
 * it; nothing in it needs to start at zero.  Calls that overlap in time on
 * one GPU (different streams or host threads) race on the array and must be
 * ordered by the caller.
 */
int dsa_sparse_attn_decode_noalloc(const dsa_varlen* vl, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* indices, int32_t topk,
                                   int64_t row_begin, int64_t row_count, int32_t n_heads_q,
                                   int32_t n_heads_kv, int32_t head_dim, float softmax_scale,
                                   void* out, float* lse, hipStream_t stream);

/*
 * Device-side precondition checks (debugging aid; see the conventions above).
 * Each validates its arguments on the host like the entry points, runs one
 * or two small kernels on `stream`, waits for the stream (and so for all
 * work enqueued before it) and returns DSA_OK, or DSA_ERR_INVALID_ARGUMENT
 * with dsa_last_error() naming the first offending sequence or row, or
 * DSA_ERR_HIP.  They read only the arguments they name.
 *
 * dsa_check_varlen   cu_seqlens_q / cu_seqlens_k against the descriptor:
 *                    both start at 0, never decrease, Lq_b <= Lk_b,
 *                    Lq_b <= max_seqlen_q, Lk_b <= max_seqlen_k, and they end
 *                    at total_q / total_k.
 * dsa_check_indices  the varlen check, then every row of an index list
 *                    int32 [row_count, topk] for query rows row_begin ..:
 *                    each entry is -1 or a causal position 0..p, and no
 *                    position appears twice (the selected set is causal and
 *                    unique, page 5 section 1).
 * dsa_check_scores   the varlen check, then columns 0..p of every row of
 *                    fp32 scores [row_count, ld_scores] are finite.
 */
int dsa_check_varlen(const dsa_varlen* vl, hipStream_t stream);
int dsa_check_indices(const dsa_varlen* vl, const int32_t* indices, int32_t topk,
                      int64_t row_begin, int64_t row_count, hipStream_t stream);
int dsa_check_scores(const dsa_varlen* vl, const float* scores, int64_t ld_scores,
                     int64_t row_begin, int64_t row_count, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
