// dsa_internal.h -- host-side launchers behind the C ABI (validated inputs only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

hipError_t launch_index_scores(const dsa_varlen& vl, const uint16_t* q_idx, const uint16_t* k_idx,
                               const float* w, int n_heads, int d, int64_t row_begin,
                               int64_t row_count, float* scores, int64_t ld, hipStream_t stream);

// Where one indexer launch sends its scores (rows are window-local).
// Score mode writes rows of `scores`; key j of a row is position
// j * key_stride (1 but for sampling every key_stride-th key).  Candidate
// mode (key_stride 1) keeps only the scores >= tau[row] and appends them as
// (score bits, position) to the row's list of `cap` entries, counting every
// survivor in count[row] (a count above cap means entries were dropped; the
// stream kernel adds to count, which must start at zero).
struct IndexOut {
  float* scores = nullptr;
  int64_t ld = 0;
  int32_t key_stride = 1;
  const float* tau = nullptr;
  uint32_t* count = nullptr;
  uint2* cand = nullptr;
  int32_t cap = 0;
};
hipError_t launch_index_scores_to(const dsa_varlen& vl, const uint16_t* q_idx,
                                  const uint16_t* k_idx, const float* w, int n_heads, int d,
                                  int64_t row_begin, int64_t row_count, const IndexOut& out,
                                  bool candidates, hipStream_t stream);

// Fused indexer -> top-k over a window (the indexer keeps only candidates
// above a per-row threshold read off a sample of the row's scores; rows it
// cannot settle exactly are recomputed unfused).  `workspace` as sized by
// index_topk_workspace_bytes; it starts with the rows' candidate counts,
// then (256-byte aligned) their fallback flags.
size_t index_topk_workspace_bytes(const dsa_varlen& vl, int64_t row_count, int k);
hipError_t launch_index_topk(const dsa_varlen& vl, const uint16_t* q_idx, const uint16_t* k_idx,
                             const float* w, int n_heads, int d, int64_t row_begin,
                             int64_t row_count, int k, int32_t* indices, void* workspace,
                             hipStream_t stream);

// Indexer scores from fp8 (e4m3) codes with one scale per query head and
// per key.
hipError_t launch_index_scores_fp8(const dsa_varlen& vl, const uint8_t* q8, const float* q_scale,
                                   const uint8_t* k8, const float* k_scale, const float* w,
                                   int n_heads, int d, int64_t row_begin, int64_t row_count,
                                   float* scores, int64_t ld, hipStream_t stream);

// bf16 vectors of d values -> e4m3 codes and one binary32 scale per vector.
hipError_t launch_quantize_fp8(const uint16_t* x, int64_t rows, int d, uint8_t* codes,
                               float* scales, hipStream_t stream);

// Per-row top-k; rows of the window in [row_begin, row_begin + row_count).
hipError_t launch_topk(const dsa_varlen& vl, const float* scores, int64_t ld, int64_t row_begin,
                       int64_t row_count, int k, int32_t* indices, hipStream_t stream);

// Attention over selected positions.  splits > 1 writes per-split partial
// results to `partial` and merges them in a second kernel (decode).
size_t attn_workspace_bytes(int64_t rows, int n_heads_q, int head_dim, int splits);
int attn_decode_splits(int64_t rows, int n_heads_kv, int topk);

// The decode partials' fixed device scratch (the entry point that allocates
// nothing): its size, and its address on the current device (looked up on
// the first call per device).
size_t attn_scratch_bytes();
hipError_t attn_scratch(float** ptr);

hipError_t launch_sparse_attn(const dsa_varlen& vl, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const int32_t* indices, int topk,
                              int64_t row_begin, int64_t row_count, int n_heads_q, int n_heads_kv,
                              int head_dim, float scale, uint16_t* out, float* lse, int splits,
                              float* partial, hipStream_t stream);

// Grouped prefill attention: 16 adjacent rows served from the union of their
// (ascending) index rows; `workspace` holds the unions.
size_t grouped_attn_workspace_bytes(int64_t row_count, int topk);
hipError_t launch_grouped_attn(const dsa_varlen& vl, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* indices, int topk,
                               int64_t row_begin, int64_t row_count, int n_heads_q,
                               int n_heads_kv, int head_dim, float scale, uint16_t* out,
                               float* lse, void* workspace, hipStream_t stream);

// Indexer warm-up loss per query row and its gradient with respect to the
// scores (grad may be null, or equal to scores with the same ld).
hipError_t launch_indexer_kl(const dsa_varlen& vl, const uint16_t* q, const uint16_t* k,
                             const float* scores, int64_t ld, int64_t row_begin,
                             int64_t row_count, int n_heads_q, int n_heads_kv, int head_dim,
                             float scale, float* loss, float* grad, int64_t ld_grad,
                             hipStream_t stream);

// Backward of the indexer score: dq and dw of the window's rows (written)
// and their contribution to dk (added); any of the two outputs may be
// skipped (dq and dw go together).  The workspace holds the transposed keys
// (for dq) and the window's transposed, weighted queries (for dk).
size_t index_backward_tiles_bytes(int64_t tiles, int d);
size_t index_backward_rows_bytes(int64_t row_count, int d, int hp);
size_t index_backward_workspace_bytes(const dsa_varlen& vl, int n_heads, int d, int64_t row_count,
                                      bool want_dq, bool want_dk);
hipError_t launch_index_backward(const dsa_varlen& vl, const uint16_t* q_idx,
                                 const uint16_t* k_idx, const float* w, int n_heads, int d,
                                 int64_t row_begin, int64_t row_count, const float* grad,
                                 int64_t ld, float* dq, float* dw, float* dk, void* workspace,
                                 hipStream_t stream);

// Device-side precondition checks.  Each clears a report word, runs one
// kernel on `stream`, waits for the stream and stores the first finding as
// (item << 8) | code, or all ones when there is none.  The first call on a
// device allocates its report word (kept until the process ends); checks
// are serialised by a lock held until their finding is read back.
enum CheckCode {
  kCheckOffsetStart = 1,         // cu_seqlens_q[0] or cu_seqlens_k[0] != 0
  kCheckOffsetOrder = 2,         // cu_seqlens decreases
  kCheckMoreQueriesThanKeys = 3, // Lq_b > Lk_b
  kCheckAboveMax = 4,            // Lq_b > max_seqlen_q or Lk_b > max_seqlen_k
  kCheckTotal = 5,               // cu_seqlens[B] != total
  kCheckIndexRange = 6,          // an entry neither -1 nor in 0..p
  kCheckIndexDuplicate = 7,      // a position listed twice in one row
  kCheckScoreNotFinite = 8,      // NaN or infinity among columns 0..p
};
constexpr unsigned long long kNoFinding = ~0ull;

hipError_t check_offsets(const dsa_varlen& vl, hipStream_t stream, unsigned long long* finding);
// Rows of the window; the offsets must already have passed check_offsets.
// empty_outside: entries outside 0..p are empty slots (the attention
// kernels' reading) rather than errors; repeats among 0..p are still errors.
hipError_t check_indices(const dsa_varlen& vl, const int32_t* indices, int topk,
                         int64_t row_begin, int64_t row_count, bool empty_outside,
                         hipStream_t stream, unsigned long long* finding);
hipError_t check_scores(const dsa_varlen& vl, const float* scores, int64_t ld, int64_t row_begin,
                        int64_t row_count, hipStream_t stream, unsigned long long* finding);

}  // namespace dsa
