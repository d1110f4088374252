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

// Per-row top-k; rows of the window in [row_begin, row_begin + row_count).
hipError_t launch_topk(const dsa_varlen& vl, const float* scores, int64_t ld, int64_t row_begin,
                       int64_t row_count, int k, int32_t* indices, hipStream_t stream);

// Attention over selected positions.  splits > 1 writes per-split partial
// results to `partial` and merges them in a second kernel (decode).
size_t attn_workspace_bytes(int64_t rows, int n_heads_q, int head_dim, int splits);
int attn_decode_splits(int64_t rows, int n_heads_kv, int topk);

hipError_t launch_sparse_attn(const dsa_varlen& vl, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const int32_t* indices, int topk,
                              int64_t row_begin, int64_t row_count, int n_heads_q, int n_heads_kv,
                              int head_dim, float scale, uint16_t* out, float* lse, int splits,
                              float* partial, hipStream_t stream);

}  // namespace dsa
