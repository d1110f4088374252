// dsa_api.hip -- the C ABI of libdsa.so: host-side validation and launches.
// Behaviour of every entry point is specified in include/dsa.h.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>

#include "dsa.h"
#include "dsa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return DSA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_varlen(const dsa_varlen* vl) {
  if (vl == nullptr) return fail(DSA_ERR_INVALID_ARGUMENT, "varlen descriptor is NULL");
  if (vl->batch < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", vl->batch);
  if (vl->cu_seqlens_q == nullptr || vl->cu_seqlens_k == nullptr)
    return fail(DSA_ERR_INVALID_ARGUMENT, "cu_seqlens pointer is NULL");
  if (!aligned(vl->cu_seqlens_q, 4) || !aligned(vl->cu_seqlens_k, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "cu_seqlens pointers must be 4-byte aligned");
  if (vl->total_q < 0 || vl->total_k < 1)
    return fail(DSA_ERR_INVALID_ARGUMENT, "total_q must be >= 0 and total_k >= 1");
  if (vl->max_seqlen_q < 0 || vl->max_seqlen_k < 1)
    return fail(DSA_ERR_INVALID_ARGUMENT, "max_seqlen_k must be >= 1");
  if (vl->max_seqlen_k > vl->total_k || vl->max_seqlen_q > vl->total_q)
    return fail(DSA_ERR_INVALID_ARGUMENT, "max_seqlen exceeds the packed total");
  if (vl->total_q > INT32_MAX || vl->total_k > INT32_MAX)
    return fail(DSA_ERR_UNSUPPORTED, "packed totals must fit int32");
  return DSA_OK;
}

int check_window(const dsa_varlen* vl, int64_t row_begin, int64_t row_count) {
  if (row_begin < 0 || row_count < 0 || row_begin + row_count > vl->total_q)
    return fail(DSA_ERR_INVALID_ARGUMENT, "row window [%lld, %lld) outside [0, %lld)",
                (long long)row_begin, (long long)(row_begin + row_count), (long long)vl->total_q);
  if (row_count > INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "row_count must fit int32");
  return DSA_OK;
}

int check_scores(const dsa_varlen* vl, const float* scores, int64_t ld) {
  if (scores == nullptr) return fail(DSA_ERR_INVALID_ARGUMENT, "scores pointer is NULL");
  if (!aligned(scores, 16)) return fail(DSA_ERR_INVALID_ARGUMENT, "scores must be 16-byte aligned");
  if (ld < vl->max_seqlen_k)
    return fail(DSA_ERR_INVALID_ARGUMENT, "ld_scores (%lld) < max_seqlen_k (%d)", (long long)ld,
                vl->max_seqlen_k);
  if (ld % 4 != 0) return fail(DSA_ERR_INVALID_ARGUMENT, "ld_scores must be a multiple of 4");
  return DSA_OK;
}

int check_bf16(const void* p, const char* name) {
  if (p == nullptr) return fail(DSA_ERR_INVALID_ARGUMENT, "%s pointer is NULL", name);
  if (!aligned(p, 16)) return fail(DSA_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", name);
  return DSA_OK;
}

// DSA_SCALE_DEFAULT (0) selects the usual 1 / sqrt(head_dim).
float resolve_scale(float scale, int32_t head_dim) {
  return scale == 0.0f && head_dim > 0 ? 1.0f / std::sqrt(static_cast<float>(head_dim)) : scale;
}

int check_attn_shape(int32_t hq, int32_t hkv, int32_t d, int32_t topk, float scale) {
  if (hq < 1 || hkv < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "head counts must be >= 1");
  if (hq % hkv != 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "n_heads_q (%d) is not a multiple of n_heads_kv (%d)",
                hq, hkv);
  if (d != 64 && d != 128) return fail(DSA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", d);
  if (hkv > 8) return fail(DSA_ERR_UNSUPPORTED, "n_heads_kv %d > 8", hkv);
  if (hq / hkv > 16) return fail(DSA_ERR_UNSUPPORTED, "group size %d > 16", hq / hkv);
  if (topk < 1 || topk > 4096) return fail(DSA_ERR_UNSUPPORTED, "topk %d not in 1..4096", topk);
  if (!std::isfinite(scale)) return fail(DSA_ERR_INVALID_ARGUMENT, "softmax_scale is not finite");
  return DSA_OK;
}

// The attention kernels address one sequence's K or V rows with 32-bit
// byte offsets.
int check_attn_extent(const dsa_varlen* vl, int32_t hkv, int32_t d) {
  if (static_cast<int64_t>(vl->max_seqlen_k) * hkv * d * 2 > INT32_MAX)
    return fail(DSA_ERR_UNSUPPORTED, "one sequence's K or V rows exceed 2 GiB (max_seqlen_k %d)",
                vl->max_seqlen_k);
  return DSA_OK;
}

// The indexer kernels address one sequence's keys with 32-bit byte offsets.
int check_index_extent(const dsa_varlen* vl, int32_t d, int elem_bytes) {
  if (static_cast<int64_t>(vl->max_seqlen_k) * d * elem_bytes > INT32_MAX)
    return fail(DSA_ERR_UNSUPPORTED, "one sequence's indexer keys exceed 2 GiB (max_seqlen_k %d)",
                vl->max_seqlen_k);
  return DSA_OK;
}

int check_index_shape(int32_t n_heads_idx, int32_t d_idx) {
  if (d_idx != 64 && d_idx != 128) return fail(DSA_ERR_UNSUPPORTED, "d_idx %d not in {64, 128}", d_idx);
  if (n_heads_idx < 1 || n_heads_idx > 64)
    return fail(DSA_ERR_UNSUPPORTED, "n_heads_idx %d not in 1..64", n_heads_idx);
  return DSA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// DSA_CHECK set to anything but "" or "0" turns the device-side checks on
// in every entry point.  Read at each call, so a process may toggle it.
bool checks_enabled() {
  const char* e = std::getenv("DSA_CHECK");
  return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
}

int finding_status(hipError_t e, unsigned long long finding, int64_t row_begin) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "device check: %s", hipGetErrorString(e));
  if (finding == dsa::kNoFinding) return ok();
  const long long item = static_cast<long long>(finding >> 8);
  const long long row = static_cast<long long>(row_begin) + item;
  switch (static_cast<int>(finding & 0xff)) {
    case dsa::kCheckOffsetStart:
      return fail(DSA_ERR_INVALID_ARGUMENT, "cu_seqlens_q[0] and cu_seqlens_k[0] must be 0");
    case dsa::kCheckOffsetOrder:
      return fail(DSA_ERR_INVALID_ARGUMENT, "cu_seqlens decrease at sequence %lld", item);
    case dsa::kCheckMoreQueriesThanKeys:
      return fail(DSA_ERR_INVALID_ARGUMENT, "sequence %lld has more queries than keys", item);
    case dsa::kCheckAboveMax:
      return fail(DSA_ERR_INVALID_ARGUMENT,
                  "sequence %lld is longer than max_seqlen_q or max_seqlen_k", item);
    case dsa::kCheckTotal:
      return fail(DSA_ERR_INVALID_ARGUMENT,
                  "cu_seqlens_q[B] or cu_seqlens_k[B] differs from total_q or total_k");
    case dsa::kCheckIndexRange:
      return fail(DSA_ERR_INVALID_ARGUMENT, "row %lld: an index is neither -1 nor in 0..p", row);
    case dsa::kCheckIndexDuplicate:
      return fail(DSA_ERR_INVALID_ARGUMENT, "row %lld lists a position twice", row);
    case dsa::kCheckScoreNotFinite:
      return fail(DSA_ERR_INVALID_ARGUMENT, "row %lld: a score in columns 0..p is not finite",
                  row);
    default:
      return fail(DSA_ERR_HIP, "device check: unknown finding %llu", finding);
  }
}

int device_offsets(const dsa_varlen* vl, hipStream_t stream) {
  unsigned long long f = dsa::kNoFinding;
  const hipError_t e = dsa::check_offsets(*vl, stream, &f);
  return finding_status(e, f, 0);
}

// empty_outside: the attention entry points treat an index outside 0..p
// as an empty slot, so their checked calls accept it (dsa_check_indices
// itself holds lists to the -1-or-causal form dsa_topk writes).
int device_indices(const dsa_varlen* vl, const int32_t* indices, int32_t topk, int64_t row_begin,
                   int64_t row_count, hipStream_t stream, bool empty_outside) {
  int st;
  if ((st = device_offsets(vl, stream))) return st;
  if (row_count == 0) return ok();
  unsigned long long f = dsa::kNoFinding;
  const hipError_t e =
      dsa::check_indices(*vl, indices, topk, row_begin, row_count, empty_outside, stream, &f);
  return finding_status(e, f, row_begin);
}

int device_scores(const dsa_varlen* vl, const float* scores, int64_t ld, int64_t row_begin,
                  int64_t row_count, hipStream_t stream) {
  int st;
  if ((st = device_offsets(vl, stream))) return st;
  if (row_count == 0) return ok();
  unsigned long long f = dsa::kNoFinding;
  const hipError_t e = dsa::check_scores(*vl, scores, ld, row_begin, row_count, stream, &f);
  return finding_status(e, f, row_begin);
}

}  // namespace

extern "C" {

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARGUMENT: return "DSA_ERR_INVALID_ARGUMENT";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
    default: return "DSA_ERR_UNKNOWN";
  }
}

const char* dsa_last_error(void) { return g_last_error; }

int dsa_index_scores(const dsa_varlen* vl, const void* q_idx, const void* k_idx, const float* w,
                     int32_t n_heads_idx, int32_t d_idx, int64_t row_begin, int64_t row_count,
                     float* scores, int64_t ld_scores, hipStream_t stream) {
  int st;
  if ((st = check_varlen(vl))) return st;
  if ((st = check_window(vl, row_begin, row_count))) return st;
  if ((st = check_bf16(q_idx, "q_idx"))) return st;
  if ((st = check_bf16(k_idx, "k_idx"))) return st;
  if (w == nullptr || !aligned(w, 4)) return fail(DSA_ERR_INVALID_ARGUMENT, "w is NULL or misaligned");
  if ((st = check_scores(vl, scores, ld_scores))) return st;
  if ((st = check_index_shape(n_heads_idx, d_idx))) return st;
  if ((st = check_index_extent(vl, d_idx, 2))) return st;
  if (checks_enabled() && (st = device_offsets(vl, stream))) return st;
  if (row_count == 0) return ok();
  return hip_status(dsa::launch_index_scores(*vl, static_cast<const uint16_t*>(q_idx),
                                             static_cast<const uint16_t*>(k_idx), w, n_heads_idx,
                                             d_idx, row_begin, row_count, scores, ld_scores, stream),
                    "index_scores launch");
}

int dsa_quantize_fp8(const void* x, int64_t rows, int32_t dim, uint8_t* codes, float* scales,
                     hipStream_t stream) {
  int st;
  if ((st = check_bf16(x, "x"))) return st;
  if (codes == nullptr || !aligned(codes, 16))
    return fail(DSA_ERR_INVALID_ARGUMENT, "codes is NULL or not 16-byte aligned");
  if (scales == nullptr || !aligned(scales, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "scales is NULL or misaligned");
  if (rows < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "rows < 0");
  if (dim != 64 && dim != 128) return fail(DSA_ERR_UNSUPPORTED, "dim %d not in {64, 128}", dim);
  if (rows == 0) return ok();
  return hip_status(dsa::launch_quantize_fp8(static_cast<const uint16_t*>(x), rows, dim, codes,
                                             scales, stream),
                    "quantize_fp8 launch");
}

int dsa_index_scores_fp8(const dsa_varlen* vl, const uint8_t* q_codes, const float* q_scales,
                         const uint8_t* k_codes, const float* k_scales, const float* w,
                         int32_t n_heads_idx, int32_t d_idx, int64_t row_begin, int64_t row_count,
                         float* scores, int64_t ld_scores, hipStream_t stream) {
  int st;
  if ((st = check_varlen(vl))) return st;
  if ((st = check_window(vl, row_begin, row_count))) return st;
  if (q_codes == nullptr || !aligned(q_codes, 16) || k_codes == nullptr || !aligned(k_codes, 16))
    return fail(DSA_ERR_INVALID_ARGUMENT, "q_codes / k_codes NULL or not 16-byte aligned");
  if (q_scales == nullptr || !aligned(q_scales, 4) || k_scales == nullptr || !aligned(k_scales, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "q_scales / k_scales NULL or misaligned");
  if (w == nullptr || !aligned(w, 4)) return fail(DSA_ERR_INVALID_ARGUMENT, "w is NULL or misaligned");
  if ((st = check_scores(vl, scores, ld_scores))) return st;
  if ((st = check_index_shape(n_heads_idx, d_idx))) return st;
  if ((st = check_index_extent(vl, d_idx, 1))) return st;
  if (checks_enabled() && (st = device_offsets(vl, stream))) return st;
  if (row_count == 0) return ok();
  return hip_status(dsa::launch_index_scores_fp8(*vl, q_codes, q_scales, k_codes, k_scales, w,
                                                 n_heads_idx, d_idx, row_begin, row_count, scores,
                                                 ld_scores, stream),
                    "index_scores_fp8 launch");
}

int dsa_topk_workspace_size(const dsa_varlen* vl, int64_t row_count, int32_t k, size_t* bytes) {
  int st;
  if ((st = check_varlen(vl))) return st;
  if (bytes == nullptr) return fail(DSA_ERR_INVALID_ARGUMENT, "bytes pointer is NULL");
  if (row_count < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "row_count < 0");
  if (k < 1 || k > 2048) return fail(DSA_ERR_UNSUPPORTED, "k %d not in 1..2048", k);
  *bytes = 0;
  return ok();
}

int dsa_topk(const dsa_varlen* vl, const float* scores, int64_t ld_scores, int64_t row_begin,
             int64_t row_count, int32_t k, int32_t* indices, void* workspace,
             size_t workspace_bytes, hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  int st;
  if ((st = check_varlen(vl))) return st;
  if ((st = check_window(vl, row_begin, row_count))) return st;
  if ((st = check_scores(vl, scores, ld_scores))) return st;
  if (indices == nullptr || !aligned(indices, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "indices is NULL or misaligned");
  if (k < 1 || k > 2048) return fail(DSA_ERR_UNSUPPORTED, "k %d not in 1..2048", k);
  if (checks_enabled() &&
      (st = device_scores(vl, scores, ld_scores, row_begin, row_count, stream)))
    return st;
  if (row_count == 0) return ok();
  return hip_status(dsa::launch_topk(*vl, scores, ld_scores, row_begin, row_count, k, indices, stream),
                    "topk launch");
}

int dsa_index_topk_workspace_size(const dsa_varlen* vl, int64_t row_count, int32_t k,
                                  size_t* bytes) {
  int st;
  if ((st = check_varlen(vl))) return st;
  if (bytes == nullptr) return fail(DSA_ERR_INVALID_ARGUMENT, "bytes pointer is NULL");
  if (row_count < 0 || row_count > vl->total_q)
    return fail(DSA_ERR_INVALID_ARGUMENT, "row_count %lld outside [0, total_q]",
                static_cast<long long>(row_count));
  if (k < 1 || k > 2048) return fail(DSA_ERR_UNSUPPORTED, "k %d not in 1..2048", k);
  *bytes = dsa::index_topk_workspace_bytes(*vl, row_count, k);
  return ok();
}

int dsa_index_topk(const dsa_varlen* vl, const void* q_idx, const void* k_idx, const float* w,
                   int32_t n_heads_idx, int32_t d_idx, int64_t row_begin, int64_t row_count,
                   int32_t k, int32_t* indices, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  int st;
  if ((st = check_varlen(vl))) return st;
  if ((st = check_window(vl, row_begin, row_count))) return st;
  if ((st = check_bf16(q_idx, "q_idx"))) return st;
  if ((st = check_bf16(k_idx, "k_idx"))) return st;
  if (w == nullptr || !aligned(w, 4)) return fail(DSA_ERR_INVALID_ARGUMENT, "w is NULL or misaligned");
  if (indices == nullptr || !aligned(indices, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "indices is NULL or misaligned");
  if ((st = check_index_shape(n_heads_idx, d_idx))) return st;
  if ((st = check_index_extent(vl, d_idx, 2))) return st;
  if (k < 1 || k > 2048) return fail(DSA_ERR_UNSUPPORTED, "k %d not in 1..2048", k);
  if (checks_enabled() && (st = device_offsets(vl, stream))) return st;
  if (row_count == 0) return ok();
  const size_t need = dsa::index_topk_workspace_bytes(*vl, row_count, k);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256))
    return fail(DSA_ERR_WORKSPACE, "index_topk workspace needs %zu bytes (256-byte aligned), got %zu",
                need, workspace_bytes);
  return hip_status(dsa::launch_index_topk(*vl, static_cast<const uint16_t*>(q_idx),
                                           static_cast<const uint16_t*>(k_idx), w, n_heads_idx,
                                           d_idx, row_begin, row_count, k, indices, workspace,
                                           stream),
                    "index_topk launch");
}

int dsa_sparse_attn_prefill(const dsa_varlen* vl, const void* q, const void* k, const void* v,
                            const int32_t* indices, int32_t topk, int64_t row_begin,
                            int64_t row_count, int32_t n_heads_q, int32_t n_heads_kv,
                            int32_t head_dim, float softmax_scale, void* out, float* lse,
                            hipStream_t stream) {
  softmax_scale = resolve_scale(softmax_scale, head_dim);
  int st;
  if ((st = check_varlen(vl))) return st;
  if ((st = check_window(vl, row_begin, row_count))) return st;
  if ((st = check_bf16(q, "q"))) return st;
  if ((st = check_bf16(k, "k"))) return st;
  if ((st = check_bf16(v, "v"))) return st;
  if ((st = check_bf16(out, "out"))) return st;
  if (indices == nullptr || !aligned(indices, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "indices is NULL or misaligned");
  if (lse != nullptr && !aligned(lse, 4)) return fail(DSA_ERR_INVALID_ARGUMENT, "lse misaligned");
  if ((st = check_attn_shape(n_heads_q, n_heads_kv, head_dim, topk, softmax_scale))) return st;
  if ((st = check_attn_extent(vl, n_heads_kv, head_dim))) return st;
  if (checks_enabled() &&
      (st = device_indices(vl, indices, topk, row_begin, row_count, stream, true)))
    return st;
  if (row_count == 0) return ok();
  return hip_status(
      dsa::launch_sparse_attn(*vl, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                              static_cast<const uint16_t*>(v), indices, topk, row_begin, row_count,
                              n_heads_q, n_heads_kv, head_dim, softmax_scale,
                              static_cast<uint16_t*>(out), lse, 1, nullptr, stream),
      "sparse_attn_prefill launch");
}

int dsa_sparse_attn_prefill_grouped_workspace_size(const dsa_varlen* vl, int64_t row_count,
                                                   int32_t topk, size_t* bytes) {
  int st;
  if ((st = check_varlen(vl))) return st;
  if (bytes == nullptr) return fail(DSA_ERR_INVALID_ARGUMENT, "bytes pointer is NULL");
  if (row_count < 0 || row_count > vl->total_q)
    return fail(DSA_ERR_INVALID_ARGUMENT, "row_count %lld outside [0, total_q]",
                static_cast<long long>(row_count));
  if (topk < 1 || topk > 4096) return fail(DSA_ERR_UNSUPPORTED, "topk %d not in 1..4096", topk);
  *bytes = row_count == 0 ? 0 : dsa::grouped_attn_workspace_bytes(row_count, topk);
  return ok();
}

int dsa_sparse_attn_prefill_grouped(const dsa_varlen* vl, const void* q, const void* k,
                                    const void* v, const int32_t* indices, int32_t topk,
                                    int64_t row_begin, int64_t row_count, int32_t n_heads_q,
                                    int32_t n_heads_kv, int32_t head_dim, float softmax_scale,
                                    void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  softmax_scale = resolve_scale(softmax_scale, head_dim);
  int st;
  if ((st = check_varlen(vl))) return st;
  if ((st = check_window(vl, row_begin, row_count))) return st;
  if ((st = check_bf16(q, "q"))) return st;
  if ((st = check_bf16(k, "k"))) return st;
  if ((st = check_bf16(v, "v"))) return st;
  if ((st = check_bf16(out, "out"))) return st;
  if (indices == nullptr || !aligned(indices, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "indices is NULL or misaligned");
  if (lse != nullptr && !aligned(lse, 4)) return fail(DSA_ERR_INVALID_ARGUMENT, "lse misaligned");
  if ((st = check_attn_shape(n_heads_q, n_heads_kv, head_dim, topk, softmax_scale))) return st;
  const int32_t group_heads = n_heads_q / n_heads_kv;
  if ((group_heads & (group_heads - 1)) != 0 || group_heads > 8)
    return fail(DSA_ERR_UNSUPPORTED, "n_heads_q / n_heads_kv = %d is not 1, 2, 4 or 8",
                group_heads);
  // The grouped kernels address all K (and V) rows with 32-bit offsets.
  if (vl->total_k * n_heads_kv * head_dim * 2 > INT32_MAX)
    return fail(DSA_ERR_UNSUPPORTED, "K or V rows exceed 2 GiB (total_k %lld)",
                static_cast<long long>(vl->total_k));
  if (checks_enabled() &&
      (st = device_indices(vl, indices, topk, row_begin, row_count, stream, true)))
    return st;
  if (row_count == 0) return ok();
  const size_t need = dsa::grouped_attn_workspace_bytes(row_count, topk);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256))
    return fail(DSA_ERR_WORKSPACE, "grouped workspace needs %zu bytes (256-byte aligned), got %zu",
                need, workspace_bytes);
  return hip_status(
      dsa::launch_grouped_attn(*vl, static_cast<const uint16_t*>(q),
                               static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                               indices, topk, row_begin, row_count, n_heads_q, n_heads_kv,
                               head_dim, softmax_scale, static_cast<uint16_t*>(out), lse,
                               workspace, stream),
      "sparse_attn_prefill_grouped launch");
}

int dsa_indexer_kl(const dsa_varlen* vl, const void* q, const void* k, const float* scores,
                   int64_t ld_scores, int64_t row_begin, int64_t row_count, int32_t n_heads_q,
                   int32_t n_heads_kv, int32_t head_dim, float softmax_scale, float* loss,
                   float* grad, int64_t ld_grad, hipStream_t stream) {
  softmax_scale = resolve_scale(softmax_scale, head_dim);
  int st;
  if ((st = check_varlen(vl))) return st;
  if ((st = check_window(vl, row_begin, row_count))) return st;
  if ((st = check_bf16(q, "q"))) return st;
  if ((st = check_bf16(k, "k"))) return st;
  if ((st = check_scores(vl, scores, ld_scores))) return st;
  if (loss == nullptr || !aligned(loss, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "loss is NULL or misaligned");
  if (grad != nullptr) {
    if (!aligned(grad, 4)) return fail(DSA_ERR_INVALID_ARGUMENT, "grad misaligned");
    if (ld_grad < vl->max_seqlen_k)
      return fail(DSA_ERR_INVALID_ARGUMENT, "ld_grad (%lld) < max_seqlen_k (%d)",
                  static_cast<long long>(ld_grad), vl->max_seqlen_k);
    if (grad == scores && ld_grad != ld_scores)
      return fail(DSA_ERR_INVALID_ARGUMENT, "grad may replace scores only with ld_grad == ld_scores");
  }
  if ((st = check_attn_shape(n_heads_q, n_heads_kv, head_dim, 1, softmax_scale))) return st;
  if (!(softmax_scale > 0.0f))
    return fail(DSA_ERR_UNSUPPORTED, "softmax_scale %g is not positive", softmax_scale);
  if (n_heads_q > 64 || (n_heads_q & (n_heads_q - 1)) != 0)
    return fail(DSA_ERR_UNSUPPORTED, "n_heads_q %d not in {1, 2, 4, ..., 64}", n_heads_q);
  if ((st = check_attn_extent(vl, n_heads_kv, head_dim))) return st;
  if (checks_enabled() &&
      (st = device_scores(vl, scores, ld_scores, row_begin, row_count, stream)))
    return st;
  if (row_count == 0) return ok();
  return hip_status(
      dsa::launch_indexer_kl(*vl, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                             scores, ld_scores, row_begin, row_count, n_heads_q, n_heads_kv,
                             head_dim, softmax_scale, loss, grad, ld_grad, stream),
      "indexer_kl launch");
}

int dsa_index_scores_backward_workspace_size(const dsa_varlen* vl, int32_t n_heads_idx,
                                             int32_t d_idx, int64_t row_count, int want_dq,
                                             int want_dk, size_t* bytes) {
  int st;
  if ((st = check_varlen(vl))) return st;
  if (bytes == nullptr) return fail(DSA_ERR_INVALID_ARGUMENT, "bytes pointer is NULL");
  if (row_count < 0 || row_count > vl->total_q)
    return fail(DSA_ERR_INVALID_ARGUMENT, "row_count %lld outside [0, total_q]",
                static_cast<long long>(row_count));
  if ((st = check_index_shape(n_heads_idx, d_idx))) return st;
  *bytes = dsa::index_backward_workspace_bytes(*vl, n_heads_idx, d_idx, row_count, want_dq != 0,
                                               want_dk != 0);
  return ok();
}

int dsa_index_scores_backward(const dsa_varlen* vl, const void* q_idx, const void* k_idx,
                              const float* w, int32_t n_heads_idx, int32_t d_idx,
                              int64_t row_begin, int64_t row_count, const float* grad,
                              int64_t ld_grad, float* dq_idx, float* dw, float* dk_idx,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st;
  if ((st = check_varlen(vl))) return st;
  if ((st = check_window(vl, row_begin, row_count))) return st;
  if ((st = check_bf16(q_idx, "q_idx"))) return st;
  if ((st = check_bf16(k_idx, "k_idx"))) return st;
  if (w == nullptr || !aligned(w, 4)) return fail(DSA_ERR_INVALID_ARGUMENT, "w is NULL or misaligned");
  if (grad == nullptr || !aligned(grad, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "grad is NULL or misaligned");
  if (ld_grad < vl->max_seqlen_k)
    return fail(DSA_ERR_INVALID_ARGUMENT, "ld_grad (%lld) < max_seqlen_k (%d)",
                static_cast<long long>(ld_grad), vl->max_seqlen_k);
  if ((dq_idx == nullptr) != (dw == nullptr))
    return fail(DSA_ERR_INVALID_ARGUMENT, "dq_idx and dw are given together or not at all");
  if (dq_idx == nullptr && dk_idx == nullptr)
    return fail(DSA_ERR_INVALID_ARGUMENT, "no output requested (dq_idx, dw and dk_idx all NULL)");
  if ((dq_idx != nullptr && !aligned(dq_idx, 4)) || (dw != nullptr && !aligned(dw, 4)) ||
      (dk_idx != nullptr && !aligned(dk_idx, 4)))
    return fail(DSA_ERR_INVALID_ARGUMENT, "dq_idx, dw or dk_idx misaligned");
  if ((st = check_index_shape(n_heads_idx, d_idx))) return st;
  if ((st = check_index_extent(vl, d_idx, 4))) return st;  // dk rows of one sequence in fp32
  if (checks_enabled() && (st = device_offsets(vl, stream))) return st;
  if (row_count == 0) return ok();
  const size_t need = dsa::index_backward_workspace_bytes(*vl, n_heads_idx, d_idx, row_count,
                                                          dq_idx != nullptr, dk_idx != nullptr);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256))
    return fail(DSA_ERR_WORKSPACE,
                "index backward workspace needs %zu bytes (256-byte aligned), got %zu", need,
                workspace_bytes);
  return hip_status(dsa::launch_index_backward(*vl, static_cast<const uint16_t*>(q_idx),
                                               static_cast<const uint16_t*>(k_idx), w, n_heads_idx,
                                               d_idx, row_begin, row_count, grad, ld_grad, dq_idx,
                                               dw, dk_idx, workspace, stream),
                    "index backward launch");
}

int dsa_sparse_attn_decode_workspace_size(const dsa_varlen* vl, int64_t row_count,
                                          int32_t n_heads_q, int32_t head_dim, int32_t topk,
                                          size_t* bytes) {
  int st;
  if ((st = check_varlen(vl))) return st;
  if (bytes == nullptr) return fail(DSA_ERR_INVALID_ARGUMENT, "bytes pointer is NULL");
  if (row_count < 0 || row_count > vl->batch)
    return fail(DSA_ERR_INVALID_ARGUMENT, "row_count %lld outside [0, batch]",
                static_cast<long long>(row_count));
  if (n_heads_q < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "n_heads_q must be >= 1");
  if (head_dim != 64 && head_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
  if (topk < 1 || topk > 4096) return fail(DSA_ERR_UNSUPPORTED, "topk %d not in 1..4096", topk);
  const int splits = dsa::attn_decode_splits(row_count, 1, topk);
  *bytes = dsa::attn_workspace_bytes(row_count, n_heads_q, head_dim, splits);
  return ok();
}

int dsa_sparse_attn_decode(const dsa_varlen* vl, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* indices, int32_t topk,
                           int64_t row_begin, int64_t row_count, int32_t n_heads_q,
                           int32_t n_heads_kv, int32_t head_dim, float softmax_scale, void* out,
                           float* lse, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  softmax_scale = resolve_scale(softmax_scale, head_dim);
  int st;
  if ((st = check_varlen(vl))) return st;
  if (vl->total_q != vl->batch || vl->max_seqlen_q != 1)
    return fail(DSA_ERR_INVALID_ARGUMENT, "decode needs exactly one query per sequence");
  if ((st = check_window(vl, row_begin, row_count))) return st;
  if ((st = check_bf16(q, "q"))) return st;
  if ((st = check_bf16(k_cache, "k_cache"))) return st;
  if ((st = check_bf16(v_cache, "v_cache"))) return st;
  if ((st = check_bf16(out, "out"))) return st;
  if (indices == nullptr || !aligned(indices, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "indices is NULL or misaligned");
  if (lse != nullptr && !aligned(lse, 4)) return fail(DSA_ERR_INVALID_ARGUMENT, "lse misaligned");
  if ((st = check_attn_shape(n_heads_q, n_heads_kv, head_dim, topk, softmax_scale))) return st;
  if ((st = check_attn_extent(vl, n_heads_kv, head_dim))) return st;
  if (checks_enabled() &&
      (st = device_indices(vl, indices, topk, row_begin, row_count, stream, true)))
    return st;
  if (row_count == 0) return ok();
  const int splits = dsa::attn_decode_splits(row_count, n_heads_kv, topk);
  const size_t need = dsa::attn_workspace_bytes(row_count, n_heads_q, head_dim, splits);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256)))
    return fail(DSA_ERR_WORKSPACE, "decode workspace needs %zu bytes (256-byte aligned), got %zu",
                need, workspace_bytes);
  return hip_status(
      dsa::launch_sparse_attn(*vl, static_cast<const uint16_t*>(q),
                              static_cast<const uint16_t*>(k_cache),
                              static_cast<const uint16_t*>(v_cache), indices, topk, row_begin,
                              row_count, n_heads_q, n_heads_kv, head_dim, softmax_scale,
                              static_cast<uint16_t*>(out), lse, splits,
                              static_cast<float*>(workspace), stream),
      "sparse_attn_decode launch");
}

int dsa_sparse_attn_decode_noalloc(const dsa_varlen* vl, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* indices, int32_t topk,
                                   int64_t row_begin, int64_t row_count, int32_t n_heads_q,
                                   int32_t n_heads_kv, int32_t head_dim, float softmax_scale,
                                   void* out, float* lse, hipStream_t stream) {
  softmax_scale = resolve_scale(softmax_scale, head_dim);
  int st;
  if ((st = check_varlen(vl))) return st;
  if (vl->total_q != vl->batch || vl->max_seqlen_q != 1)
    return fail(DSA_ERR_INVALID_ARGUMENT, "decode needs exactly one query per sequence");
  if ((st = check_window(vl, row_begin, row_count))) return st;
  if ((st = check_bf16(q, "q"))) return st;
  if ((st = check_bf16(k_cache, "k_cache"))) return st;
  if ((st = check_bf16(v_cache, "v_cache"))) return st;
  if ((st = check_bf16(out, "out"))) return st;
  if (indices == nullptr || !aligned(indices, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "indices is NULL or misaligned");
  if (lse != nullptr && !aligned(lse, 4)) return fail(DSA_ERR_INVALID_ARGUMENT, "lse misaligned");
  if ((st = check_attn_shape(n_heads_q, n_heads_kv, head_dim, topk, softmax_scale))) return st;
  if ((st = check_attn_extent(vl, n_heads_kv, head_dim))) return st;
  const int splits = dsa::attn_decode_splits(row_count, n_heads_kv, topk);
  const size_t need = dsa::attn_workspace_bytes(row_count, n_heads_q, head_dim, splits);
  if (need > dsa::attn_scratch_bytes())
    return fail(DSA_ERR_UNSUPPORTED,
                "decode partials need %zu bytes, above the fixed scratch of %zu bytes; use "
                "dsa_sparse_attn_decode with a workspace",
                need, dsa::attn_scratch_bytes());
  if (checks_enabled() &&
      (st = device_indices(vl, indices, topk, row_begin, row_count, stream, true)))
    return st;
  if (row_count == 0) return ok();
  float* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = dsa::attn_scratch(&scratch);
    if (e != hipSuccess) return hip_status(e, "decode scratch lookup");
  }
  return hip_status(
      dsa::launch_sparse_attn(*vl, static_cast<const uint16_t*>(q),
                              static_cast<const uint16_t*>(k_cache),
                              static_cast<const uint16_t*>(v_cache), indices, topk, row_begin,
                              row_count, n_heads_q, n_heads_kv, head_dim, softmax_scale,
                              static_cast<uint16_t*>(out), lse, splits, scratch, stream),
      "sparse_attn_decode_noalloc launch");
}

int dsa_check_varlen(const dsa_varlen* vl, hipStream_t stream) {
  int st;
  if ((st = check_varlen(vl))) return st;
  return device_offsets(vl, stream);
}

int dsa_check_indices(const dsa_varlen* vl, const int32_t* indices, int32_t topk,
                      int64_t row_begin, int64_t row_count, hipStream_t stream) {
  int st;
  if ((st = check_varlen(vl))) return st;
  if ((st = check_window(vl, row_begin, row_count))) return st;
  if (indices == nullptr || !aligned(indices, 4))
    return fail(DSA_ERR_INVALID_ARGUMENT, "indices is NULL or misaligned");
  if (topk < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "topk must be >= 1");
  return device_indices(vl, indices, topk, row_begin, row_count, stream, false);
}

int dsa_check_scores(const dsa_varlen* vl, const float* scores, int64_t ld_scores,
                     int64_t row_begin, int64_t row_count, hipStream_t stream) {
  int st;
  if ((st = check_varlen(vl))) return st;
  if ((st = check_window(vl, row_begin, row_count))) return st;
  if ((st = check_scores(vl, scores, ld_scores))) return st;
  return device_scores(vl, scores, ld_scores, row_begin, row_count, stream);
}

}  // extern "C"
