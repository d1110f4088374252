// index_topk.hip -- the indexer fused with the top-k (dsa_index_topk).
//
// The k best positions of each query row by indexer score (Keye-VL-2.0
// report summary, page 5 section 1: the scout scores every position and the
// k = 2048 best are kept; section 8: the selection is deterministic) without
// writing the row's scores out and reading them back.
//
// The indexer (index_scores.hip, candidate mode) keeps only the scores at or
// above a per-row threshold tau and appends them as (score bits, position)
// to the row's candidate list; the streaming select of topk_core.h then runs
// over that list instead of the whole score row.  The result is exact
// whatever tau is: when at least k scores reach tau and none was dropped,
// every one of the row's k best (ties included) is a candidate, and the
// select's tie rule is the one dsa_topk applies.  Any other row is flagged
// and recomputed the unfused way by a fallback kernel.  tau only decides how
// much work that is.  It is read off a sample of the row's own scores (every
// stride-th key, scored by the same MFMA core, so with the same bits) at the
// rank where about kCandTarget scores of the whole row are expected above
// it; rows with at most kCandCap keys keep every score.
//
// Launches per call: the indexer on every stride-th key (the sample), the
// thresholds, the indexer in candidate mode, the select, and the fallback
// (whose workgroups leave at once unless their row is flagged).
#include "dsa_common.h"
#include "dsa_internal.h"
#include "index_core.h"
#include "topk_core.h"

namespace dsa {

namespace {

using namespace core;
using namespace topk;

constexpr int kCandTarget = 5120;    // expected candidates of a long row
constexpr int kCandCap = 10240;      // list entries per row (rows up to this many keys keep all)
constexpr int kSampleMax = 4096;     // sampled keys of the longest row at most
constexpr int kThresholdRows = 4;    // rows (waves) per threshold workgroup
constexpr int kThresholdBits = 16;   // tau resolved to the top 16 bits of the order key
constexpr int kSelThreads = 512;     // select workgroup
constexpr int kSelPer = kCandCap / kSelThreads;  // candidates per select thread
constexpr int kSpanWords = 4096;     // positions marked per emit pass: 131072

int sample_stride(int32_t max_seqlen_k) {
  return max(64, (max_seqlen_k + kSampleMax - 1) / kSampleMax);
}

// One wave per window row: clears the row's candidate counter and sets its
// threshold.  A row of at most `cap` keys admits everything (tau = -inf).
// Otherwise tau is the m-th largest of the row's sampled scores (positions
// 0, stride, 2 stride, ..., scored by the indexer into `samples`) rounded
// down to the top kThresholdBits bits of its order key, m = target *
// samples / keys (at least 1): at least m sampled scores, and about
// `target` of the row's, reach it.  RPL samples per lane (RPL * 64 >= the
// longest row's sample count).
template <int RPL>
__global__ __launch_bounds__(kThresholdRows * kWave) void threshold_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    int64_t row_begin, int64_t row_count, const float* __restrict__ samples, int64_t ld_s,
    int stride, int cap, int target, float* __restrict__ tau, uint32_t* __restrict__ count) {
  const int lane = lane_id();
  const int64_t local = static_cast<int64_t>(blockIdx.x) * kThresholdRows +
                        __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  if (local >= row_count) return;
  const RowInfo ri = row_info(cu_q, cu_k, batch, row_begin + local);
  const int32_t n = ri.pos + 1;
  if (lane == 0) count[local] = 0u;
  if (n <= cap) {
    if (lane == 0) tau[local] = -__builtin_inff();
    return;
  }
  const int32_t ns = visible_keys(ri.pos, stride);
  const int64_t want = (static_cast<int64_t>(target) * ns + n - 1) / n;
  const uint32_t m = static_cast<uint32_t>(want < 1 ? 1 : (want > ns ? ns : want));
  const float* srow = samples + local * ld_s;
  uint32_t key[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {  // clamped loads, no branch: all in flight at once
    const int32_t j = r * kWave + lane;
    const uint32_t kv = order_key_bits(__float_as_uint(srow[min(j, ns - 1)]));
    key[r] = j < ns ? kv : 0u;  // 0: below every score
  }
  // The largest K (a multiple of 2^(32 - kThresholdBits)) with at least m
  // keys >= K, bit by bit from the top.
  uint32_t ans = 0u;
  for (int b = 31; b >= 32 - kThresholdBits; --b) {
    const uint32_t c = ans | (1u << b);
    uint32_t cnt = 0u;
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      cnt += static_cast<uint32_t>(__popcll(__builtin_amdgcn_ballot_w64(key[r] >= c)));
    if (cnt >= m) ans = c;
  }
  // ans <= the m-th largest sampled key, so "score >= the float of ans"
  // admits at least those m sampled scores.  Every finite score's key is at
  // least 2^23 (that of -inf is 2^23 - 1), a multiple of 2^16, so ans >= 2^23
  // and its float is finite.
  if (lane == 0) tau[local] = __uint_as_float((ans & 0x80000000u) ? (ans ^ 0x80000000u) : ~ans);
}

// The select: one workgroup per row holds the row's whole candidate list in
// registers (kSelPer entries a thread), finds the k-th largest order key by
// the relative-range radix select of topk_core.h (then the position cut
// among keys equal to it: ties go to the lower position), marks the k kept
// positions in an LDS bitmask and writes them in ascending order by prefix
// counts over its words.  A row the list cannot settle (fewer than k
// candidates, or more than the list holds) is flagged for the fallback.
using SelImpl = TopkImpl<1, kCandCap, kSelThreads, 512, 3, 2>;  // its select_kth: kSelPer a thread
static_assert(SelImpl::kPerThread == kSelPer, "one select entry per register");

struct SelShared {
  uint32_t hist[SelImpl::kBins];
  uint32_t red[2 * SelImpl::kWaves];
  uint32_t sel[5];
  uint32_t mask[kSpanWords];
  uint32_t pre[kSpanWords];
  uint32_t chunk[kSpanWords / kWave];
};

__global__ __launch_bounds__(kSelThreads) void cand_select_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    int64_t row_begin, int64_t row_count, int k, const uint32_t* __restrict__ count,
    const uint2* __restrict__ cand, int cap, int32_t* __restrict__ indices,
    uint32_t* __restrict__ flags) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t local = row_count - 1 - static_cast<int64_t>(blockIdx.x);
  const RowInfo ri = row_info(cu_q, cu_k, batch, row_begin + local);
  const int32_t n = ri.pos + 1;
  int32_t* orow = indices + local * k;
  if (n <= k) {
    for (int j = tid; j < k; j += kSelThreads) orow[j] = j < n ? j : -1;
    if (tid == 0) flags[local] = 0u;
    return;
  }
  const uint32_t cnt = count[local];
  const bool settled = cnt >= static_cast<uint32_t>(k) && cnt <= static_cast<uint32_t>(cap);
  if (tid == 0) flags[local] = settled ? 0u : 1u;
  if (!settled) return;
  // Entry j of this thread: candidate j * kSelThreads + tid (coalesced),
  // clamped loads, invalid entries key 0.
  const uint2* list = cand + local * cap;
  uint32_t key[kSelPer], pos[kSelPer];
#pragma unroll
  for (int j = 0; j < kSelPer; ++j) {
    const uint32_t at = static_cast<uint32_t>(j * kSelThreads + tid);
    const uint2 e = list[min(at, cnt - 1u)];
    key[j] = at < cnt ? order_key_bits(e.x) : 0u;
    pos[j] = e.y;
  }
  auto valid = [&](int j) { return static_cast<uint32_t>(j * kSelThreads + tid) < cnt; };
  uint32_t tau, above, equal;
  SelImpl::select_kth(sh, static_cast<uint32_t>(k), [&](int j) { return key[j]; }, valid, tau, above,
                      equal);
  const uint32_t need = static_cast<uint32_t>(k) - above;
  uint32_t pos_cut = 0xFFFFFFFFu;
  if (equal > need) {
    uint32_t t2, a2, e2;
    SelImpl::select_kth(sh, need, [&](int j) { return ~pos[j]; },
                        [&](int j) { return valid(j) && key[j] == tau; }, t2, a2, e2);
    pos_cut = ~t2;
  }
  bool keep[kSelPer];
#pragma unroll
  for (int j = 0; j < kSelPer; ++j)
    keep[j] = valid(j) && (key[j] > tau || (key[j] == tau && pos[j] <= pos_cut));
  // Ascending emission, kSpanWords * 32 positions per pass.
  uint32_t base = 0;
  for (int32_t span0 = 0; span0 < n; span0 += kSpanWords * 32) {
    const int words = min(kSpanWords, (n - span0 + 31) / 32);
    const int chunks = (words + kWave - 1) / kWave;
    for (int i = tid; i < words; i += kSelThreads) sh.mask[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
      const uint32_t p = pos[j] - static_cast<uint32_t>(span0);
      if (keep[j] && p < static_cast<uint32_t>(kSpanWords * 32)) atomicOr(&sh.mask[p >> 5], 1u << (p & 31));
    }
    __syncthreads();
    for (int c = wave; c < chunks; c += SelImpl::kWaves) {
      const int i = c * kWave + lane;
      const uint32_t wc = i < words ? static_cast<uint32_t>(__popc(sh.mask[i])) : 0u;
      const uint32_t incl = wave_prefix_sum(wc);
      if (i < words) sh.pre[i] = incl - wc;
      if (lane == kWave - 1) sh.chunk[c] = incl;
    }
    __syncthreads();
    if (wave == 0) {  // chunks <= 64: one wave-wide exclusive scan
      const uint32_t tot = lane < chunks ? sh.chunk[lane] : 0u;
      const uint32_t incl = wave_prefix_sum(tot);
      if (lane < chunks) sh.chunk[lane] = incl - tot;
      if (lane == kWave - 1) sh.red[0] = incl;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
      const uint32_t p = pos[j] - static_cast<uint32_t>(span0);
      if (keep[j] && p < static_cast<uint32_t>(kSpanWords * 32)) {
        const uint32_t wd = p >> 5;
        const uint32_t below = sh.mask[wd] & ((1u << (p & 31)) - 1u);
        orow[base + sh.chunk[wd / kWave] + sh.pre[wd] + __popc(below)] = static_cast<int32_t>(pos[j]);
      }
    }
    base += sh.red[0];
    __syncthreads();  // the arrays are rewritten by the next span
  }
}

// The exact fallback, one workgroup per row; rows without a flag leave at
// once.  The workgroup's waves score the whole row (each a contiguous range
// of keys, with the same MFMA core) into the row's score buffer, then the
// select of dsa_topk runs over it.
using FallbackImpl = TopkImpl<1, 4096, 256, 512, 3, 2>;

template <int D, int MT>
__global__ __launch_bounds__(FallbackImpl::kThreads) void fallback_select_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx,
    const float* __restrict__ w, int n_heads, int64_t row_begin, int64_t row_count, int k,
    const uint32_t* __restrict__ flags, float* __restrict__ scores, int64_t ld,
    int32_t* __restrict__ indices) {
  using Impl = FallbackImpl;
  __shared__ typename Impl::Shared sh;
  const int64_t local = row_count - 1 - static_cast<int64_t>(blockIdx.x);
  if (flags[local] == 0u) return;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int64_t row = row_begin + local;
  const RowInfo ri = row_info(cu_q, cu_k, batch, row);
  const int32_t n = ri.pos + 1;
  float* srow = scores + local * ld;
  const int32_t q = (n + Impl::kWaves * 64 - 1) / (Impl::kWaves * 64) * 64;
  const int32_t c0 = wave * q, c1 = min(n, c0 + q);
  if (c0 < c1) {
    RowState<D, MT> st;
    load_row_state<D, MT>(st, q_idx, w, row, n_heads, col, half);
    row_direct<D, MT>(st, k_idx, ri, 1, c0, c1, col, half,
                      [&](float v, int32_t j) {
                        if (j < c1) srow[j] = v;
                      },
                      []() {});
  }
  __syncthreads();  // the row's scores are complete and visible to the workgroup
  typename Impl::FillT fl;
  Impl::select_row(sh, ScoreSource{srow, n, 0}, n, k, fl);
  int32_t* orow = indices + local * k;
  Impl::emit_sorted(sh, fl, k, n, orow);
  for (int j = static_cast<int>(fl.total()) + tid; j < k; j += Impl::kThreads) orow[j] = -1;
}

// Workspace of one call, every piece 256-byte aligned.
struct Layout {
  size_t counts, flags, tau, samples, cand, scores, total;
  int64_t ld_s, ld;
  int stride;
};

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

Layout layout(const dsa_varlen& vl, int64_t rows) {
  Layout l;
  l.stride = sample_stride(vl.max_seqlen_k);
  l.ld_s = (static_cast<int64_t>(visible_keys(vl.max_seqlen_k - 1, l.stride)) + 63) / 64 * 64;
  l.ld = (static_cast<int64_t>(vl.max_seqlen_k) + 63) / 64 * 64;
  size_t at = 0;
  l.counts = at;
  at += align256(rows * sizeof(uint32_t));
  l.flags = at;
  at += align256(rows * sizeof(uint32_t));
  l.tau = at;
  at += align256(rows * sizeof(float));
  l.samples = at;
  at += align256(static_cast<size_t>(rows) * l.ld_s * sizeof(float));
  l.cand = at;
  at += align256(static_cast<size_t>(rows) * kCandCap * sizeof(uint2));
  l.scores = at;
  at += align256(static_cast<size_t>(rows) * l.ld * sizeof(float));
  l.total = at;
  return l;
}

template <int D, int MT>
hipError_t launch_dm(const dsa_varlen& vl, const uint16_t* q_idx, const uint16_t* k_idx,
                     const float* w, int n_heads, int d, int64_t row_begin, int64_t row_count,
                     int k, int32_t* indices, void* workspace, hipStream_t stream) {
  const Layout l = layout(vl, row_count);
  char* ws = static_cast<char*>(workspace);
  uint32_t* counts = reinterpret_cast<uint32_t*>(ws + l.counts);
  uint32_t* flags = reinterpret_cast<uint32_t*>(ws + l.flags);
  float* tau = reinterpret_cast<float*>(ws + l.tau);
  float* samples = reinterpret_cast<float*>(ws + l.samples);
  uint2* cand = reinterpret_cast<uint2*>(ws + l.cand);
  float* scores = reinterpret_cast<float*>(ws + l.scores);
  const dim3 rows(static_cast<unsigned>(row_count));
  hipError_t e;
  // 1. Sampled scores (every stride-th key), needed only by rows longer than
  //    a candidate list.
  if (vl.max_seqlen_k > kCandCap) {
    IndexOut so;
    so.scores = samples;
    so.ld = l.ld_s;
    so.key_stride = l.stride;
    if ((e = launch_index_scores_to(vl, q_idx, k_idx, w, n_heads, d, row_begin, row_count, so,
                                    false, stream)) != hipSuccess)
      return e;
  }
  // 2. Per-row thresholds; counters cleared.
  const dim3 tgrid(static_cast<unsigned>((row_count + kThresholdRows - 1) / kThresholdRows));
  if (visible_keys(vl.max_seqlen_k - 1, l.stride) <= 32 * kWave)
    hipLaunchKernelGGL(threshold_kernel<32>, tgrid, dim3(kThresholdRows * kWave), 0, stream,
                       vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, row_begin, row_count, samples,
                       l.ld_s, l.stride, kCandCap, kCandTarget, tau, counts);
  else
    hipLaunchKernelGGL(threshold_kernel<kSampleMax / kWave>, tgrid, dim3(kThresholdRows * kWave),
                       0, stream, vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, row_begin,
                       row_count, samples, l.ld_s, l.stride, kCandCap, kCandTarget, tau, counts);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 3. The indexer in candidate mode.
  IndexOut co;
  co.tau = tau;
  co.count = counts;
  co.cand = cand;
  co.cap = kCandCap;
  if ((e = launch_index_scores_to(vl, q_idx, k_idx, w, n_heads, d, row_begin, row_count, co, true,
                                  stream)) != hipSuccess)
    return e;
  // 4. The exact top-k of every candidate list; unsettled rows flagged.
  hipLaunchKernelGGL(cand_select_kernel, rows, dim3(kSelThreads), 0, stream, vl.cu_seqlens_q,
                     vl.cu_seqlens_k, vl.batch, row_begin, row_count, k, counts, cand, kCandCap,
                     indices, flags);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 5. Flagged rows the unfused way.
  hipLaunchKernelGGL((fallback_select_kernel<D, MT>), rows, dim3(FallbackImpl::kThreads), 0, stream,
                     vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, q_idx, k_idx, w, n_heads,
                     row_begin, row_count, k, flags, scores, l.ld, indices);
  return hipGetLastError();
}

}  // namespace

size_t index_topk_workspace_bytes(const dsa_varlen& vl, int64_t row_count, int k) {
  (void)k;
  return row_count == 0 ? 0 : layout(vl, row_count).total;
}

hipError_t launch_index_topk(const dsa_varlen& vl, const uint16_t* q_idx, const uint16_t* k_idx,
                             const float* w, int n_heads, int d, int64_t row_begin,
                             int64_t row_count, int k, int32_t* indices, void* workspace,
                             hipStream_t stream) {
  if (d == 128) {
    if (n_heads > 32)
      return launch_dm<128, 2>(vl, q_idx, k_idx, w, n_heads, d, row_begin, row_count, k, indices,
                               workspace, stream);
    return launch_dm<128, 1>(vl, q_idx, k_idx, w, n_heads, d, row_begin, row_count, k, indices,
                             workspace, stream);
  }
  if (n_heads > 32)
    return launch_dm<64, 2>(vl, q_idx, k_idx, w, n_heads, d, row_begin, row_count, k, indices,
                            workspace, stream);
  return launch_dm<64, 1>(vl, q_idx, k_idx, w, n_heads, d, row_begin, row_count, k, indices,
                          workspace, stream);
}

}  // namespace dsa
