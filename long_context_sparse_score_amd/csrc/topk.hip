// topk.hip -- deterministic per-row top-k of indexer scores.
//
// For each query row keep the n = min(k, p + 1) positions with the largest
// score, ties towards the lower position, and write them in ascending
// position order padded with -1 (Keye-VL-2.0 report summary, page 5: section
// 1 keeps the k = 2048 best positions per query token; section 8 needs the
// selection to be deterministic so training and inference agree).
//
// One workgroup of 1024 threads owns one row and reads it from HBM exactly
// once, in position order, 4096 scores per step.  A score survives only if
// its order-preserving key beats the running threshold; survivors are
// appended to a candidate buffer in LDS (one LDS atomic per wave per step,
// slots assigned by ballot prefix counts).  When the buffer could overflow
// on the next step it is compacted to exactly k entries by a three-level
// radix select over the buffer (11 + 11 + 10 bits of the key), ties at the
// threshold resolved by a second radix select on the position.  The new
// threshold is the k-th key: later scores equal to it sit at higher positions
// and can never displace the kept ties, so the test is a strict "greater
// than".  At the end the k kept positions are sorted by a bitonic network in
// LDS.  Every decision depends only on key and position values, never on the
// order in which lanes appended, so the output is bitwise repeatable.
#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kChunk = 4 * kThreads;  // scores per step (one float4 per thread)
constexpr int kCap = 8192;            // candidate buffer entries (>= k + kChunk)
constexpr int kPerThread = kCap / kThreads;
constexpr int kBins = 2048;
constexpr int kMaxK = 2048;

struct TopkShared {
  uint32_t key[kCap];
  uint32_t pos[kCap];
  uint32_t hist[kBins];
  uint32_t count;
  uint32_t prefix;
  uint32_t remaining;
  uint32_t above;
  uint32_t equal;
};

// Monotone map float -> uint32 (larger float, larger key); -0 maps like +0.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// m-th largest of keyf(e) over buffer entries e < cnt with pred(e) (needs
// 1 <= m <= number of such entries).  Returns tau, the count strictly above
// it and the count equal to it.  Block-wide; all threads must call.
template <class KeyF, class Pred>
__device__ void select_kth(TopkShared& sh, uint32_t cnt, uint32_t m, KeyF keyf, Pred pred,
                           uint32_t& tau, uint32_t& above, uint32_t& equal) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0, remaining = m, gt = 0;
#pragma unroll
  for (int level = 0; level < 3; ++level) {
    const int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
    const int bins = level == 2 ? 1024 : 2048;
    for (int b = tid; b < bins; b += kThreads) sh.hist[b] = 0u;
    __syncthreads();
    for (uint32_t e = tid; e < cnt; e += kThreads) {
      if (pred(e)) {
        const uint32_t kv = keyf(e);
        if ((kv & mask) == prefix) atomicAdd(&sh.hist[(kv >> shift) & (bins - 1)], 1u);
      }
    }
    __syncthreads();
    if (tid < kWave) {
      const int lane = tid;
      const int per = bins / kWave;
      uint32_t local = 0;
      for (int b = 0; b < per; ++b) local += sh.hist[lane * per + b];
      uint32_t suffix = local;  // inclusive suffix sum over lanes
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t t = __shfl_down(suffix, off);
        if (lane + off < kWave) suffix += t;
      }
      const unsigned long long ok = __ballot(suffix >= remaining);
      const int last = ok ? 63 - __builtin_clzll(ok) : 0;
      if (lane == last) {
        uint32_t run = suffix - local;  // entries in higher lanes' bins
        int digit = lane * per;
        for (int b = lane * per + per - 1; b >= lane * per; --b) {
          const uint32_t c = sh.hist[b];
          if (run + c >= remaining) { digit = b; break; }
          run += c;
        }
        sh.prefix = prefix | (static_cast<uint32_t>(digit) << shift);
        sh.above = gt + run;
        sh.remaining = remaining - run;
        sh.equal = sh.hist[digit];
      }
    }
    __syncthreads();
    prefix = sh.prefix;
    gt = sh.above;
    remaining = sh.remaining;
    mask |= static_cast<uint32_t>(bins - 1) << shift;
  }
  tau = prefix;
  above = gt;
  equal = sh.equal;
  __syncthreads();
}

// Keep exactly the m best entries (key desc, position asc).  Returns the
// m-th key, the new acceptance threshold.
__device__ uint32_t compact_to(TopkShared& sh, uint32_t m) {
  const int tid = threadIdx.x;
  const uint32_t cnt = sh.count;
  uint32_t tau, above, equal;
  select_kth(
      sh, cnt, m, [&](uint32_t e) { return sh.key[e]; }, [](uint32_t) { return true; }, tau,
      above, equal);
  const uint32_t need = m - above;
  uint32_t pos_cut = 0xFFFFFFFFu;
  if (equal > need) {
    uint32_t t2, a2, e2;
    select_kth(
        sh, cnt, need, [&](uint32_t e) { return ~sh.pos[e]; },
        [&](uint32_t e) { return sh.key[e] == tau; }, t2, a2, e2);
    pos_cut = ~t2;
  }
  uint32_t kk[kPerThread], pp[kPerThread];
  bool keep[kPerThread];
  uint32_t nk = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const uint32_t e = tid + j * kThreads;
    keep[j] = false;
    if (e < cnt) {
      kk[j] = sh.key[e];
      pp[j] = sh.pos[e];
      keep[j] = kk[j] > tau || (kk[j] == tau && pp[j] <= pos_cut);
    }
    nk += keep[j] ? 1u : 0u;
  }
  __syncthreads();
  if (tid == 0) sh.count = 0u;
  __syncthreads();
  uint32_t slot = nk ? atomicAdd(&sh.count, nk) : 0u;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    if (keep[j]) {
      sh.key[slot] = kk[j];
      sh.pos[slot] = pp[j];
      ++slot;
    }
  }
  __syncthreads();
  return tau;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const float* __restrict__ scores, int64_t ld, int64_t row_begin, int64_t row_count, int k,
    int32_t* __restrict__ indices) {
  __shared__ TopkShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // Later rows are longer: hand them out first.
  const int64_t local = row_count - 1 - static_cast<int64_t>(blockIdx.x);
  const RowInfo ri = row_info(cu_q, cu_k, batch, row_begin + local);
  const int32_t n = ri.pos + 1;
  int32_t* orow = indices + local * k;
  if (n <= k) {
    for (int j = tid; j < k; j += kThreads) orow[j] = j < n ? j : -1;
    return;
  }
  const float* srow = scores + local * ld;
  if (tid == 0) sh.count = 0u;
  __syncthreads();

  uint32_t thr = 0u;  // accept key > thr; 0 admits every finite score
  float4 cur = make_float4(0.f, 0.f, 0.f, 0.f);
  if (4 * tid < n) cur = *reinterpret_cast<const float4*>(srow + 4 * tid);
  for (int32_t base = 0; base < n; base += kChunk) {
    const int32_t j = base + 4 * tid;
    float4 nxt = make_float4(0.f, 0.f, 0.f, 0.f);
    if (j + kChunk < n) nxt = *reinterpret_cast<const float4*>(srow + j + kChunk);
    const float xs[4] = {cur.x, cur.y, cur.z, cur.w};
    uint32_t kv[4];
    unsigned long long mk[4];
    uint32_t total = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kv[e] = order_key(xs[e]);
      const bool acc = (j + e < n) && kv[e] > thr;
      mk[e] = __ballot(acc);
      total += __popcll(mk[e]);
    }
    if (total) {
      uint32_t wbase = 0;
      if (lane == 0) wbase = atomicAdd(&sh.count, total);
      wbase = __shfl(wbase, 0);
      const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((mk[e] >> lane) & 1ull) {
          const uint32_t s = wbase + __popcll(mk[e] & below);
          sh.key[s] = kv[e];
          sh.pos[s] = static_cast<uint32_t>(j + e);
        }
        wbase += __popcll(mk[e]);
      }
    }
    __syncthreads();
    if (sh.count > static_cast<uint32_t>(kCap - kChunk) && base + kChunk < n)
      thr = compact_to(sh, k);
    cur = nxt;
  }
  if (sh.count > static_cast<uint32_t>(k)) compact_to(sh, k);

  // Sort the k kept positions ascending (bitonic network over a power of two).
  int k2 = 1;
  while (k2 < k) k2 <<= 1;
  for (int e = k + tid; e < k2; e += kThreads) sh.pos[e] = 0xFFFFFFFFu;
  __syncthreads();
  for (int size = 2; size <= k2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (k2 >> 1); t += kThreads) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint32_t a = sh.pos[lo], b = sh.pos[hi];
        if ((a > b) == up) {
          sh.pos[lo] = b;
          sh.pos[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int e = tid; e < k; e += kThreads) orow[e] = static_cast<int32_t>(sh.pos[e]);
}

}  // namespace

hipError_t launch_topk(const dsa_varlen& vl, const float* scores, int64_t ld, int64_t row_begin,
                       int64_t row_count, int k, int32_t* indices, hipStream_t stream) {
  static_assert(kCap >= kMaxK + kChunk, "candidate buffer too small");
  hipLaunchKernelGGL(topk_kernel, dim3(static_cast<unsigned>(row_count)), dim3(kThreads), 0,
                     stream, vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, scores, ld, row_begin,
                     row_count, k, indices);
  return hipGetLastError();
}

}  // namespace dsa
