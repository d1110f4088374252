// topk_core.h -- the streaming per-row top-k select shared by dsa_topk and the
// fused indexer -> top-k (gfx950 device code); the design is described at
// the top of topk.hip.
#pragma once

#include "dsa_common.h"

namespace dsa {
namespace topk {

constexpr int kMaxK = 2048;
constexpr int kSampleMinRow = 8192;     // shorter rows start from threshold zero

// Fill levels of the per-wave segments, held in registers (uniform).
template <int W>
struct Fill {
  uint32_t f[W];
  __device__ uint32_t total() const {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) t += f[w];
    return t;
  }
  // The fill of wave `wave`'s own segment (a select chain: no dynamic
  // register indexing).
  __device__ uint32_t of(int wave) const {
    uint32_t o = 0;
#pragma unroll
    for (int w = 0; w < W; ++w)
      if (w == wave) o = f[w];
    return o;
  }
};

// Monotone map float bits -> uint32 (larger float, larger key); -0 maps
// like +0.
__device__ __forceinline__ uint32_t order_key_bits(uint32_t u) {
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// For finite x, "order_key_bits(x) > thr" is the float test x >= lim with
// lim = the float whose order key is thr + 1: the key map is monotone, and -0
// and +0 share a key as they compare equal.  Keys below that of -inf belong
// to NaN bit patterns; a threshold there admits every finite score (lim =
// -inf), and thr = 2^32 - 1 admits nothing (lim is a NaN).
__device__ __forceinline__ float admit_limit(uint32_t thr) {
  const uint32_t k1 = thr + 1u;
  if (k1 != 0u && k1 <= 0x007FFFFFu) return -__builtin_inff();
  return __uint_as_float((k1 & 0x80000000u) ? (k1 ^ 0x80000000u) : ~k1);
}

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// Wave-wide scans and reductions by DPP (six VALU steps, no LDS round
// trips): row shifts by 1, 2, 4, 8 build the prefix within each row of 16
// lanes; a broadcast of lane 15 into rows 1 and 3, then of lane 31 into
// rows 2 and 3, carries it across rows.  Lanes without a source take the
// operation's identity.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x, uint32_t identity, Op op) {
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(identity, x, 0x111, 0xf, 0xf, false)));
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(identity, x, 0x112, 0xf, 0xf, false)));
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(identity, x, 0x114, 0xf, 0xf, false)));
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(identity, x, 0x118, 0xf, 0xf, false)));
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(identity, x, 0x142, 0xa, 0xf, false)));
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(identity, x, 0x143, 0xc, 0xf, false)));
  return x;
}

// Inclusive prefix sum over the lanes.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t x) {
  return wave_scan(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  return __builtin_amdgcn_readlane(
      wave_scan(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return min(a, b); }), kWave - 1);
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  return __builtin_amdgcn_readlane(
      wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return max(a, b); }), kWave - 1);
}

// Element source for the streaming select.  fetch(j) loads elements
// j..j+3 (j a multiple of 4) with a branch-free, clamped address -- a load
// under a branch would make the compiler wait for it right away and defeat
// the prefetch ring; the caller masks elements >= n.  unpack() turns them
// into (order key, position) pairs.

// Scores of one row: element j is position pos0 + j.  unpack() leaves the
// raw float bits; the order key is formed only for survivors.
struct ScoreSource {
  const float* row;  // score of element 0
  int32_t n;
  int32_t pos0;
  using Raw = float4;
  __device__ Raw fetch(int32_t j) const {
    return *reinterpret_cast<const float4*>(row + min(j, (n - 1) & ~3));
  }
  __device__ void unpack(const Raw& r, int32_t j, uint32_t (&bits)[4], uint32_t (&pv)[4]) const {
    bits[0] = __float_as_uint(r.x); bits[1] = __float_as_uint(r.y);
    bits[2] = __float_as_uint(r.z); bits[3] = __float_as_uint(r.w);
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = static_cast<uint32_t>(pos0 + j + e);
  }
};

// Candidate list of one row (the fused indexer -> top-k): element j is the
// pair (score bits, position) cand[j]; the list is in no particular order.
struct CandSource {
  const uint2* list;
  int32_t n;
  struct Raw {
    u32x4 a, b;
  };
  __device__ Raw fetch(int32_t j) const {
    const u32x4* p = reinterpret_cast<const u32x4*>(list + min(j, (n - 1) & ~3));
    return Raw{p[0], p[1]};
  }
  __device__ void unpack(const Raw& r, int32_t, uint32_t (&bits)[4], uint32_t (&pv)[4]) const {
    bits[0] = r.a.x; pv[0] = r.a.y; bits[1] = r.a.z; pv[1] = r.a.w;
    bits[2] = r.b.x; pv[2] = r.b.y; bits[3] = r.b.z; pv[3] = r.b.w;
  }
};

// One configuration of the row select: THREADS threads, VEC 16-byte loads
// per thread and step (a step covers 4 VEC THREADS scores), a candidate
// buffer of CAP entries in LDS, radix digits of log2(BINS) bits, and a
// start threshold read off 4 SVEC THREADS sampled scores that TARGET2 k / 2
// scores of a row are expected to pass.
template <int VEC, int CAP, int THREADS, int BINS, int TARGET2, int SVEC>
struct TopkImpl {
  static constexpr int kThreads = THREADS;
  static constexpr int kWaves = kThreads / kWave;
  static constexpr int kSampleVec = SVEC;             // sampled 16-byte pieces per thread
  static constexpr int kSamples = 4 * kSampleVec * kThreads;  // scores sampled for the start threshold
  static constexpr int kBins = BINS;
  static constexpr int kDigitBits = __builtin_ctz(BINS);
  static constexpr int kBinsPerThread = kBins / kThreads;
  static constexpr int kVec = VEC;
  static constexpr int kChunk = 4 * kVec * kThreads;  // scores per step
  static constexpr int kWaveStep = 4 * kVec * kWave;  // most entries one wave appends per step
  static constexpr int kDepth = 4;                    // step buffers: kDepth - 1 steps in flight
  static_assert(kDepth == 4, "the stream loop names four step buffers");
  static constexpr int kCap = CAP;                    // candidate buffer entries
  static constexpr int kSeg = kCap / kWaves;          // one buffer segment per wave
  static constexpr int kPerThread = kSeg / kWave;     // a lane's entries of its wave's segment
  static constexpr int kMaskBits = kCap * 32;         // longest row emitted through the bitmask
  static_assert((kBins & (kBins - 1)) == 0 && kBins % kThreads == 0,
                "bins: a power of two, split evenly over threads");
  static_assert(kSeg % kWave == 0, "segments split evenly over lanes");
  static_assert(kSeg - kWaveStep >= (kMaxK + kWaves - 1) / kWaves, "segments too small");
  static_assert(kPerThread >= 4 * kSampleVec, "a thread's sample fits its select entries");
  using FillT = Fill<kWaves>;

  struct Shared {
    // Candidates: raw score bits and position, segment w at [w kSeg, (w+1) kSeg).
    // The kWave entries past kCap take the writes of lanes without a
    // candidate, so an append needs no divergent branch.  key is reused as
    // the position bitmask when emitting.
    uint32_t key[kCap + kWave];
    uint32_t pos[kCap + kWave];
    uint32_t hist[kBins];      // radix histogram
    uint32_t red[2 * kWaves];  // per-wave partials: key ranges, kept counts, prefix sums
    uint32_t sel[5];           // one select level's outcome: lo, hi, above, remaining, equal
    uint32_t fill[2][kWaves];  // per-wave segment fill, double-buffered by step parity
    uint32_t count;
  };

  // A wave's lanes hold the entries of its own segment: entry j of lane l of
  // wave w is buffer slot w kSeg + l + 64 j, valid below the segment's fill.
  static __device__ __forceinline__ int slot(int tid, int j) {
    return (tid / kWave) * kSeg + (tid & (kWave - 1)) + kWave * j;
  }
  static __device__ __forceinline__ bool slot_valid(uint32_t own_fill, int tid, int j) {
    return static_cast<uint32_t>((tid & (kWave - 1)) + kWave * j) < own_fill;
  }

  // m-th largest value of keyf(j) over this thread's entries j = 0..kPerThread-1
  // (slot(tid, j)) for which pred(j) holds, across the workgroup (needs
  // 1 <= m <= number of such entries).  Returns tau, the count of entries
  // strictly above it and the count equal to it.  Block-wide: every thread
  // calls it with the same m.  Sh: any shared struct with this Impl's hist,
  // red and sel members.
  //
  // Radix select with digits relative to the keys' range: each level counts
  // the entries of the current range [lo, hi] into kBins bins of equal
  // width; a workgroup-wide suffix count over the bins (thread t owns
  // kBinsPerThread consecutive bins) finds the bin holding the m-th largest,
  // whose range is the next level's.
  template <class Sh, class KeyF, class Pred>
  static __device__ __attribute__((always_inline)) void select_kth(Sh& sh, uint32_t m, KeyF keyf,
                                                           Pred pred, uint32_t& tau, uint32_t& above,
                                                           uint32_t& equal) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    uint32_t kv[kPerThread];
    bool in[kPerThread];
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  #pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      in[j] = pred(j);
      kv[j] = in[j] ? keyf(j) : 0u;
      if (in[j]) {
        lo = min(lo, kv[j]);
        hi = max(hi, kv[j]);
      }
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) {
      sh.red[wave] = lo;
      sh.red[kWaves + wave] = hi;
    }
    for (int b = tid; b < kBins; b += kThreads) sh.hist[b] = 0u;
    __syncthreads();
    lo = sh.red[0];
    hi = sh.red[kWaves];
  #pragma unroll
    for (int i = 1; i < kWaves; ++i) {
      lo = min(lo, sh.red[i]);
      hi = max(hi, sh.red[kWaves + i]);
    }
    __syncthreads();  // sh.red is reused below
    uint32_t gt = 0, remaining = m;
    while (true) {
      // Histogram of (key - lo) >> shift over [lo, hi]; a single value is one bin.
      const uint32_t span = hi - lo;
      const int bits = span == 0u ? 0 : 32 - __builtin_clz(span);  // span < 2^bits
      const int shift = bits > kDigitBits ? bits - kDigitBits : 0;  // digit < kBins
  #pragma unroll
      for (int j = 0; j < kPerThread; ++j)
        if (in[j] && kv[j] >= lo && kv[j] <= hi) atomicAdd(&sh.hist[(kv[j] - lo) >> shift], 1u);
      __syncthreads();
      // Suffix counts: thread t owns bins [t kBinsPerThread, (t+1) kBinsPerThread).
      uint32_t hb[kBinsPerThread];
      uint32_t local = 0;
  #pragma unroll
      for (int i = 0; i < kBinsPerThread; ++i) {
        hb[i] = sh.hist[tid * kBinsPerThread + i];
        local += hb[i];
      }
      // Inclusive suffix sum within the wave: wave total minus the exclusive prefix.
      const uint32_t incl = wave_prefix_sum(local);
      const uint32_t wave_total = __builtin_amdgcn_readlane(incl, kWave - 1);
      uint32_t suffix = wave_total - incl + local;
      if (lane == 0) sh.red[wave] = wave_total;
      __syncthreads();
      for (int wv = wave + 1; wv < kWaves; ++wv) suffix += sh.red[wv];
      // The owner of the crossing bin: suffix >= remaining > suffix - local.
      if (suffix >= remaining && suffix - local < remaining) {
        uint32_t run = suffix - local;  // entries in higher bins
        int digit = tid * kBinsPerThread;
  #pragma unroll
        for (int i = kBinsPerThread - 1; i >= 0; --i) {
          if (run + hb[i] >= remaining) { digit = tid * kBinsPerThread + i; break; }
          run += hb[i];
        }
        const uint32_t nlo = lo + (static_cast<uint32_t>(digit) << shift);
        const uint32_t width_m1 = shift == 0 ? 0u : ((1u << shift) - 1u);
        sh.sel[0] = nlo;
        sh.sel[1] = (hi - nlo <= width_m1) ? hi : nlo + width_m1;  // no wrap-around
        sh.sel[2] = gt + run;
        sh.sel[3] = remaining - run;
        sh.sel[4] = hb[digit - tid * kBinsPerThread];
      }
      __syncthreads();
      lo = sh.sel[0];
      hi = sh.sel[1];
      gt = sh.sel[2];
      remaining = sh.sel[3];
      equal = sh.sel[4];
      // Every thread has read the level's results and its bins: clear them.
      for (int b = tid; b < kBins; b += kThreads) sh.hist[b] = 0u;
      __syncthreads();
      if (shift == 0) break;
    }
    tau = lo;
    above = gt;
  }

  // Keep the valid entries with key > tau, or key == tau and position <=
  // pos_cut, and lay them out round-robin over the segments (kept/kWaves
  // each).  Slots follow (wave, entry, lane) order, so the layout is
  // deterministic.  Updates the fill levels.  Block-wide.
  static __device__ __attribute__((always_inline)) void regroup(Shared& sh, FillT& fl, uint32_t tau,
                                                        uint32_t pos_cut) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const uint32_t own = fl.of(wave);
    uint32_t kk[kPerThread], pp[kPerThread], at[kPerThread];
    bool keep[kPerThread];
    uint32_t nw = 0;  // kept entries of this wave (uniform)
  #pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      kk[j] = sh.key[slot(tid, j)];
      pp[j] = sh.pos[slot(tid, j)];
      const uint32_t kv = order_key_bits(kk[j]);
      keep[j] = slot_valid(own, tid, j) && (kv > tau || (kv == tau && pp[j] <= pos_cut));
      const unsigned long long mk = __builtin_amdgcn_ballot_w64(keep[j]);
      at[j] = nw + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mk >> 32),
                                             __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mk), 0u));
      nw += static_cast<uint32_t>(__popcll(mk));
    }
    if (lane == 0) sh.red[wave] = nw;
    __syncthreads();  // every entry is read and every wave's count published
    uint32_t base = 0, kept = 0;
  #pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t c = sh.red[w];
      base += w < wave ? c : 0u;
      kept += c;
    }
  #pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      if (keep[j]) {
        const uint32_t s2 = base + at[j];
        const uint32_t e = (s2 % kWaves) * kSeg + s2 / kWaves;  // round-robin over segments
        sh.key[e] = kk[j];
        sh.pos[e] = pp[j];
      }
    }
  #pragma unroll
    for (int w = 0; w < kWaves; ++w) fl.f[w] = (kept + kWaves - 1 - w) / kWaves;
    __syncthreads();  // the new layout is complete before anyone reads it
  }

  // Keep exactly the m best valid entries (key desc, position asc), needs more
  // than m valid entries.  Returns the m-th key, the new acceptance threshold.
  static __device__ __attribute__((always_inline)) uint32_t compact_to(Shared& sh, uint32_t m, FillT& fl) {
    const int tid = threadIdx.x;
    const uint32_t own = fl.of(tid / kWave);
    uint32_t tau, above, equal;
    select_kth(
        sh, m, [&](int j) { return order_key_bits(sh.key[slot(tid, j)]); },
        [&](int j) { return slot_valid(own, tid, j); }, tau, above, equal);
    const uint32_t need = m - above;
    uint32_t pos_cut = 0xFFFFFFFFu;
    if (equal > need) {
      uint32_t t2, a2, e2;
      select_kth(
          sh, need, [&](int j) { return ~sh.pos[slot(tid, j)]; },
          [&](int j) { return slot_valid(own, tid, j) && order_key_bits(sh.key[slot(tid, j)]) == tau; }, t2,
          a2, e2);
      pos_cut = ~t2;
    }
    regroup(sh, fl, tau, pos_cut);
    return tau;
  }

  // Write the kept positions (valid entries, k of them) in ascending order.
  static __device__ __attribute__((always_inline)) void emit_sorted(Shared& sh, const FillT& fl, int k, int32_t n,
                              int32_t* __restrict__ orow) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const uint32_t own = fl.of(wave);
    uint32_t pv[kPerThread];
  #pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      pv[j] = slot_valid(own, tid, j) ? sh.pos[slot(tid, j)] : 0xFFFFFFFFu;
    __syncthreads();  // the key array becomes the bitmask / the pos array is rewritten
    if (n <= kMaskBits) {
      // Bitmask over positions 0..n-1 in the (now free) key array; the rank of
      // a kept position is the number of kept positions below it.  Word
      // prefix counts go to the (now free) position array and chunk prefix
      // counts (64 words per chunk) to the histogram; every pass reads the
      // words lane by lane, so no two lanes of a wave share a bank.
      uint32_t* mask = sh.key;
      uint32_t* pre = sh.pos;
      uint32_t* chunk = sh.hist;
      const int words = (n + 31) / 32;
      const int chunks = (words + kWave - 1) / kWave;
      static_assert(kCap / kWave <= kBins, "chunk prefixes fit the histogram");
      for (int i = tid; i < words; i += kThreads) mask[i] = 0u;
      __syncthreads();
  #pragma unroll
      for (int j = 0; j < kPerThread; ++j)
        if (pv[j] != 0xFFFFFFFFu) atomicOr(&mask[pv[j] >> 5], 1u << (pv[j] & 31));
      __syncthreads();
      for (int c = wave; c < chunks; c += kWaves) {
        const int i = c * kWave + lane;
        const uint32_t cnt = i < words ? static_cast<uint32_t>(__popc(mask[i])) : 0u;
        const uint32_t incl = wave_prefix_sum(cnt);  // inclusive prefix within the chunk
        if (i < words) pre[i] = incl - cnt;
        if (lane == kWave - 1) chunk[c] = incl;
      }
      __syncthreads();
      if (wave == 0) {
        uint32_t carry = 0;
        for (int c0 = 0; c0 < chunks; c0 += kWave) {
          const int c = c0 + lane;
          const uint32_t tot = c < chunks ? chunk[c] : 0u;
          const uint32_t incl = wave_prefix_sum(tot);
          if (c < chunks) chunk[c] = carry + incl - tot;
          carry += __builtin_amdgcn_readlane(incl, kWave - 1);
        }
      }
      __syncthreads();
  #pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        if (pv[j] != 0xFFFFFFFFu) {
          const uint32_t wd = pv[j] >> 5;
          const uint32_t below = mask[wd] & ((1u << (pv[j] & 31)) - 1u);
          orow[chunk[wd / kWave] + pre[wd] + __popc(below)] = static_cast<int32_t>(pv[j]);
        }
      }
      return;
    }
    // Very long rows: gather the k positions densely, then a bitonic sort.
    if (tid == 0) sh.count = 0u;
    __syncthreads();
    uint32_t nv = 0;
  #pragma unroll
    for (int j = 0; j < kPerThread; ++j) nv += pv[j] != 0xFFFFFFFFu ? 1u : 0u;
    uint32_t s = nv ? atomicAdd(&sh.count, nv) : 0u;
  #pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (pv[j] != 0xFFFFFFFFu) sh.pos[s++] = pv[j];
    int k2 = 1;
    while (k2 < k) k2 <<= 1;
    __syncthreads();
    for (int e = static_cast<int>(sh.count) + tid; e < k2; e += kThreads) sh.pos[e] = 0xFFFFFFFFu;
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

  // Streams the n elements of src once (twice if the sampled start threshold
  // proves too high) and leaves exactly the k best of them (key desc,
  // position asc; needs n > k) as the valid entries of the candidate buffer.
  // Block-wide.
  // ORDERED: the source lists elements in ascending position order (a score
  // row), so after a cut an element equal to the k-th key can never beat a
  // kept tie and the admission test stays a strict "greater than".  For an
  // unordered source (candidate lists) ties are readmitted ("at least") and
  // the next cut or the final one settles them by position.
  template <bool ORDERED = true, class Src>
  static __device__ __attribute__((always_inline)) void select_row(Shared& sh, const Src& src, int32_t n,
                                                           int k, FillT& fl) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    // Start threshold: the m-th largest of a spread sample (piece i of
    // thread t: 4 elements at (t kSampleVec + i) / (kThreads kSampleVec) of
    // the stream), m chosen so that about mult TARGET2 k / 2 elements of the
    // stream are expected above it (0, admitting every finite score, when
    // that rank is past the sample).  Block-wide.
    auto sampled_thr = [&](int mult) __attribute__((always_inline)) -> uint32_t {
      uint32_t sk[4 * kSampleVec];
#pragma unroll
      for (int i = 0; i < kSampleVec; ++i) {
        const int32_t at = static_cast<int32_t>(
                               (static_cast<int64_t>(tid * kSampleVec + i) * n) / (kThreads * kSampleVec)) &
                           ~3;
        uint32_t b4[4], p4[4];
        src.unpack(src.fetch(at), at, b4, p4);
#pragma unroll
        for (int e = 0; e < 4; ++e) sk[4 * i + e] = order_key_bits(b4[e]);
      }
      const int64_t want =
          (static_cast<int64_t>(mult) * TARGET2 * k * kSamples + 2 * static_cast<int64_t>(n) - 1) /
          (2 * static_cast<int64_t>(n));
      if (mult > 1 && want > kSamples) return 0u;
      const uint32_t m = static_cast<uint32_t>(want < 1 ? 1 : (want > kSamples ? kSamples : want));
      uint32_t tau, above, equal;
      select_kth(
          sh, m, [&](int j) { return sk[j % (4 * kSampleVec)]; },
          [](int j) { return j < 4 * kSampleVec; }, tau, above, equal);
      // Keys equal to tau are not admitted; lower it by one so they are.
      return tau > 0u ? tau - 1u : 0u;
    };
    // accept key > thr; 0 admits every finite score
    const uint32_t thr0 = n > kSampleMinRow ? sampled_thr(1) : 0u;
    uint32_t thr = thr0;
    int restarts = 0;
    uint32_t mine = 0u;  // this wave's segment fill (uniform within the wave)
    int parity = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) fl.f[w] = 0u;
    float lim = admit_limit(thr);
    int32_t next = 0;  // first element of the next stretch
    bool cut = false;
    const uint32_t seg0 = static_cast<uint32_t>(wave * kSeg);
    const uint32_t dump = static_cast<uint32_t>(kCap + lane);
    // One step covers kChunk elements from `base`: kVec 16-byte loads per
    // thread, held in buf.  Once they are tested, buf is refilled with the
    // step kDepth ahead (after the test, so old and new values never share
    // the registers' lifetime and the loop needs no copies).  When a step
    // leaves a segment nearly full and elements remain, `cut` is set and
    // `next` names the first element not yet tested; later steps of the same
    // group then admit nothing.  BOUNDED steps also test the position
    // against n (only the last steps of a row need it).
    auto step = [&](auto bounded, typename Src::Raw (&buf)[kVec], int32_t base, bool refill) {
      // All compares first (one ballot each, straight from the compare),
      // then the appends: an element group (one element per lane) without
      // survivors costs one scalar test; otherwise each lane writes its
      // (raw bits, position) either to the wave's next free slot (rank among
      // the survivors by mbcnt) or, without a survivor, to its own dump
      // slot -- no divergent branch.  After a cut the limit is a NaN and
      // nothing passes.
      const float lim_s = cut ? __builtin_nanf("") : lim;
      uint32_t bits[kVec][4], pv[kVec][4];
      bool ok[kVec][4];
      unsigned long long mk[kVec][4];
      unsigned long long any = 0ull;
  #pragma unroll
      for (int v = 0; v < kVec; ++v) {
        const int32_t j = base + v * 4 * kThreads + 4 * tid;
        src.unpack(buf[v], j, bits[v], pv[v]);
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          ok[v][e] = __uint_as_float(bits[v][e]) >= lim_s;
          if (decltype(bounded)::value) ok[v][e] = ok[v][e] && j + e < n;
          mk[v][e] = __builtin_amdgcn_ballot_w64(ok[v][e]);
          any |= mk[v][e];
        }
      }
      if (any != 0ull) {
  #pragma unroll
        for (int v = 0; v < kVec; ++v) {
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (mk[v][e] != 0ull) {
              const uint32_t rank = __builtin_amdgcn_mbcnt_hi(
                  static_cast<uint32_t>(mk[v][e] >> 32),
                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mk[v][e]), mine));
              const uint32_t at = ok[v][e] ? seg0 + rank : dump;
              sh.key[at] = bits[v][e];
              sh.pos[at] = pv[v][e];
              mine += static_cast<uint32_t>(__popcll(mk[v][e]));
            }
          }
        }
      }
      if (refill) {
  #pragma unroll
        for (int v = 0; v < kVec; ++v)
          buf[v] = src.fetch(base + kDepth * kChunk + v * 4 * kThreads + 4 * tid);
      }
      // Publish the fill level under this step's parity; the slots of the other
      // parity are only rewritten after the next barrier, when every wave has
      // read them.
      if (lane == 0) sh.fill[parity][wave] = mine;
      __syncthreads();
  #pragma unroll
      for (int w = 0; w < kWaves; ++w) fl.f[w] = sh.fill[parity][w];
      parity ^= 1;
      bool full = false;
  #pragma unroll
      for (int w = 0; w < kWaves; ++w) full |= fl.f[w] > static_cast<uint32_t>(kSeg - kWaveStep);
      const bool now = !cut && full && base + kChunk < n;
      next = now ? base + kChunk : next;
      cut = cut || now;
    };
    // The stream runs in stretches: a stretch ends at the row's end or after
    // the group of steps in which a cut was called for.  The loop holds
    // nothing but the stream (kDepth named buffers, kDepth - 1 steps in
    // flight while one is tested) and leaves only at its latch: an exit
    // from the middle of the group would share the latch in the compiled
    // control flow with loads still pending, and the loop's first wait
    // would become a full drain.  The loads in flight when a stretch ends
    // are dropped, and the next stretch issues them again.
    while (true) {
      // The loads are issued in buffer order, as the loop refills them
      // (scheduling barriers keep that order): the wait before the loop's
      // first test then lets the later steps stay in flight.
      typename Src::Raw b0[kVec], b1[kVec], b2[kVec], b3[kVec];
      const int32_t j0 = next + 4 * tid;
  #pragma unroll
      for (int v = 0; v < kVec; ++v) b0[v] = src.fetch(j0 + v * 4 * kThreads);
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int v = 0; v < kVec; ++v) b1[v] = src.fetch(j0 + kChunk + v * 4 * kThreads);
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int v = 0; v < kVec; ++v) b2[v] = src.fetch(j0 + 2 * kChunk + v * 4 * kThreads);
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int v = 0; v < kVec; ++v) b3[v] = src.fetch(j0 + 3 * kChunk + v * 4 * kThreads);
      __builtin_amdgcn_sched_barrier(0);
      cut = false;
      // Whole groups of kDepth full steps, then the rest of the row (fewer
      // than kDepth steps, the last one possibly partial) with bound checks.
      int32_t base = next;
      for (; base + kDepth * kChunk <= n && !cut; base += kDepth * kChunk) {
        step(BoolTag<false>{}, b0, base, true);
        step(BoolTag<false>{}, b1, base + kChunk, true);
        step(BoolTag<false>{}, b2, base + 2 * kChunk, true);
        step(BoolTag<false>{}, b3, base + 3 * kChunk, true);
      }
      if (!cut && base < n) {
        step(BoolTag<true>{}, b0, base, false);
        if (base + kChunk < n) step(BoolTag<true>{}, b1, base + kChunk, false);
        if (base + 2 * kChunk < n) step(BoolTag<true>{}, b2, base + 2 * kChunk, false);
        if (base + 3 * kChunk < n) step(BoolTag<true>{}, b3, base + 3 * kChunk, false);
      }
      if (cut) {
        // One segment is nearly full.  With more than k entries held, cut to
        // the k best and raise the threshold; otherwise (survivors crowd one
        // wave's segment) keep them all and spread them evenly.
        if (fl.total() > static_cast<uint32_t>(k)) {
          thr = compact_to(sh, k, fl);
          if (!ORDERED) thr = thr > 0u ? thr - 1u : 0u;
          lim = admit_limit(thr);
        } else {
          regroup(sh, fl, 0u, 0xFFFFFFFFu);
        }
        mine = fl.of(wave);
        continue;
      }
      // Done when k elements are held, or when the threshold was already zero
      // (every finite score passes it, so only non-finite input can leave
      // fewer; the row then gets fewer positions, padded, and never loops).
      if (fl.total() >= static_cast<uint32_t>(k) || thr == 0u) break;
      // The sampled threshold was too high (fewer than k elements beat it and
      // no cut happened): stream again, first from the same sample's rank
      // for four times as many survivors, then from zero.  (A restart from
      // zero admits every score until the first cut and then cuts about
      // k ln(n / k) / (CAP - k) more times.)
      const uint32_t lower = restarts == 0 && n > kSampleMinRow ? sampled_thr(4) : 0u;
      thr = lower < thr ? lower : 0u;
      ++restarts;
      lim = admit_limit(thr);
      next = 0;
      mine = 0u;
  #pragma unroll
      for (int w = 0; w < kWaves; ++w) fl.f[w] = 0u;
      __syncthreads();
    }
    if (fl.total() > static_cast<uint32_t>(k)) compact_to(sh, k, fl);
  }

};

}  // namespace topk
}  // namespace dsa
