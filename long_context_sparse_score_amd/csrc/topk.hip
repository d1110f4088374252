// topk.hip -- deterministic per-row top-k of indexer scores.
//
// For each query row keep the n = min(k, p + 1) positions with the largest
// score, ties towards the lower position, and write them in ascending
// position order padded with -1 (Keye-VL-2.0 report summary, page 5: section
// 1 keeps the k = 2048 best positions per query token; section 8 needs the
// selection to be deterministic so training and inference agree).
//
// One workgroup of 256 threads owns one row and reads it from HBM exactly
// once, in position order, two steps in flight.  Many rows use steps of
// 1024 scores and ~37 KB of LDS, so four rows run per CU and hide each
// other's latencies; few long rows (decode) use steps of 4096 scores and a
// candidate buffer twice as large, so one row alone keeps 32 KB in flight.
// Barriers span only four waves.
//
// A score survives only if its order-preserving key beats the running
// threshold; survivors are appended to a candidate buffer in LDS (each wave
// to its own segment, slots assigned by ballot prefix counts).  Long
// rows start from a threshold read off a 1024-score sample of the row (256
// spread 16-byte pieces) at the rank where about 2.5 k scores of the whole
// row are expected above it, so the buffer is cut once or twice per row
// instead of a dozen times.  The estimate only decides speed: if fewer than
// k scores beat it, the row is streamed again from threshold zero, so the
// result is exact for any input.  When
// the buffer could overflow on the next step it is cut to exactly k entries
// by a radix select whose digits are taken relative to the range of the
// candidates' keys (min..max, 1024 bins): the bins spread over the values
// actually present, so atomics rarely collide and each level shrinks the
// range 1024-fold.  Ties at the k-th key are cut by a second select on the
// position.  The new threshold is the k-th key: later scores equal to it sit
// at higher positions and can never displace the kept ties, so the test
// stays a strict "greater than".  At the end the kept positions are marked
// in an LDS bitmask and written in ascending order by a prefix count over
// its words (a bitonic sort serves rows too long for the bitmask).  Every
// decision depends only on key and position values, never on the order in
// which lanes appended, so the output is bitwise repeatable.
#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

namespace {
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kSamples = 4 * kThreads;  // scores sampled for the start threshold
constexpr int kBins = 1024;
constexpr int kBinsPerThread = kBins / kThreads;
constexpr int kMaxK = 2048;
constexpr int kSampleMinRow = 8192;     // shorter rows start from threshold zero

// Fill levels of the four segments, held in registers (uniform).
struct Fill {
  uint32_t f[kWaves];
  __device__ uint32_t total() const {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += f[w];
    return t;
  }
};

// Monotone map float bits -> uint32 (larger float, larger key); -0 maps
// like +0.
__device__ __forceinline__ uint32_t order_key_bits(uint32_t u) {
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// "order_key_bits(u) > thr" with one integer compare, valid when thr >= 2^31
// (the threshold is +0 or a positive float): then only positive scores can
// pass, and for them the key is u + 2^31.
__device__ __forceinline__ bool above_nonneg_threshold(uint32_t u, uint32_t thr) {
  return static_cast<int32_t>(u) > static_cast<int32_t>(thr ^ 0x80000000u);
}

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, static_cast<uint32_t>(__shfl_xor(v, off)));
  return v;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(v, off)));
  return v;
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

// One configuration of the row select: VEC 16-byte loads per thread and step
// (a step covers 4 VEC 256 scores), a candidate buffer of CAP entries in LDS.
// Many rows: VEC = 1, CAP = 4096 (37 KB of LDS, four rows per CU hide each
// other's latencies).  Few long rows: VEC = 4, CAP = 8192 (69 KB), so that
// one row keeps 32 KB of scores in flight.
template <int VEC, int CAP>
struct TopkImpl {
  static constexpr int kVec = VEC;
  static constexpr int kChunk = 4 * kVec * kThreads;  // scores per step
  static constexpr int kWaveStep = 4 * kVec * kWave;  // most entries one wave appends per step
  static constexpr int kCap = CAP;                    // candidate buffer entries
  static constexpr int kSeg = kCap / kWaves;          // one buffer segment per wave
  static constexpr int kPerThread = kCap / kThreads;
  static constexpr int kSegPerThread = kPerThread / kWaves;  // a thread's entries in one segment
  static constexpr int kMaskBits = kCap * 32;         // longest row emitted through the bitmask
  static_assert(kSeg == kThreads * kSegPerThread, "entry j of a thread lies in segment j / kSegPerThread");
  static_assert(kSeg - kWaveStep >= (kMaxK + kWaves - 1) / kWaves, "segments too small");

  struct Shared {
    uint32_t key[kCap];  // reused as the position bitmask when emitting
    uint32_t pos[kCap];
    uint32_t hist[kBins];
    uint32_t red[2 * kWaves];
    uint32_t fill[2][kWaves];  // per-wave segment fill, double-buffered by step parity
    uint32_t count;
    uint32_t lo, hi, above, remaining, equal;
  };

  // Entry j of thread t is buffer slot t + 256 j, i.e. segment j / kSegPerThread
  // at offset t + 256 (j % kSegPerThread).
  static __device__ __forceinline__ bool slot_valid(const Fill& fl, int tid, int j) {
    return static_cast<uint32_t>(tid + kThreads * (j % kSegPerThread)) < fl.f[j / kSegPerThread];
  }

  // m-th largest value of keyf(j) over this thread's entries j = 0..kPerThread-1
  // (slot tid + 256 j) for which pred(j) holds, across the workgroup (needs
  // 1 <= m <= number of such entries).  Returns tau, the count of entries
  // strictly above it and the count equal to it.  Block-wide: every thread
  // calls it with the same m.
  template <class KeyF, class Pred>
  static __device__ __attribute__((always_inline)) void select_kth(Shared& sh, uint32_t m, KeyF keyf, Pred pred, uint32_t& tau,
                             uint32_t& above, uint32_t& equal) {
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
      const int shift = bits > 10 ? bits - 10 : 0;                  // digit < 1024
  #pragma unroll
      for (int j = 0; j < kPerThread; ++j)
        if (in[j] && kv[j] >= lo && kv[j] <= hi) atomicAdd(&sh.hist[(kv[j] - lo) >> shift], 1u);
      __syncthreads();
      // Suffix counts: thread t owns bins [t*4, t*4 + 4).
      uint32_t hb[kBinsPerThread];
      uint32_t local = 0;
  #pragma unroll
      for (int i = 0; i < kBinsPerThread; ++i) {
        hb[i] = sh.hist[tid * kBinsPerThread + i];
        local += hb[i];
      }
      uint32_t suffix = local;  // inclusive suffix sum within the wave
  #pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t t = __shfl_down(suffix, off);
        if (lane + off < kWave) suffix += t;
      }
      if (lane == 0) sh.red[wave] = suffix;  // wave total
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
        sh.lo = nlo;
        sh.hi = (hi - nlo <= width_m1) ? hi : nlo + width_m1;  // no wrap-around
        sh.above = gt + run;
        sh.remaining = remaining - run;
        sh.equal = hb[digit - tid * kBinsPerThread];
      }
      __syncthreads();
      lo = sh.lo;
      hi = sh.hi;
      gt = sh.above;
      remaining = sh.remaining;
      equal = sh.equal;
      // Every thread has read the level's results and its bins: clear them.
      for (int b = tid; b < kBins; b += kThreads) sh.hist[b] = 0u;
      __syncthreads();
      if (shift == 0) break;
    }
    tau = lo;
    above = gt;
  }

  // Keep the valid entries with key > tau, or key == tau and position <=
  // pos_cut, and lay them out round-robin over the four segments (kept/4 each).
  // Updates the fill levels.  Block-wide.
  static __device__ __attribute__((always_inline)) void regroup(Shared& sh, Fill& fl, uint32_t tau,
                                                        uint32_t pos_cut) {
    const int tid = threadIdx.x;
    uint32_t kk[kPerThread], pp[kPerThread];
    uint32_t nk = 0;
  #pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      kk[j] = 0u;
      pp[j] = 0u;
      if (slot_valid(fl, tid, j)) {
        const uint32_t kv = sh.key[tid + kThreads * j], pv = sh.pos[tid + kThreads * j];
        if (kv > tau || (kv == tau && pv <= pos_cut)) {
          kk[j] = kv;
          pp[j] = pv | 0x80000000u;  // mark as kept (positions < 2^31)
          ++nk;
        }
      }
    }
    if (tid == 0) sh.count = 0u;
    __syncthreads();
    uint32_t s = nk ? atomicAdd(&sh.count, nk) : 0u;
  #pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      if (pp[j] & 0x80000000u) {
        const int e = (s & (kWaves - 1)) * kSeg + (s >> 2);  // round-robin over segments
        sh.key[e] = kk[j];
        sh.pos[e] = pp[j] & 0x7FFFFFFFu;
        ++s;
      }
    }
    __syncthreads();
    const uint32_t kept = sh.count;
  #pragma unroll
    for (int w = 0; w < kWaves; ++w) fl.f[w] = (kept + kWaves - 1 - w) / kWaves;
    __syncthreads();  // everyone has read sh.count before it is reused
  }

  // Keep exactly the m best valid entries (key desc, position asc), needs more
  // than m valid entries.  Returns the m-th key, the new acceptance threshold.
  static __device__ __attribute__((always_inline)) uint32_t compact_to(Shared& sh, uint32_t m, Fill& fl) {
    const int tid = threadIdx.x;
    uint32_t tau, above, equal;
    select_kth(
        sh, m, [&](int j) { return sh.key[tid + kThreads * j]; },
        [&](int j) { return slot_valid(fl, tid, j); }, tau, above, equal);
    const uint32_t need = m - above;
    uint32_t pos_cut = 0xFFFFFFFFu;
    if (equal > need) {
      uint32_t t2, a2, e2;
      select_kth(
          sh, need, [&](int j) { return ~sh.pos[tid + kThreads * j]; },
          [&](int j) { return slot_valid(fl, tid, j) && sh.key[tid + kThreads * j] == tau; }, t2,
          a2, e2);
      pos_cut = ~t2;
    }
    regroup(sh, fl, tau, pos_cut);
    return tau;
  }

  // Write the kept positions (valid entries, k of them) in ascending order.
  static __device__ __attribute__((always_inline)) void emit_sorted(Shared& sh, const Fill& fl, int k, int32_t n,
                              int32_t* __restrict__ orow) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    uint32_t pv[kPerThread];
  #pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      pv[j] = slot_valid(fl, tid, j) ? sh.pos[tid + kThreads * j] : 0xFFFFFFFFu;
    __syncthreads();  // the key array becomes the bitmask / the pos array is rewritten
    if (n <= kMaskBits) {
      // Bitmask over positions 0..n-1 in the (now free) key array.
      uint32_t* mask = sh.key;
      const int words = (n + 31) / 32;
      for (int i = tid; i < words; i += kThreads) mask[i] = 0u;
      __syncthreads();
  #pragma unroll
      for (int j = 0; j < kPerThread; ++j)
        if (pv[j] != 0xFFFFFFFFu) atomicOr(&mask[pv[j] >> 5], 1u << (pv[j] & 31));
      __syncthreads();
      // Thread t owns words [t*per, t*per + per).
      const int per = (words + kThreads - 1) / kThreads;
      const int w0 = tid * per;
      uint32_t cnt = 0;
      for (int i = 0; i < per; ++i)
        if (w0 + i < words) cnt += __popc(mask[w0 + i]);
      uint32_t incl = cnt;  // inclusive prefix within the wave
  #pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      if (lane == kWave - 1) sh.red[wave] = incl;
      __syncthreads();
      uint32_t base = incl - cnt;
      for (int i = 0; i < wave; ++i) base += sh.red[i];
      for (int i = 0; i < per; ++i) {
        if (w0 + i >= words) break;
        uint32_t bitsw = mask[w0 + i];
        while (bitsw) {
          const int b = __builtin_ctz(bitsw);
          orow[base++] = (w0 + i) * 32 + b;
          bitsw &= bitsw - 1u;
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

  // Streams the n elements of src once (twice if the sampled start threshold
  // proves too high) and leaves exactly the k best of them (key desc,
  // position asc; needs n > k) as the valid entries of the candidate buffer.
  // Block-wide.
  template <class Src>
  static __device__ __attribute__((always_inline)) void select_row(Shared& sh, const Src& src, int32_t n,
                                                           int k, Fill& fl) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    for (int b = tid; b < kBins; b += kThreads) sh.hist[b] = 0u;
    uint32_t thr0 = 0u;  // accept key > thr; 0 admits every finite score
    if (n > kSampleMinRow) {
      // Start threshold: the m-th largest of a spread sample (thread t reads 4
      // elements at t/256 of the stream), m chosen so that about 2.5 k
      // elements of the stream are expected above it.
      const int32_t at = (static_cast<int32_t>((static_cast<int64_t>(tid) * n) / kThreads)) & ~3;
      uint32_t sk[4], sp[4];
      src.unpack(src.fetch(at), at, sk, sp);
#pragma unroll
      for (int e = 0; e < 4; ++e) sk[e] = order_key_bits(sk[e]);
      const int64_t want = (static_cast<int64_t>(5 * k) * kSamples + 2 * static_cast<int64_t>(n) - 1) /
                           (2 * static_cast<int64_t>(n));
      const uint32_t m = static_cast<uint32_t>(want < 1 ? 1 : (want > kSamples ? kSamples : want));
      uint32_t tau, above, equal;
      select_kth(
          sh, m, [&](int j) { return sk[j & 3]; }, [](int j) { return j < 4; }, tau, above, equal);
      // Keys equal to tau are not admitted; lower it by one so they are.
      thr0 = tau > 0u ? tau - 1u : 0u;
    }
    uint32_t thr = thr0;
    uint32_t mine;  // this wave's segment fill (uniform within the wave)
    uint32_t* seg_key = sh.key + wave * kSeg;
    uint32_t* seg_pos = sh.pos + wave * kSeg;
    int parity;
  restart:
  #pragma unroll
    for (int w = 0; w < kWaves; ++w) fl.f[w] = 0u;
    mine = 0u;
    parity = 0;
    // Each step covers kChunk elements: kVec 16-byte loads per thread, issued
    // together.  Two steps are in flight; the loop is unrolled by two so each
    // step keeps its registers (rotating loaded values between registers would
    // make the compiler wait for the loads as soon as they are copied), and it
    // runs whole pairs of steps (steps past n admit nothing).
    auto step = [&](typename Src::Raw (&buf)[kVec], int32_t base) {
      uint32_t kvs[kVec][4], pvs[kVec][4];
  #pragma unroll
      for (int v = 0; v < kVec; ++v) {
        const int32_t j = base + v * 4 * kThreads + 4 * tid;
        src.unpack(buf[v], j, kvs[v], pvs[v]);
        buf[v] = src.fetch(j + 2 * kChunk);
      }
      // Append this wave's survivors to its own segment: slots by ballot
      // prefix counts, no shared counter.  Above a non-negative threshold one
      // integer compare of the raw bits decides; the order key is formed only
      // for survivors.
      // Per element group (one element per lane) only a compare and a ballot
      // unless the group holds survivors; a survivor's slot is the lane's
      // rank among them (mbcnt).  Only the last step of a row needs the
      // bound check.
      auto append = [&](auto fast, auto tail) {
  #pragma unroll
        for (int v = 0; v < kVec; ++v) {
          const int32_t j = base + v * 4 * kThreads + 4 * tid;
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t u = kvs[v][e];
            bool acc = decltype(fast)::value ? above_nonneg_threshold(u, thr)
                                             : order_key_bits(u) > thr;
            if (decltype(tail)::value) acc = acc && (j + e < n);
            const unsigned long long mk = __ballot(acc);
            if (mk != 0ull) {
              if (acc) {
                const uint32_t s = mine + __builtin_amdgcn_mbcnt_hi(
                    static_cast<uint32_t>(mk >> 32),
                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mk), 0u));
                seg_key[s] = order_key_bits(u);
                seg_pos[s] = pvs[v][e];
              }
              mine += __popcll(mk);
            }
          }
        }
      };
      const bool tail = base + kChunk > n;
      if (thr >= 0x80000000u) {
        if (tail) append(BoolTag<true>{}, BoolTag<true>{});
        else append(BoolTag<true>{}, BoolTag<false>{});
      } else {
        if (tail) append(BoolTag<false>{}, BoolTag<true>{});
        else append(BoolTag<false>{}, BoolTag<false>{});
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
      if (full && base + kChunk < n) {
        // One segment is nearly full.  With more than k entries held, cut to
        // the k best and raise the threshold; otherwise (survivors crowd one
        // wave's segment) keep them all and spread them evenly.
        if (fl.total() > static_cast<uint32_t>(k))
          thr = compact_to(sh, k, fl);
        else
          regroup(sh, fl, 0u, 0xFFFFFFFFu);
  #pragma unroll
        for (int w = 0; w < kWaves; ++w)
          if (w == wave) mine = fl.f[w];  // no dynamic register indexing
      }
    };
    typename Src::Raw buf_a[kVec], buf_b[kVec];
  #pragma unroll
    for (int v = 0; v < kVec; ++v) {
      buf_a[v] = src.fetch(v * 4 * kThreads + 4 * tid);
      buf_b[v] = src.fetch(kChunk + v * 4 * kThreads + 4 * tid);
    }
    for (int32_t base = 0; base < n; base += 2 * kChunk) {
      step(buf_a, base);
      step(buf_b, base + kChunk);
    }
    if (fl.total() < static_cast<uint32_t>(k)) {
      // The sampled threshold was too high (fewer than k elements beat it and
      // no cut happened): stream again from zero.
      thr = 0u;
      __syncthreads();
      goto restart;
    }
    if (fl.total() > static_cast<uint32_t>(k)) compact_to(sh, k, fl);
  }

};

// One workgroup per row: the whole row streamed once, k positions out.
template <class Impl>
__global__ __launch_bounds__(kThreads) void topk_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const float* __restrict__ scores, int64_t ld, int64_t row_begin, int64_t row_count, int k,
    int32_t* __restrict__ indices) {
  __shared__ typename Impl::Shared sh;
  const int tid = threadIdx.x;
  // Later rows are longer: hand them out first.
  const int64_t local = row_count - 1 - static_cast<int64_t>(blockIdx.x);
  const RowInfo ri = row_info(cu_q, cu_k, batch, row_begin + local);
  const int32_t n = ri.pos + 1;
  int32_t* orow = indices + local * k;
  if (n <= k) {
    for (int j = tid; j < k; j += kThreads) orow[j] = j < n ? j : -1;
    return;
  }
  Fill fl;
  Impl::select_row(sh, ScoreSource{scores + local * ld, n, 0}, n, k, fl);
  Impl::emit_sorted(sh, fl, k, n, orow);
}

}  // namespace

hipError_t launch_topk(const dsa_varlen& vl, const float* scores, int64_t ld, int64_t row_begin,
                       int64_t row_count, int k, int32_t* indices, hipStream_t stream) {
  static_assert(kBins % kThreads == 0, "bins split evenly over threads");
  // With fewer rows than two per CU, rows cannot hide each other's
  // latencies: give each row the wide configuration.
  if (row_count < 512)
    hipLaunchKernelGGL((topk_kernel<TopkImpl<4, 8192>>), dim3(static_cast<unsigned>(row_count)),
                       dim3(kThreads), 0, stream, vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, scores,
                       ld, row_begin, row_count, k, indices);
  else
    hipLaunchKernelGGL((topk_kernel<TopkImpl<1, 4096>>), dim3(static_cast<unsigned>(row_count)),
                       dim3(kThreads), 0, stream, vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, scores,
                       ld, row_begin, row_count, k, indices);
  return hipGetLastError();
}

}  // namespace dsa
