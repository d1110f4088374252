// index_backward.hip -- gradient of the indexer score with respect to the
// indexer's queries, keys and head weights (gfx950).
//
// Keye-VL-2.0 report summary, page 5 section 1: in the dense warm-up only
// the indexer is trained (its distribution pulled towards the full
// attention's), so the loss's gradient must reach the indexer's own inputs.
// With the score I[t, s] = sum_h w[t, h] relu(x[t, h, s]),
// x = qI[t, h, :] . kI[s, :], and an upstream gradient G[t, s] = dL / dI
// over s = 0..p(t), and taking the ReLU's derivative as 1 for x > 0 and 0
// otherwise:
//   dw[t, h]    = sum_s G[t, s] relu(x[t, h, s])
//   dq[t, h, :] = w[t, h] sum_{s : x > 0} G[t, s] kI[s, :]
//   dk[s, :]   += sum_t sum_{h : x > 0} G[t, s] w[t, h] qI[t, h, :]
// Both gradients are small GEMMs around the recomputed head products x,
// which are recomputed exactly as the forward kernels compute them (bf16
// operands, fp32 MFMA accumulation, the same contraction order).  dw needs
// no pass of its own: relu(x) = [x > 0] qI . kI, so dw[t, h] is qI[t, h, :]
// dotted with the dq sum before the weight (Euler's identity for the
// degree-one homogeneous score).
//
// The MQA shape makes dq 64 times larger than dk per position, so the two
// are computed by two kernels, each keeping its own output in registers:
//
//  * dq / dw: 4 query rows per workgroup, each row's heads split over two
//    waves (32 heads each, two waves per SIMD).  The row's queries are the
//    stationary MFMA operand; stages of 128 keys stream through LDS by
//    buffer->LDS DMA.  x is computed as a keys x heads tile, so each lane
//    holds one head and 16 of the tile's keys: after the mask (x > 0) and
//    the gradient are applied those registers already are the A operand of
//    the dq GEMM (heads x keys), whose B operand, keys x d, is a
//    pre-transposed copy of the keys.
//  * dk: 256 keys of one sequence per workgroup, 32 per wave.  The keys are
//    the stationary operand; pairs of rows stream through LDS.  x is
//    computed as a heads x keys tile (lane = key, registers = heads), which
//    after the mask is the A operand of the dk GEMM (keys x heads); its B
//    operand is a per-row transposed copy of the queries with w folded in
//    (heads x d).  Every key block is owned by one workgroup, which adds its
//    result to dk.
//
// In both, every LDS fragment is read a few MFMAs ahead of its use (the
// order pinned with scheduling groups), and the second wave on each SIMD
// covers the other's mask epilogue.  A prep kernel writes the two
// transposed copies into the caller's workspace, with the LDS bank swizzle
// part of the layout so that the DMA is a straight copy.  The GEMM operands
// G [x > 0] and w qI are rounded to bf16.
//
// Stage buffers are separate LDS variables and the stage loops are unrolled
// by two, and every LDS read's address stays a short chain of offsets from
// its variable: only then does the compiler know which buffer an in-flight
// DMA copy writes, and it places no wait for the next stage's copy before
// reads of the current one (otherwise every stage began with a drain).
#include <type_traits>

#include "dsa_common.h"
#include "dsa_internal.h"
#include "index_core.h"

namespace dsa {

namespace {

constexpr int kDqStageKeys = 128;     // keys per LDS stage of the dq kernel
constexpr int kDqRows = 4;            // query rows per dq workgroup
constexpr int kDkWaves = 8;           // waves per dk workgroup, 32 keys each
constexpr int kDkBlockKeys = kDkWaves * 32;
constexpr int kDkStageRows = 2;       // rows per LDS stage of the dk kernel
// The dk work of a window is one workgroup per key block, each running over
// every window row that sees its keys, so the window takes as many rounds of
// the longest blocks as the block count needs on the chip's CUs: 32 blocks
// (a prefill's first 8192-row window) leave most CUs idle, 288 take two
// rounds for 1.125 rounds of work.  Each block's rows are therefore split
// over the workgroup count (at most kDkMaxSplit) that wastes the least of
// the last round.  Each split writes its own partial dk to the workspace (at
// most kDkSlots block partials in all) and a second kernel adds them to dk
// in split order, so the sum stays deterministic.
constexpr int kDkMaxSplit = 8;
constexpr int kDkSlots = 1024;

// Transposed key tiles.  Tile j of sequence b (its keys 32 j .. 32 j + 31)
// is tile number cu_k[b] / 32 + b + j of the workspace: sequences never
// share a tile, and the count stays below total_k / 32 + batch + 1.  A tile
// is d_idx rows of 32 bf16 (4 chunks of 16 bytes); logical chunk c = 2 kk + h
// of row d holds, as element e, key 16 kk + 8 (e / 4) + 4 h + e % 4 -- the
// keys that lane half h feeds to k-step kk of the dq GEMM -- and is stored
// at chunk c ^ swz4(d).
//
// The swizzles make a fragment read (lane l reads row d0 + l % 32) free of
// LDS bank conflicts whether the 16-byte reads are served 16 lanes at a time
// over 64 banks or 8 lanes at a time over 32 banks: the lanes of either
// group land in distinct 16-byte slots of the bank window.
__host__ __device__ __forceinline__ int swz4(int d) {   // rows of 64 bytes
  return ((d >> 2) & 1) | ((((d >> 1) ^ (d >> 3)) & 1) << 1);
}
__host__ __device__ __forceinline__ int swz8(int d) {   // rows of 128 bytes
  return ((d >> 1) & 3) | (((d ^ (d >> 3)) & 1) << 2);
}
__host__ __device__ __forceinline__ int64_t kt_tile(int32_t key_start, int b) {
  return static_cast<int64_t>(key_start / 32) + b;
}
__host__ __device__ __forceinline__ int kt_phys(int c, int d) { return c ^ swz4(d); }

// Transposed queries with the head weight folded in, one block per row:
// d_idx rows of HP = 32 MT bf16 (heads padded with zeros); logical chunk
// c = 2 kk + h of row d holds, as element e, head 16 kk + 8 (e / 4) + 4 h +
// e % 4 times its weight, and is stored at chunk c ^ swz8(d) (HP = 64) or
// c ^ swz4(d) (HP = 32).
template <int HP>
__host__ __device__ __forceinline__ int qw_phys(int c, int d) {
  return HP == 64 ? (c ^ swz8(d)) : (c ^ swz4(d));
}

__device__ __forceinline__ int slot_key(int c, int e) {  // element e of logical chunk c
  return 16 * (c >> 1) + 8 * (e >> 2) + 4 * (c & 1) + (e & 3);
}

// Sequence b whose blocks cover index i, where sequence b's blocks start at
// cu_k[b] / unit + b (strictly increasing in b).
__device__ __forceinline__ int block_sequence(const int32_t* __restrict__ cu_k, int batch,
                                             int64_t i, int unit) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (static_cast<int64_t>(cu_k[mid] / unit) + mid <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The dk blocks a window can touch: from the first block of its first row's
// sequence to the block of the last key its last row sees (blocks of
// sequences in between may have no rows; they only make the count an upper
// bound), and the row split: the s in 1..kDkMaxSplit with the fewest rounds
// of 1/s-size pieces, ceil(count s / cus) / s, ties to the smaller s.
struct DkPlan {
  int64_t first;  // block index of the first candidate block
  int32_t count;  // number of candidate blocks
  int32_t split;  // workgroups per block (1: each block adds to dk itself)
};
__device__ __forceinline__ DkPlan dk_plan(const int32_t* __restrict__ cu_q,
                                          const int32_t* __restrict__ cu_k, int batch,
                                          int64_t row_begin, int64_t row_count, int unit, int cus) {
  const int b1 = find_sequence(cu_q, batch, row_begin);
  const int64_t last = row_begin + row_count - 1;
  const int b2 = find_sequence(cu_q, batch, last);
  const int32_t lk2 = cu_k[b2 + 1] - cu_k[b2];
  const int32_t seen = lk2 - (cu_q[b2 + 1] - cu_q[b2]) + static_cast<int32_t>(last - cu_q[b2]) + 1;
  DkPlan pl;
  pl.first = static_cast<int64_t>(cu_k[b1] / unit) + b1;
  const int64_t end = static_cast<int64_t>(cu_k[b2] / unit) + b2 + (seen + unit - 1) / unit;
  pl.count = static_cast<int32_t>(end - pl.first);
  pl.split = 1;
  int64_t best_rounds = (pl.count + cus - 1) / cus;  // in units of 1/split of a block
  for (int sp = 2; sp <= kDkMaxSplit && static_cast<int64_t>(pl.count) * sp <= kDkSlots; ++sp) {
    const int64_t rounds = (static_cast<int64_t>(pl.count) * sp + cus - 1) / cus;
    if (rounds * pl.split < best_rounds * sp) {  // rounds / sp < best_rounds / split
      best_rounds = rounds;
      pl.split = sp;
    }
  }
  return pl;
}

// ---------------------------------------------------------------- prep

// One workgroup per transposed key tile.
template <int D>
__global__ __launch_bounds__(256) void prep_key_tiles(const int32_t* __restrict__ cu_k, int batch,
                                                      const uint16_t* __restrict__ k_idx,
                                                      uint16_t* __restrict__ kt) {
  __shared__ uint16_t tile[32 * D];
  const int64_t i = blockIdx.x;
  const int b = block_sequence(cu_k, batch, i, 32);
  const int32_t k0 = cu_k[b], len = cu_k[b + 1] - k0;
  const int32_t j = static_cast<int32_t>(i - kt_tile(k0, b));
  if (j < 0 || 32 * j >= len) return;  // a gap between sequences: never read
  const int32_t n = min(32, len - 32 * j);
  constexpr int CH = D / 8;
  for (int f = threadIdx.x; f < 32 * CH; f += blockDim.x) {
    const int key = f / CH, s = f % CH;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (key < n) v = *reinterpret_cast<const uint4*>(k_idx + (k0 + 32 * j + key) * static_cast<int64_t>(D) + s * 8);
    *reinterpret_cast<uint4*>(&tile[key * D + s * 8]) = v;
  }
  __syncthreads();
  uint16_t* out = kt + i * (32 * D);
  for (int f = threadIdx.x; f < D * 4; f += blockDim.x) {
    const int d = f / 4, c = f % 4;
    uint16_t e[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) e[x] = tile[slot_key(c, x) * D + d];
    uint4 v;
    v.x = e[0] | (static_cast<uint32_t>(e[1]) << 16);
    v.y = e[2] | (static_cast<uint32_t>(e[3]) << 16);
    v.z = e[4] | (static_cast<uint32_t>(e[5]) << 16);
    v.w = e[6] | (static_cast<uint32_t>(e[7]) << 16);
    *reinterpret_cast<uint4*>(out + d * 32 + kt_phys(c, d) * 8) = v;
  }
}

// One workgroup per window row: bf16(w[t, h] * qI[t, h, d]), transposed.
template <int D, int HP>
__global__ __launch_bounds__(256) void prep_query_rows(const uint16_t* __restrict__ q_idx,
                                                       const float* __restrict__ w, int n_heads,
                                                       int64_t row_begin,
                                                       uint16_t* __restrict__ qw) {
  __shared__ float wq[HP];
  __shared__ uint16_t q[HP * D];
  const int64_t local = blockIdx.x, row = row_begin + local;
  constexpr int CH = D / 8;
  for (int f = threadIdx.x; f < HP * CH; f += blockDim.x) {
    const int h = f / CH, s = f % CH;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (h < n_heads) v = *reinterpret_cast<const uint4*>(q_idx + (row * n_heads + h) * D + s * 8);
    *reinterpret_cast<uint4*>(&q[h * D + s * 8]) = v;
  }
  for (int h = threadIdx.x; h < HP; h += blockDim.x) wq[h] = h < n_heads ? w[row * n_heads + h] : 0.0f;
  __syncthreads();
  constexpr int CPR = HP / 8;  // chunks per transposed row
  uint16_t* out = qw + local * (static_cast<int64_t>(D) * HP);
  for (int f = threadIdx.x; f < D * CPR; f += blockDim.x) {
    const int d = f / CPR, c = f % CPR;
    uint32_t e[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int h = slot_key(c, x);
      const float qv = __uint_as_float(static_cast<uint32_t>(q[h * D + d]) << 16);
      e[x] = f32_to_bf16_bits(wq[h] * qv);
    }
    uint4 v;
    v.x = e[0] | (e[1] << 16);
    v.y = e[2] | (e[3] << 16);
    v.z = e[4] | (e[5] << 16);
    v.w = e[6] | (e[7] << 16);
    *reinterpret_cast<uint4*>(out + d * HP + qw_phys<HP>(c, d) * 8) = v;
  }
}

// Eight fp32 values as a bf16 MFMA operand (round to nearest even).
__device__ __forceinline__ bf16x8 to_bf16x8(const float (&m)[8]) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  typedef __bf16 bf16v8 __attribute__((ext_vector_type(8)));
  const f32x8 f = {m[0], m[1], m[2], m[3], m[4], m[5], m[6], m[7]};
  return __builtin_bit_cast(bf16x8, __builtin_convertvector(f, bf16v8));
}

// LDS stage buffers, one variable per (array, buffer) pair: with each stage's
// buffer known at compile time the compiler can tell the buffer a DMA is
// filling from the one being read and places no wait for the copy in flight
// before reads of the other (one array indexed by the stage parity made it
// drain every copy in flight at the start of each stage).
template <typename T, int ELEMS, int ID, int B>
__device__ __forceinline__ T* stage_lds() {
  __shared__ __attribute__((aligned(16))) T buf[ELEMS];
  return buf;
}

// A zero the compiler cannot see through: added to a stage buffer's address
// at every stage, it keeps both buffers' per-lane addresses from being held
// in registers across the stage loop.
__device__ __forceinline__ int32_t opaque_zero() {
  int32_t z = 0;
  asm volatile("" : "+s"(z));
  return z;
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// ---------------------------------------------------------------- dq / dw

// 4 query rows per workgroup, each row's heads split over MT waves (32 heads
// each): wave w serves row w % 4 and heads 32 (w / 4) .. 32 (w / 4) + 31.
// With 32 heads a wave's dq accumulator takes 64 registers, so two waves
// fit on a SIMD and each covers the other's epilogue and LDS waits.
template <int D, int MT>
__global__ __launch_bounds__(kDqRows * MT * kWave, 1) void index_bwd_dq_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const uint16_t* __restrict__ q_idx, const uint16_t* k_idx, const uint16_t* kt,
    const float* __restrict__ w, int n_heads, int64_t row_begin, int64_t row_count,
    const float* grad, int64_t ld, float* __restrict__ dq, float* __restrict__ dw) {
  constexpr int SK = kDqStageKeys, KS = D / 16, CH = D / 8, ND = D / 32, TILES = SK / 32;
  constexpr int NT = kDqRows * MT * kWave;
  constexpr int KPI = NT / CH;  // keys per DMA instruction of the workgroup
  constexpr int DMA_K = SK * CH / NT;
  static_assert(KPI % CH == 0 && DMA_K * NT == SK * CH, "stage shape");
  // Stage buffers: keys (swizzled rows), transposed tiles, gradient rows.
  auto ks_lds = [](auto bb) { return stage_lds<uint16_t, SK * D, 0, decltype(bb)::value>(); };
  auto kt_lds = [](auto bb) { return stage_lds<uint16_t, SK * D, 1, decltype(bb)::value>(); };
  auto g_lds = [](auto bb) { return stage_lds<float, kDqRows * SK, 2, decltype(bb)::value>(); };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int slot = wave % kDqRows, mt = wave / kDqRows;  // row slot, head tile
  const int col = lane & 31, half = lane >> 5;
  const int64_t blk = static_cast<int64_t>(gridDim.x) - 1 - blockIdx.x;  // long rows first
  const int64_t first = blk * kDqRows;
  const int64_t last = min(first + kDqRows, row_count) - 1;
  const int64_t local = first + slot;
  const bool active = local < row_count;
  const int64_t row = row_begin + (active ? local : last);
  const int b_me = find_sequence(cu_q, batch, row);
  const int b_lo = find_sequence(cu_q, batch, row_begin + first);
  const int b_hi = find_sequence(cu_q, batch, row_begin + last);
  const RowInfo ri = row_info(cu_q, cu_k, batch, row);

  // This wave's 32 heads of the row's queries: the B operand of x (lane =
  // head, eight d_idx values per lane half and k-step).
  bf16x8 qa[KS];
  {
    const int h = mt * 32 + col;
    const int hl = min(h, n_heads - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 x = load_bf16x8(q_idx + (row * n_heads + hl) * D + half * (D / 2) + ks * 8);
      qa[ks] = h < n_heads ? x : zero_bf16x8();
    }
  }
  f32x16 dqacc[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) dqacc[nd] = f32x16{};

  const int f = wave * kWave + lane;
  const int key0 = f / CH, s0 = f % CH;
  for (int b = b_lo; b <= b_hi; ++b) {
    // Keys 0..pmax of sequence b, pmax the position of the block's last row in b.
    const int32_t q0 = cu_q[b], q1 = cu_q[b + 1], kb = cu_k[b], lk = cu_k[b + 1] - kb;
    if (q1 == q0) continue;  // no query rows (uniform: every wave skips it)
    const int64_t last_in_b = min(row_begin + last, static_cast<int64_t>(q1) - 1);
    const int32_t nkeys = lk - (q1 - q0) + static_cast<int32_t>(last_in_b - q0) + 1;
    const bool mine = active && b_me == b;
    const __amdgpu_buffer_rsrc_t rk = raw_buffer(k_idx + static_cast<int64_t>(kb) * D, nkeys * D * 2);
    const __amdgpu_buffer_rsrc_t rt =
        raw_buffer(kt + kt_tile(kb, b) * (32 * D), ((nkeys + 31) / 32) * D * 64);
    const __amdgpu_buffer_rsrc_t rg = raw_buffer(grad + local * ld, mine ? (ri.pos + 1) * 4 : 0);
    auto fill = [&](auto bb, int32_t c) __attribute__((always_inline)) {
      uint16_t* ksd = ks_lds(bb);
      uint16_t* ktd = kt_lds(bb);
      float* gd = g_lds(bb);
#pragma unroll
      for (int i = 0; i < DMA_K; ++i) {
        const int key = c + i * KPI + key0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (__attribute__((address_space(3))) void*)(&ksd[(i * NT + wave * kWave) * 8]),
            16, key * (D * 2) + ((s0 ^ (key0 & (CH - 1))) * 16), 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < DMA_K; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rt, (__attribute__((address_space(3))) void*)(&ktd[(i * NT + wave * kWave) * 8]),
            16, c * (D * 2) + (i * NT + f) * 16, 0, 0, 0);
      }
      // The row's gradient: each of its head waves copies half of it.
#pragma unroll
      for (int i = 0; i < SK / kWave / MT; ++i) {
        const int o = (i * MT + mt) * kWave;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rg, (__attribute__((address_space(3))) void*)(&gd[slot * SK + o]), 4,
            (c + o + lane) * 4, 0, 0, 0);
      }
    };
    fill(B0{}, 0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
    // One stage: keys [c, c + SK) from buffer bsel, the next stage's copy into
    // the other buffer.
    auto stage = [&](auto bsel, int32_t c) __attribute__((always_inline)) {
      constexpr int B = decltype(bsel)::value;
      if (c + SK < nkeys) fill(std::integral_constant<int, 1 - B>{}, c + SK);
      const int32_t z = opaque_zero();
      const uint16_t* kst = ks_lds(bsel) + z;
      const uint16_t* ktt = kt_lds(bsel) + z;
      const float* gst = g_lds(bsel);
      // A tile takes NF fragments from LDS: KS key fragments for x (A
      // operand, lane = key), then 2 ND transposed-key fragments for dq
      // (B operand, lane = d).  Each is read PF fragments ahead of its MFMA,
      // so no MFMA waits on the read it needs.
      constexpr int NF = KS + 2 * ND, PF = 3;
      auto frag = [&](int tj, int i) -> bf16x8 {
        if (i < KS) {
          const int sl = (half * KS + i) ^ (col & (CH - 1));
          return lds_frag(&kst[(tj * 32 + col) * D + sl * 8]);
        }
        const int nd = (i - KS) >> 1, kk = (i - KS) & 1, d = nd * 32 + col;
        return lds_frag(&ktt[tj * (32 * D) + d * 32 + kt_phys(2 * kk + half, d) * 8]);
      };
#pragma unroll 2  // (a full unroll hoists loads until registers spill)
      for (int tj = 0; tj < TILES; ++tj) {
        bf16x8 fr[NF];
#pragma unroll
        for (int i = 0; i < PF; ++i) fr[i] = frag(tj, i);
        float g[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&gst[slot * SK + tj * 32 + 8 * i + 4 * half]);
          g[4 * i] = v[0];
          g[4 * i + 1] = v[1];
          g[4 * i + 2] = v[2];
          g[4 * i + 3] = v[3];
        }
        // The schedule is pinned: the first PF fragment reads and the four
        // gradient reads go first, then every MFMA is followed by the read
        // PF fragments ahead (left to itself the scheduler sinks each read
        // next to its use and the MFMA waits for it).
        __builtin_amdgcn_sched_group_barrier(0x100, PF + 4, 0);
        // x as keys x heads: lane = head 32 mt + col, register v = key
        // 8 (v / 4) + 4 half + v % 4 of the tile.
        f32x16 x;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + PF < NF) fr[ks + PF] = frag(tj, ks + PF);
          x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[ks], qa[ks], ks == 0 ? f32x16{} : x, 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        // The mask and the gradient: G [x > 0] as the A operand of dq (heads
        // x keys); dw comes from dq at the end.
        float lo[8], hi[8];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float mv = x[v] > 0.0f ? g[v] : 0.0f;
          if (v < 8) lo[v] = mv; else hi[v - 8] = mv;
        }
        const bf16x8 m[2] = {to_bf16x8(lo), to_bf16x8(hi)};
#pragma unroll
        for (int i = 0; i < 2 * ND; ++i) {
          if (KS + i + PF < NF) fr[KS + i + PF] = frag(tj, KS + i + PF);
          dqacc[i >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(m[i & 1], fr[KS + i], dqacc[i >> 1], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (KS + i + PF < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      lds_barrier();
    };
    for (int32_t c = 0; c < nkeys; c += 2 * SK) {
      stage(B0{}, c);
      if (c + SK < nkeys) stage(B1{}, c + SK);
    }
  }
  if (!active) return;
  // acc = sum_s G [x > 0] kI[s, :] for head 32 mt + 8 (v / 4) + 4 half + v % 4
  // (register v of tile nd), column d = 32 nd + col.  dq = w * acc, and
  // since relu(x) = [x > 0] qI . kI, dw = sum_s G relu(x) = qI . acc
  // (Euler's identity for the degree-one homogeneous score): each lane
  // multiplies its 4 columns, then the 32 lanes of a half sum them.
  float wv[16], dwp[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int hr = mt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
    const int hc = min(hr, n_heads - 1);
    const float x = w[row * n_heads + hc];
    wv[v] = hr < n_heads ? x : 0.0f;
    float p = 0.0f;
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      const float q = __uint_as_float(static_cast<uint32_t>(q_idx[(row * n_heads + hc) * D + nd * 32 + col]) << 16);
      p += q * dqacc[nd][v];
    }
    dwp[v] = p;
  }
  const __amdgpu_buffer_rsrc_t rq = raw_buffer(dq + local * n_heads * D, n_heads * D * 4);
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int h = mt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(wv[v] * dqacc[nd][v]), rq,
                                            (h * D + nd * 32 + col) * 4, 0, 0);
    }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) dwp[v] += __shfl_xor(dwp[v], off);
    const int h = mt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
    if (col == 0 && h < n_heads) dw[local * n_heads + h] = dwp[v];
  }
}

// ---------------------------------------------------------------- dk

// 256 keys of one sequence per workgroup, 32 per wave (8 waves, two per
// SIMD so that each covers the other's epilogue); rows stream through LDS
// two at a time.
template <int D, int MT>
__global__ __launch_bounds__(kDkWaves * kWave, 1) void index_bwd_dk_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const uint16_t* q_idx, const uint16_t* __restrict__ k_idx, const uint16_t* qw, int n_heads,
    int64_t row_begin, int64_t row_count, const float* grad, int64_t ld, float* dk,
    float* __restrict__ part, int cus) {
  constexpr int HP = 32 * MT, KS = D / 16, CH = D / 8, ND = D / 32;
  constexpr int RS = kDkStageRows, KB = kDkBlockKeys, HALF = D / 2, NT = kDkWaves * kWave;
  constexpr int QCH = RS * HP * CH;                     // 16-byte chunks of a stage's queries
  constexpr int DMA_Q = QCH / NT;
  constexpr int DMA_W = RS * D * HP / 8 / NT;           // chunks of a stage's transposed rows
  static_assert(DMA_Q * NT == QCH && DMA_W * NT * 8 == RS * D * HP, "stage shape");
  static_assert(RS * KB == NT, "one gradient word per thread and stage");
  // Stage buffers: queries [row][head][chunk ^ head], weighted transposed
  // queries [row][d][phys chunk], gradient rows.
  auto q_lds = [](auto bb) { return stage_lds<uint16_t, RS * HP * D, 3, decltype(bb)::value>(); };
  auto w_lds = [](auto bb) { return stage_lds<uint16_t, RS * D * HP, 4, decltype(bb)::value>(); };
  auto g_lds = [](auto bb) { return stage_lds<float, RS * KB, 5, decltype(bb)::value>(); };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int col = lane & 31, half = lane >> 5;
  const int64_t bi = blockIdx.x;
  const int b = block_sequence(cu_k, batch, bi, KB);
  const int32_t q0 = cu_q[b], q1 = cu_q[b + 1], kb = cu_k[b], lk = cu_k[b + 1] - kb;
  const int32_t j = static_cast<int32_t>(bi - (kb / KB + b));
  const int32_t key_lo = j * KB;
  // Split workgroups (blockIdx.y < split) each take a share of the rows and
  // store a partial; with split == 1 the block adds to dk directly.
  const DkPlan pl = dk_plan(cu_q, cu_k, batch, row_begin, row_count, KB, cus);
  const int sy = blockIdx.y;
  if (sy >= pl.split) return;
  const bool split = pl.split > 1;
  const int64_t slot = bi - pl.first;
  if (split && (slot < 0 || slot >= pl.count)) return;  // not a block of this window
  float* pout = split ? part + (static_cast<int64_t>(sy) * pl.count + slot) * (KB * D) : nullptr;
  auto zero_partial = [&]() {
    for (int i = threadIdx.x; i < KB * D; i += NT) pout[i] = 0.0f;
  };
  if (j < 0 || key_lo >= lk) {
    if (split) zero_partial();
    return;
  }
  // Window rows of sequence b whose position reaches key_lo (this split's share).
  const int32_t shift = lk - (q1 - q0);  // position of local query i is shift + i
  int64_t r_lo = max(max(row_begin, static_cast<int64_t>(q0)),
                     static_cast<int64_t>(q0) + key_lo - shift);
  int64_t r_hi = min(row_begin + row_count, static_cast<int64_t>(q1));
  if (split && r_lo < r_hi) {
    const int64_t share = (r_hi - r_lo + pl.split - 1) / pl.split;
    r_lo += sy * share;
    r_hi = min(r_hi, r_lo + share);
  }
  if (r_lo >= r_hi) {
    if (split) zero_partial();
    return;
  }

  // This wave's 32 keys as the stationary B operand of x (lane = key).
  const int32_t wkey = key_lo + wave * 32;
  const __amdgpu_buffer_rsrc_t rk = raw_buffer(k_idx + static_cast<int64_t>(kb) * D, lk * D * 2);
  bf16x8 kop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rk, (wkey + col) * (D * 2) + (half * HALF + ks * 8) * 2, 0, 0);
    kop[ks] = __builtin_bit_cast(bf16x8, v);
  }
  f32x16 acc[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) acc[nd] = f32x16{};

  const int f = wave * kWave + lane;
  // Stage resources start at the stage's first row, so offsets stay small
  // whatever the window size; rows past the window read as zeros.
  auto fill = [&](auto bb, int64_t r0) __attribute__((always_inline)) {
    uint16_t* qd = q_lds(bb);
    uint16_t* wd = w_lds(bb);
    float* gd = g_lds(bb);
    const int64_t l0 = r0 - row_begin;  // window-local first row of the stage
    const int nrows = static_cast<int>(min(static_cast<int64_t>(RS), row_count - l0));
    const __amdgpu_buffer_rsrc_t rq = raw_buffer(q_idx + r0 * n_heads * D, nrows * n_heads * D * 2);
    const __amdgpu_buffer_rsrc_t rw = raw_buffer(qw + l0 * D * HP, nrows * D * HP * 2);
#pragma unroll
    for (int i = 0; i < DMA_Q; ++i) {
      const int c = i * NT + f;          // chunk of the stage
      const int r = c / (HP * CH), h = (c / CH) % HP, s = c % CH;
      const int src = (r * n_heads + h) * D * 2 + ((s ^ (h & (CH - 1))) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rq, (__attribute__((address_space(3))) void*)(&qd[(i * NT + wave * kWave) * 8]),
          16, src, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < DMA_W; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void*)(&wd[(i * NT + wave * kWave) * 8]),
          16, (i * NT + f) * 16, 0, 0, 0);
    }
    // The gradient of the stage's rows at the block's keys: wave w fetches
    // row w / 4, keys 64 (w % 4) .. 64 (w % 4) + 63.
    const int r = wave / (KB / kWave);
    const int64_t row = r0 + r;
    const int32_t p = shift + static_cast<int32_t>(row - q0);
    const __amdgpu_buffer_rsrc_t rg =
        raw_buffer(grad + (row - row_begin) * ld, row < r_hi ? (p + 1) * 4 : 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rg, (__attribute__((address_space(3))) void*)(&gd[wave * kWave]), 4,
        (key_lo + (wave % (KB / kWave)) * kWave + lane) * 4, 0, 0, 0);
  };

  // A row takes NF fragments from LDS: 2 MT KS query fragments for x (A
  // operand, lane = head), then 2 MT ND weighted-query fragments for dk
  // (B operand, lane = d); each is read PF fragments ahead of its MFMA.
  constexpr int NX = MT * KS, NF = NX + 2 * MT * ND, PF = 3;
  fill(B0{}, r_lo);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  // One stage: rows [r0, r0 + RS) from buffer bsel, the next stage's copy
  // into the other buffer.
  auto stage = [&](auto bsel, int64_t r0) __attribute__((always_inline)) {
    constexpr int B = decltype(bsel)::value;
    if (r0 + RS < r_hi) fill(std::integral_constant<int, 1 - B>{}, r0 + RS);
    const float* gs = g_lds(bsel);
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      const uint16_t* qs = q_lds(bsel) + r * HP * D;
      const uint16_t* ws = w_lds(bsel) + r * D * HP;
      auto frag = [&](int i) -> bf16x8 {
        if (i < NX) {  // x fragment (ks, mt) = (i / MT, i % MT)
          const int h = (i % MT) * 32 + col;
          return lds_frag(&qs[h * D + (((half * KS + i / MT) ^ (h & (CH - 1))) * 8)]);
        }
        const int e = i - NX, nd = e / (2 * MT), kk = e % (2 * MT), d = nd * 32 + col;
        return lds_frag(&ws[d * HP + qw_phys<HP>(2 * kk + half, d) * 8]);
      };
      bf16x8 fr[NF];
#pragma unroll
      for (int i = 0; i < PF; ++i) fr[i] = frag(i);
      const float g = gs[r * KB + wave * 32 + col];
      __builtin_amdgcn_sched_group_barrier(0x100, PF + 1, 0);
      // x as heads x keys: lane = key, register v = head 32 mt + 8 (v / 4) +
      // 4 half + v % 4.
      f32x16 x[MT];
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        if (i + PF < NF) fr[i + PF] = frag(i + PF);
        const int ks = i / MT, mt = i % MT;
        x[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i], kop[ks], ks == 0 ? f32x16{} : x[mt], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      // The mask times the gradient, as the A operand (keys x heads): k-step
      // kk = 2 mt + v / 8 holds heads 16 kk + 8 (e / 4) + 4 half + e % 4.
      bf16x8 m[2 * MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          lo[e] = x[mt][e] > 0.0f ? g : 0.0f;
          hi[e] = x[mt][8 + e] > 0.0f ? g : 0.0f;
        }
        m[2 * mt] = to_bf16x8(lo);
        m[2 * mt + 1] = to_bf16x8(hi);
      }
#pragma unroll
      for (int i = NX; i < NF; ++i) {
        if (i + PF < NF) fr[i + PF] = frag(i + PF);
        const int e = i - NX, nd = e / (2 * MT), kk = e % (2 * MT);
        acc[nd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(m[kk], fr[i], acc[nd], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + PF < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
  };
  for (int64_t r0 = r_lo; r0 < r_hi; r0 += 2 * RS) {
    stage(B0{}, r0);
    if (r0 + RS < r_hi) stage(B1{}, r0 + RS);
  }
  // dk[key, d] += acc: register v of tile nd is key 8 (v / 4) + 4 half +
  // v % 4 of this wave's 32, column d = 32 nd + col.
  if (split) {
#pragma unroll
    for (int nd = 0; nd < ND; ++nd)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = wave * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        pout[key * D + nd * 32 + col] = acc[nd][v];
      }
    return;
  }
  const __amdgpu_buffer_rsrc_t ro = raw_buffer(dk + static_cast<int64_t>(kb) * D, lk * D * 4);
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) {
    float old[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = wkey + 8 * (v >> 2) + 4 * half + (v & 3);
      old[v] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(ro, (key * D + nd * 32 + col) * 4, 0, 0));
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = wkey + 8 * (v >> 2) + 4 * half + (v & 3);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(old[v] + acc[nd][v]), ro,
                                            (key * D + nd * 32 + col) * 4, 0, 0);
    }
  }
}

// Adds the split partials of the window's blocks to dk, split 0 first: one
// workgroup per block slot, one thread per (key, d) element.
template <int D>
__global__ __launch_bounds__(256) void index_bwd_dk_reduce(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    int64_t row_begin, int64_t row_count, const float* __restrict__ part, float* __restrict__ dk,
    int cus) {
  constexpr int KB = kDkBlockKeys;
  const DkPlan pl = dk_plan(cu_q, cu_k, batch, row_begin, row_count, KB, cus);
  const int64_t slot = blockIdx.x;
  if (pl.split == 1 || slot >= pl.count) return;
  const int64_t bi = pl.first + slot;
  const int b = block_sequence(cu_k, batch, bi, KB);
  const int32_t kb = cu_k[b], lk = cu_k[b + 1] - kb;
  const int32_t j = static_cast<int32_t>(bi - (kb / KB + b));
  if (j < 0 || j * KB >= lk) return;
  const int n = min(KB, lk - j * KB) * D;
  float* out = dk + (static_cast<int64_t>(kb) + j * KB) * D;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    float sum = 0.0f;
    for (int sy = 0; sy < pl.split; ++sy) sum += part[(static_cast<int64_t>(sy) * pl.count + slot) * (KB * D) + i];
    out[i] += sum;
  }
}

template <int D, int MT>
hipError_t launch_backward(const dsa_varlen& vl, const uint16_t* q_idx, const uint16_t* k_idx,
                           const float* w, int n_heads, int64_t row_begin, int64_t row_count,
                           const float* grad, int64_t ld, float* dq, float* dw, float* dk,
                           uint8_t* ws, hipStream_t stream) {
  constexpr int HP = 32 * MT;
  uint8_t* p = ws;
  if (dq != nullptr) {
    const int64_t tiles = vl.total_k / 32 + vl.batch + 1;
    uint16_t* kt = reinterpret_cast<uint16_t*>(p);
    p += index_backward_tiles_bytes(tiles, D);
    hipLaunchKernelGGL((prep_key_tiles<D>), dim3(static_cast<unsigned>(tiles)), dim3(256), 0,
                       stream, vl.cu_seqlens_k, vl.batch, k_idx, kt);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const unsigned blocks = static_cast<unsigned>((row_count + kDqRows - 1) / kDqRows);
    hipLaunchKernelGGL((index_bwd_dq_kernel<D, MT>), dim3(blocks), dim3(kDqRows * MT * kWave), 0, stream,
                       vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, q_idx, k_idx, kt, w, n_heads,
                       row_begin, row_count, grad, ld, dq, dw);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  if (dk != nullptr) {
    uint16_t* qw = reinterpret_cast<uint16_t*>(p);
    p += index_backward_rows_bytes(row_count, D, HP);
    float* part = reinterpret_cast<float*>(p);
    int dev = 0, cus = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
    if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev); e != hipSuccess)
      return e;
    hipLaunchKernelGGL((prep_query_rows<D, HP>), dim3(static_cast<unsigned>(row_count)), dim3(256),
                       0, stream, q_idx, w, n_heads, row_begin, qw);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const int64_t blocks = vl.total_k / kDkBlockKeys + vl.batch + 1;
    hipLaunchKernelGGL((index_bwd_dk_kernel<D, MT>), dim3(static_cast<unsigned>(blocks), kDkMaxSplit),
                       dim3(kDkWaves * kWave), 0, stream, vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch,
                       q_idx, k_idx, qw, n_heads, row_begin, row_count, grad, ld, dk, part, cus);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL((index_bwd_dk_reduce<D>), dim3(kDkSlots), dim3(256), 0, stream,
                       vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, row_begin, row_count, part, dk, cus);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t index_backward_tiles_bytes(int64_t tiles, int d) {
  return (static_cast<size_t>(tiles) * 32 * d * 2 + 255) / 256 * 256;
}

size_t index_backward_rows_bytes(int64_t row_count, int d, int hp) {
  return (static_cast<size_t>(row_count) * d * hp * 2 + 255) / 256 * 256;
}

size_t index_backward_workspace_bytes(const dsa_varlen& vl, int n_heads, int d, int64_t row_count,
                                      bool want_dq, bool want_dk) {
  size_t bytes = 0;
  if (want_dq) bytes += index_backward_tiles_bytes(vl.total_k / 32 + vl.batch + 1, d);
  if (want_dk) {
    bytes += index_backward_rows_bytes(row_count, d, n_heads <= 32 ? 32 : 64);
    bytes += static_cast<size_t>(kDkSlots) * kDkBlockKeys * d * 4;  // split partials
  }
  return bytes;
}

hipError_t launch_index_backward(const dsa_varlen& vl, const uint16_t* q_idx,
                                 const uint16_t* k_idx, const float* w, int n_heads, int d,
                                 int64_t row_begin, int64_t row_count, const float* grad,
                                 int64_t ld, float* dq, float* dw, float* dk, void* workspace,
                                 hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const bool wide = n_heads > 32;
  if (d == 128)
    return wide ? launch_backward<128, 2>(vl, q_idx, k_idx, w, n_heads, row_begin, row_count, grad, ld, dq, dw, dk, ws, stream)
                : launch_backward<128, 1>(vl, q_idx, k_idx, w, n_heads, row_begin, row_count, grad, ld, dq, dw, dk, ws, stream);
  return wide ? launch_backward<64, 2>(vl, q_idx, k_idx, w, n_heads, row_begin, row_count, grad, ld, dq, dw, dk, ws, stream)
              : launch_backward<64, 1>(vl, q_idx, k_idx, w, n_heads, row_begin, row_count, grad, ld, dq, dw, dk, ws, stream);
}

}  // namespace dsa
