// index_core.h -- the indexer's MFMA core shared by the indexer kernels and
// the fused indexer -> top-k (gfx950 device code).
//
// I[t, s] = sum_h w[t, h] * max(0, qI[t, h, :] . kI[s, :])  (Keye-VL-2.0
// report summary, page 5 section 1: the lightweight scout with one MQA key
// per position).  For one query row the head-by-key product is a small GEMM
// with M = indexer heads (up to 64), N = keys, K = d_idx.  Heads sit on the
// MFMA rows so that after v_mfma_f32_32x32x16_bf16 every lane holds one key
// column and 16 heads of it: the ReLU, the weight and the head sum happen in
// registers, and one exchange between the two half-waves finishes the sum.
// The contraction over d_idx is ordered so that each half-wave covers one
// contiguous half of every qI / kI row, which keeps every load a full 16-byte
// vector.  Every kernel that scores with this core produces the same bits
// for the same (row, key).
#pragma once

#include "dsa_common.h"

namespace dsa {
namespace core {

// Keys a row at position pos sees when key j is position j * stride.
__host__ __device__ __forceinline__ int32_t visible_keys(int32_t pos, int stride) {
  return stride == 1 ? pos + 1 : pos / stride + 1;
}

// Per-wave stationary state: this row's indexer queries (A operand, heads on
// MFMA rows, MT tiles of 32 heads) and its head weights laid out like the
// accumulator rows.
template <int D, int MT>
struct RowState {
  static constexpr int KS = D / 16;
  bf16x8 a[MT][KS];
  float wv[MT][16];
};

// The row's queries as the MFMA operand: heads on the rows (lane = head),
// eight consecutive d_idx values per lane half and k-step.
template <int D, int MT>
__device__ __forceinline__ void load_row_queries(bf16x8 (&a)[MT][D / 16],
                                                 const uint16_t* __restrict__ q_idx, int64_t row,
                                                 int n_heads, int col, int half) {
  constexpr int KS = D / 16, HALF = D / 2;
  // Loads are issued for clamped heads and zeroed afterwards: a load under
  // a lane-dependent branch becomes its own basic block, and the loads would
  // no longer overlap.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = mt * 32 + col;
    const int hl = min(h, n_heads - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 x = load_bf16x8(q_idx + (row * n_heads + hl) * D + half * HALF + ks * 8);
      a[mt][ks] = h < n_heads ? x : zero_bf16x8();
    }
  }
}

// The row's head weights laid out like the accumulator rows: element v of
// this lane is head 32 mt + 8 (v / 4) + 4 half + v % 4 (0 past n_heads).
template <int MT>
__device__ __forceinline__ void load_row_weights(float (&wv)[MT][16], const float* __restrict__ w,
                                                 int64_t row, int n_heads, int half) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int hr = mt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      const float x = w[row * n_heads + min(hr, n_heads - 1)];
      wv[mt][v] = hr < n_heads ? x : 0.0f;
    }
}

// Both, interleaved per head tile (the order the forward kernels' schedules
// were tuned with).
template <int D, int MT>
__device__ __forceinline__ void load_row_state(RowState<D, MT>& st,
                                               const uint16_t* __restrict__ q_idx,
                                               const float* __restrict__ w, int64_t row,
                                               int n_heads, int col, int half) {
  constexpr int KS = D / 16, HALF = D / 2;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = mt * 32 + col;
    const int hl = min(h, n_heads - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 x = load_bf16x8(q_idx + (row * n_heads + hl) * D + half * HALF + ks * 8);
      st.a[mt][ks] = h < n_heads ? x : zero_bf16x8();
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int hr = mt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      const float x = w[row * n_heads + min(hr, n_heads - 1)];
      st.wv[mt][v] = hr < n_heads ? x : 0.0f;
    }
  }
}

// Head products of one 32-key tile.
template <int D, int MT>
__device__ __forceinline__ void tile_mfma(const RowState<D, MT>& st, const bf16x8 (&b)[D / 16],
                                          f32x16 (&acc)[MT]) {
  constexpr int KS = D / 16;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    acc[mt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(st.a[mt][ks], b[ks], acc[mt], 0, 0, 0);
  }
}

// This lane's partial sum over heads of w * relu(acc) for the tile's key
// (lane & 31): the lower half-wave holds half of the heads, the upper half
// the other half.
template <int D, int MT>
__device__ __forceinline__ float tile_partial(const RowState<D, MT>& st,
                                              const f32x16 (&acc)[MT]) {
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      s0 += st.wv[mt][v] * fmaxf(acc[mt][v], 0.0f);
      s1 += st.wv[mt][v + 1] * fmaxf(acc[mt][v + 1], 0.0f);
    }
  }
  return s0 + s1;
}

// Scores of two consecutive tiles from their partials: one
// v_permlane32_swap brings tile a's upper-half partials to its lower half and
// tile b's lower-half partials to its upper half, so one add leaves lane l
// with the score of key l of the 64 keys the two tiles cover (a's 32, then
// b's).  Each score is the lower-half plus the upper-half partial, the same
// two operands whichever tile pairing is used.  A swap runs in the VALU; a
// shuffle would go through the LDS pipeline, whose in-order counter would
// make this wait for the B-fragment reads just issued for the next tile.
__device__ __forceinline__ float pair_scores(float a, float b) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// One wave, one row, keys [c0, c1) read straight from global memory (key j
// at position j * stride).  Two register buffers alternate roles (the loop
// is unrolled by two tiles), so the next tile's load is always in flight
// while one is multiplied.  emit(score, key) takes the scores of 64
// consecutive keys, key t0 + lane at lane `lane`; tick() runs after every
// 64 keys.
template <int D, int MT, class Emit, class Tick>
__device__ void row_direct(const RowState<D, MT>& st, const uint16_t* __restrict__ k_idx,
                           const RowInfo& ri, int stride, int32_t c0, int32_t c1, int col,
                           int half, Emit emit, Tick tick) {
  constexpr int KS = D / 16, HALF = D / 2;
  const uint16_t* kbase = k_idx + ri.key_base * D + half * HALF;
  const int32_t last = visible_keys(ri.pos, stride) - 1;
  const int lane = lane_id();
  auto fetch = [&](bf16x8 (&dst)[KS], int32_t t0) {
    const int64_t key_ld = static_cast<int64_t>(min(t0 + col, last)) * stride;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) dst[ks] = load_bf16x8(kbase + key_ld * D + ks * 8);
  };
  bf16x8 x[KS], y[KS];
  fetch(x, c0);
  fetch(y, c0 + 32);
  for (int32_t t0 = c0; t0 < c1; t0 += 64) {
    f32x16 acc[MT];
    tile_mfma<D, MT>(st, x, acc);
    fetch(x, t0 + 64);
    const float pa = tile_partial<D, MT>(st, acc);
    tile_mfma<D, MT>(st, y, acc);
    fetch(y, t0 + 96);
    emit(pair_scores(pa, tile_partial<D, MT>(st, acc)), t0 + lane);
    tick();
  }
}

}  // namespace core
}  // namespace dsa
