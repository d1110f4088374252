// index_scores.hip -- Lightning-Indexer scores on gfx950 MFMA.
//
// I[t, s] = sum_h w[t, h] * max(0, qI[t, h, :] . kI[s, :])  for s = 0..p(t)
// (Keye-VL-2.0 report summary, page 5 section 1: a lightweight scout scores
// every position with one MQA key shared by all of its heads.)
//
// Mapping.  For one query row the head-by-key product is a small GEMM with
// M = indexer heads (up to 64), N = keys, K = d_idx.  Heads sit on the MFMA
// rows so that after v_mfma_f32_32x32x16_bf16 every lane holds one key column
// and 16 heads of it: the ReLU, the weight and the head sum happen in
// registers, and one exchange between the two half-waves finishes the sum.
// The contraction over d_idx is ordered so that each half-wave reads one
// contiguous half of every qI / kI row (64 B or 128 B per lane), which keeps
// every global load a full 16-byte vector.
//
// One wave owns one query row; a workgroup's four waves own four consecutive
// rows and walk the same key tiles, so the shared kI tile is served from the
// CU's L1 after the first wave touches it.  The grid's second dimension splits
// long rows into key chunks so that a handful of rows (decode) still spreads
// over the whole chip.
#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kRowsPerBlock = 4;

template <int D>
__global__ __launch_bounds__(256) void index_scores_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx,
    const float* __restrict__ w, int n_heads, int64_t row_begin, int64_t row_count,
    float* __restrict__ scores, int64_t ld, int key_chunk) {
  constexpr int KS = D / 16;   // MFMA k-steps over d_idx
  constexpr int HALF = D / 2;  // d range of one half-wave
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  // Later rows have longer causal prefixes: hand them out first.
  const int64_t blk = static_cast<int64_t>(gridDim.x) - 1 - blockIdx.x;
  const int64_t local = blk * kRowsPerBlock + wave;
  if (local >= row_count) return;
  const int64_t row = row_begin + local;
  const RowInfo ri = row_info(cu_q, cu_k, batch, row);
  const int32_t c0 = blockIdx.y * key_chunk;
  const int32_t c1 = min(c0 + key_chunk, ri.pos + 1);
  if (c0 >= c1) return;

  const int col = lane & 31;   // MFMA row (A) / column (B) owned by this lane
  const int half = lane >> 5;  // which half of d_idx this lane feeds
  const int m_tiles = (n_heads + 31) / 32;

  // Stationary operand: this row's indexer queries, heads on MFMA rows.
  bf16x8 a[2][KS];
  float wv[2][16];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int h = mt * 32 + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      a[mt][ks] = (mt < m_tiles && h < n_heads)
                      ? load_bf16x8(q_idx + (row * n_heads + h) * D + half * HALF + ks * 8)
                      : zero_bf16x8();
    }
    // Accumulator element v of this lane is MFMA row 8*(v/4) + 4*half + v%4.
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int hr = mt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      wv[mt][v] = (mt < m_tiles && hr < n_heads) ? w[row * n_heads + hr] : 0.0f;
    }
  }

  float* out_row = scores + local * ld;
  const uint16_t* kbase = k_idx + ri.key_base * D + half * HALF;
  for (int32_t t0 = c0; t0 < c1; t0 += 32) {
    const int32_t key = t0 + col;
    const int32_t key_ld = min(key, ri.pos);  // stay inside the sequence
    bf16x8 b[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) b[ks] = load_bf16x8(kbase + static_cast<int64_t>(key_ld) * D + ks * 8);
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][ks], b[ks], acc0, 0, 0, 0);
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) s += wv[0][v] * fmaxf(acc0[v], 0.0f);
    if (m_tiles > 1) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][ks], b[ks], acc1, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 16; ++v) s += wv[1][v] * fmaxf(acc1[v], 0.0f);
    }
    s += __shfl_xor(s, 32);
    if (half == 0 && key < c1) out_row[key] = s;
  }
}

}  // namespace

hipError_t launch_index_scores(const dsa_varlen& vl, const uint16_t* q_idx, const uint16_t* k_idx,
                               const float* w, int n_heads, int d, int64_t row_begin,
                               int64_t row_count, float* scores, int64_t ld, hipStream_t stream) {
  // A long row is split into chunks when there are too few rows to fill the
  // chip (decode); prefill windows keep whole rows per wave.
  const int64_t blocks_x = (row_count + kRowsPerBlock - 1) / kRowsPerBlock;
  int key_chunk = vl.max_seqlen_k;
  if (blocks_x < 2048) {
    const int64_t want_chunks = (4096 + blocks_x - 1) / blocks_x;
    int64_t c = (vl.max_seqlen_k + want_chunks - 1) / want_chunks;
    c = ((c + 31) / 32) * 32;
    key_chunk = static_cast<int>(c < 256 ? 256 : c);
  }
  key_chunk = ((key_chunk + 31) / 32) * 32;
  const int chunks = (vl.max_seqlen_k + key_chunk - 1) / key_chunk;
  dim3 grid(static_cast<unsigned>(blocks_x), static_cast<unsigned>(chunks));
  dim3 block(256);
  if (d == 128) {
    hipLaunchKernelGGL(index_scores_kernel<128>, grid, block, 0, stream, vl.cu_seqlens_q,
                       vl.cu_seqlens_k, vl.batch, q_idx, k_idx, w, n_heads, row_begin, row_count,
                       scores, ld, key_chunk);
  } else {
    hipLaunchKernelGGL(index_scores_kernel<64>, grid, block, 0, stream, vl.cu_seqlens_q,
                       vl.cu_seqlens_k, vl.batch, q_idx, k_idx, w, n_heads, row_begin, row_count,
                       scores, ld, key_chunk);
  }
  return hipGetLastError();
}

}  // namespace dsa
