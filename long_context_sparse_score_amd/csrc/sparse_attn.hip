// sparse_attn.hip -- GQA attention restricted to each query's selected positions.
//
// O[t, h] = sum_{s in Sel(t)} softmax_s(scale * Q[t, h] . K[s, g]) V[s, g],
// g = h / (Hq / Hkv), with one index set Sel(t) per query token shared by
// every query head (Keye-VL-2.0 report summary, page 5 section 1: attention
// only over the chosen positions; the GQA adaptation paragraph).
//
// Workgroup = one query row (or one slice of its index list when the list is
// split, for decode).  Wave g = KV head g with its Hq/Hkv query heads.  The
// selected rows are gathered straight from HBM: a key row of one KV head is
// contiguous (head_dim * 2 bytes), and each lane loads 16-byte pieces of it.
//
// Per tile of 32 selected positions:
//   S^T = K_sel Q^T on v_mfma_f32_16x16x32_bf16 (keys on MFMA rows, query
//   heads on columns, padded to 16), online softmax per head in fp32
//   (exp2 with log2(e) folded into the scale), then O += P V_sel on the same
//   MFMA.  The contraction order of the P V product is chosen so that every
//   lane's probabilities are already in place as the A operand; V goes
//   through LDS because its B operand needs 8 consecutive keys per lane.
#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct AttnCfg {
  static constexpr int KS = D / 32;       // k-steps of the S product
  static constexpr int QD = D / 4;        // d range of one lane quarter
  static constexpr int DT = D / 16;       // 16-wide d tiles of the O product
  static constexpr int VSTRIDE = D + 4;   // LDS row stride (bf16), spreads banks
  static constexpr int VTILE = 32 * VSTRIDE;
};

// Rows of one 32-slot tile gathered by one lane: slot 16*sub + col, d range
// of lane quarter qd, for K (kept as the A operand) and V (staged to LDS).
template <int D>
struct GatherTile {
  bf16x8 k[2][AttnCfg<D>::KS];
  u32x4 v[2][AttnCfg<D>::KS];
  bool ok[2];  // slot holds a usable position (inside the list, 0 <= p <= pos)
};

template <int D>
__device__ __forceinline__ void gather_tile(GatherTile<D>& t, const int32_t* idx, int s0,
                                            int n_slots, const RowInfo& ri,
                                            const uint16_t* __restrict__ k,
                                            const uint16_t* __restrict__ v, int n_heads_kv, int g,
                                            int col, int qd) {
  using C = AttnCfg<D>;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int slot = s0 + 16 * sub + col;
    const int32_t p = slot < n_slots ? idx[slot] : -1;
    t.ok[sub] = p >= 0 && p <= ri.pos;
    const int64_t krow = ri.key_base + (t.ok[sub] ? p : 0);
    const int64_t off = (krow * n_heads_kv + g) * D + qd * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      t.k[sub][ks] = load_bf16x8(k + off + ks * 32);
      t.v[sub][ks] = *reinterpret_cast<const u32x4*>(v + off + ks * 32);
    }
  }
}

// Online-softmax update of one tile.  m_run / l_run / acc are this lane's
// running state (head col; O rows = heads 4 qd + r).
template <int D>
__device__ __forceinline__ void attend_tile(const GatherTile<D>& t, const bf16x8 (&qb)[AttnCfg<D>::KS],
                                            uint16_t* vs, float scale_log2, int col, int qd,
                                            float& m_run, float& l_run,
                                            f32x4 (&acc)[AttnCfg<D>::DT]) {
  using C = AttnCfg<D>;
  // V rows to this wave's LDS tile (read back below in the B-operand order).
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      uint16_t* dst = vs + (16 * sub + col) * C::VSTRIDE + ks * 32 + qd * 8;
      reinterpret_cast<uint2*>(dst)[0] = make_uint2(t.v[sub][ks].x, t.v[sub][ks].y);
      reinterpret_cast<uint2*>(dst)[1] = make_uint2(t.v[sub][ks].z, t.v[sub][ks].w);
    }
  // Bit j of vm[sub] says whether slot 16*sub + j holds a usable position.
  const unsigned long long vm0 = __ballot(t.ok[0]) & 0xFFFFull;
  const unsigned long long vm1 = __ballot(t.ok[1]) & 0xFFFFull;

  // S^T tiles: rows = slots 16*sub + 4*qd + r, column = head col.
  f32x4 st[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    st[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      st[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[sub][ks], qb[ks], st[sub], 0, 0, 0);
  }
  float z[2][4];
  float mx = -INFINITY;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const unsigned long long vm = sub ? vm1 : vm0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = (vm >> (4 * qd + r)) & 1ull;
      z[sub][r] = ok ? st[sub][r] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, z[sub][r]);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(m_run, mx);
  const float corr = m_new == -INFINITY ? 1.0f : exp2f(m_run - m_new);
  float pr[2][4];
  float psum = 0.0f;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[sub][r] = z[sub][r] == -INFINITY ? 0.0f : exp2f(z[sub][r] - m_new);
      psum += pr[sub][r];
    }
  l_run = l_run * corr + psum;
  m_run = m_new;

  // P as the A operand: row = head col, contraction index 8*qd + i maps to
  // slot 4*qd + i (i < 4) and 16 + 4*qd + i - 4 (i >= 4).
  uint4 pa_u;
  pa_u.x = pack_bf16x2(pr[0][0], pr[0][1]);
  pa_u.y = pack_bf16x2(pr[0][2], pr[0][3]);
  pa_u.z = pack_bf16x2(pr[1][0], pr[1][1]);
  pa_u.w = pack_bf16x2(pr[1][2], pr[1][3]);
  const bf16x8 pa = __builtin_bit_cast(bf16x8, pa_u);

  // Rescale O rows (heads 4*qd + r) by their head's correction.
  float cr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * qd + r);
  // The V tile is private to this wave and LDS operations of one wave are
  // performed in order, so the reads below see the writes above.
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[dt][r] *= cr[r];
    const uint16_t* src = vs + dt * 16 + col;
    uint4 vb_u;
    const int r0 = 4 * qd, r1 = 16 + 4 * qd;
    vb_u.x = src[(r0 + 0) * C::VSTRIDE] | (static_cast<uint32_t>(src[(r0 + 1) * C::VSTRIDE]) << 16);
    vb_u.y = src[(r0 + 2) * C::VSTRIDE] | (static_cast<uint32_t>(src[(r0 + 3) * C::VSTRIDE]) << 16);
    vb_u.z = src[(r1 + 0) * C::VSTRIDE] | (static_cast<uint32_t>(src[(r1 + 1) * C::VSTRIDE]) << 16);
    vb_u.w = src[(r1 + 2) * C::VSTRIDE] | (static_cast<uint32_t>(src[(r1 + 3) * C::VSTRIDE]) << 16);
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, vb_u),
                                                      acc[dt], 0, 0, 0);
  }
}

template <int D>
__global__ __launch_bounds__(512) void sparse_attn_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ indices, int topk,
    int64_t row_begin, int64_t row_count, int n_heads_q, int n_heads_kv, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, int splits,
    float* __restrict__ partial) {
  using C = AttnCfg<D>;
  extern __shared__ uint16_t vs_all[];
  const int lane = lane_id();
  const int g = threadIdx.x / kWave;  // KV head of this wave
  const int G = n_heads_q / n_heads_kv;
  const int col = lane & 15;
  const int qd = lane >> 4;
  const int64_t local = row_count - 1 - static_cast<int64_t>(blockIdx.x);
  const int64_t row = row_begin + local;
  const int split = blockIdx.y;
  const RowInfo ri = row_info(cu_q, cu_k, batch, row);
  const int per_split = (topk + splits - 1) / splits;
  const int i0 = split * per_split;
  const int n_slots = max(0, min(topk, i0 + per_split) - i0);
  uint16_t* vs = vs_all + g * C::VTILE;
  // This slice of the row's index list, shared by all KV heads, in LDS.
  int32_t* idx = reinterpret_cast<int32_t*>(vs_all + n_heads_kv * C::VTILE);
  const int32_t* irow = indices + local * topk + i0;
  for (int s = threadIdx.x; s < n_slots; s += blockDim.x) idx[s] = irow[s];

  // Q^T as the B operand: column = query head of this group, contraction d
  // ordered so that lane quarter qd covers d in [qd*QD, qd*QD + QD).
  bf16x8 qb[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    qb[ks] = col < G ? load_bf16x8(q + ((row * n_heads_q) + g * G + col) * D + ks * 32 + qd * 8)
                     : zero_bf16x8();

  f32x4 acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max (log2 domain) of head `col`
  float l_run = 0.0f;       // this lane's share of the running denominator
  __syncthreads();          // index list in LDS

  // Two tiles in flight: the next tile's rows are gathered while this one
  // is multiplied (the loop is unrolled by two so each tile keeps its
  // registers).  Tiles past the list gather valid rows and contribute zero.
  GatherTile<D> ta, tb;
  gather_tile<D>(ta, idx, 0, n_slots, ri, k, v, n_heads_kv, g, col, qd);
  for (int s0 = 0; s0 < n_slots; s0 += 64) {
    gather_tile<D>(tb, idx, s0 + 32, n_slots, ri, k, v, n_heads_kv, g, col, qd);
    attend_tile<D>(ta, qb, vs, scale_log2, col, qd, m_run, l_run, acc);
    gather_tile<D>(ta, idx, s0 + 64, n_slots, ri, k, v, n_heads_kv, g, col, qd);
    attend_tile<D>(tb, qb, vs, scale_log2, col, qd, m_run, l_run, acc);
  }

  // Full denominator of head `col`: sum the four lane quarters.
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  float lr[4], mr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    lr[r] = __shfl(l_tot, 4 * qd + r);
    mr[r] = __shfl(m_run, 4 * qd + r);
  }
  if (splits == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * qd + r;
      if (h >= G) continue;
      const int hq = g * G + h;
      const float inv = lr[r] > 0.0f ? 1.0f / lr[r] : 0.0f;
      uint16_t* orow = out + (row * n_heads_q + hq) * D;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
        orow[dt * 16 + col] = static_cast<uint16_t>(f32_to_bf16_bits(acc[dt][r] * inv));
      if (lse != nullptr && col == 0)
        lse[row * n_heads_q + hq] = lr[r] > 0.0f ? (mr[r] + log2f(lr[r])) * kLn2 : -INFINITY;
    }
  } else {
    // Unnormalised partial: per head D accumulator values, then m and l.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * qd + r;
      if (h >= G) continue;
      const int hq = g * G + h;
      float* pp = partial + ((local * splits + split) * n_heads_q + hq) * (D + 2);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) pp[dt * 16 + col] = acc[dt][r];
      if (col == 0) {
        pp[D] = mr[r];
        pp[D + 1] = lr[r];
      }
    }
  }
}

// Merge split partials in split order: one thread per (row, head, d).
template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(const float* __restrict__ partial,
                                                        int splits, int n_heads_q,
                                                        int64_t row_begin, uint16_t* __restrict__ out,
                                                        float* __restrict__ lse) {
  const int64_t local = blockIdx.x;
  const int hq = blockIdx.y;
  const int d = threadIdx.x;
  float m = -INFINITY;
  for (int s = 0; s < splits; ++s)
    m = fmaxf(m, partial[((local * splits + s) * n_heads_q + hq) * (D + 2) + D]);
  float num = 0.0f, den = 0.0f;
  if (m != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const float* pp = partial + ((local * splits + s) * n_heads_q + hq) * (D + 2);
      const float ms = pp[D];
      if (ms == -INFINITY) continue;
      const float f = exp2f(ms - m);
      num += pp[d] * f;
      den += pp[D + 1] * f;
    }
  }
  const int64_t row = row_begin + local;
  const float o = den > 0.0f ? num / den : 0.0f;
  out[(row * n_heads_q + hq) * D + d] = static_cast<uint16_t>(f32_to_bf16_bits(o));
  if (lse != nullptr && d == 0) lse[row * n_heads_q + hq] = den > 0.0f ? (m + log2f(den)) * kLn2 : -INFINITY;
}

}  // namespace

size_t attn_workspace_bytes(int64_t rows, int n_heads_q, int head_dim, int splits) {
  if (splits <= 1) return 0;
  return static_cast<size_t>(rows) * splits * n_heads_q * (head_dim + 2) * sizeof(float);
}

int attn_decode_splits(int64_t rows, int n_heads_kv, int topk) {
  // About one workgroup per CU, each holding at least two 32-slot tiles:
  // more splits only add partial results to merge (measured at 64 rows x
  // 2048 slots: 4 splits 49 us, 8 splits 54 us, 16 splits 61 us).
  int splits = 1;
  while (rows * splits < 256 && (topk + 2 * splits - 1) / (2 * splits) >= 64) splits *= 2;
  (void)n_heads_kv;
  return splits;
}

hipError_t launch_sparse_attn(const dsa_varlen& vl, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const int32_t* indices, int topk,
                              int64_t row_begin, int64_t row_count, int n_heads_q, int n_heads_kv,
                              int head_dim, float scale, uint16_t* out, float* lse, int splits,
                              float* partial, hipStream_t stream) {
  const float scale_log2 = scale * kLog2e;
  dim3 grid(static_cast<unsigned>(row_count), static_cast<unsigned>(splits));
  dim3 block(kWave * n_heads_kv);
  if (head_dim == 128) {
    const size_t lds = n_heads_kv * AttnCfg<128>::VTILE * sizeof(uint16_t) +
                       static_cast<size_t>((topk + splits - 1) / splits) * sizeof(int32_t);
    hipLaunchKernelGGL(sparse_attn_kernel<128>, grid, block, lds, stream, vl.cu_seqlens_q,
                       vl.cu_seqlens_k, vl.batch, q, k, v, indices, topk, row_begin, row_count,
                       n_heads_q, n_heads_kv, scale_log2, out, lse, splits, partial);
  } else {
    const size_t lds = n_heads_kv * AttnCfg<64>::VTILE * sizeof(uint16_t) +
                       static_cast<size_t>((topk + splits - 1) / splits) * sizeof(int32_t);
    hipLaunchKernelGGL(sparse_attn_kernel<64>, grid, block, lds, stream, vl.cu_seqlens_q,
                       vl.cu_seqlens_k, vl.batch, q, k, v, indices, topk, row_begin, row_count,
                       n_heads_q, n_heads_kv, scale_log2, out, lse, splits, partial);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || splits == 1) return err;
  dim3 mgrid(static_cast<unsigned>(row_count), static_cast<unsigned>(n_heads_q));
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_merge_kernel<128>, mgrid, dim3(128), 0, stream, partial, splits,
                       n_heads_q, row_begin, out, lse);
  else
    hipLaunchKernelGGL(attn_merge_kernel<64>, mgrid, dim3(64), 0, stream, partial, splits,
                       n_heads_q, row_begin, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
