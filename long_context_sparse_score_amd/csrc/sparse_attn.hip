// sparse_attn.hip -- GQA attention restricted to each query's selected positions.
//
// O[t, h] = sum_{s in Sel(t)} softmax_s(scale * Q[t, h] . K[s, g]) V[s, g],
// g = h / (Hq / Hkv), with one index set Sel(t) per query token shared by
// every query head (Keye-VL-2.0 report summary, page 5 section 1: attention
// only over the chosen positions; the GQA adaptation paragraph).
//
// Workgroup = one query row (or one slice of its index list when the list is
// split, for decode).  Wave g = KV head g with its Hq/Hkv query heads.  The
// selected rows are gathered straight from HBM, whole rows per load
// instruction (a key row of one KV head is head_dim * 2 contiguous bytes),
// and staged through the wave's own LDS tiles.
//
// Per tile of 32 selected positions:
//   S^T = K_sel Q^T on v_mfma_f32_16x16x32_bf16 (keys on MFMA rows, query
//   heads on columns, padded to 16), online softmax per head in fp32
//   (exp2 with log2(e) folded into the scale), then O += P V_sel on the same
//   MFMA.  The contraction order of the P V product is chosen so that every
//   lane's probabilities are already in place as the A operand; V's B
//   operand (8 consecutive keys of one column per lane) comes from LDS
//   through the transposing read.
#include <mutex>
#include <type_traits>

#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Growth of a head's maximum (log2 units) that the running softmax
// reference absorbs before it is moved (P terms stay below 2^8).
constexpr float kRescaleLog2 = 8.0f;

template <int D>
struct AttnCfg {
  static constexpr int KS = D / 32;           // k-steps of the S product
  static constexpr int QD = D / 4;            // d range of one lane quarter
  static constexpr int DT = D / 16;           // 16-wide d tiles of the O product
  static constexpr int PIECES = D / 8;        // 16-byte pieces of one K or V row
  static constexpr int RPI = kWave / PIECES;  // whole rows per gather instruction
  static constexpr int LPT = 32 / RPI;        // gather instructions per 32-slot tile
  static constexpr int TILE = 32 * D;         // elements of one K or V tile in LDS
  static_assert(RPI * PIECES == kWave && LPT * RPI == 32, "tile shape");
};

// One 32-slot tile of one KV head as gathered by one lane: lane l reads
// piece l % PIECES of the rows (l / PIECES) LPT + j, j < LPT, of K and V.
// Every gather instruction thus reads RPI whole rows (RPI x 2 D bytes,
// whole cache lines): reading the MFMA operand layout directly would touch
// 16 rows per instruction in 64-byte pieces, which halves the rate the
// memory path sustains for scattered rows.
template <int D>
struct GatherTile {
  u32x4 k[AttnCfg<D>::LPT];
  u32x4 v[AttnCfg<D>::LPT];
};

// kr / vr: buffer resources over this sequence's K and V rows, so a row is
// one 32-bit offset shared by its K and V loads.
template <int D>
__device__ __forceinline__ void gather_tile(GatherTile<D>& t, const int32_t* idx, int s0,
                                            __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                            int n_heads_kv, int g, int lane) {
  using C = AttnCfg<D>;
  const int q = lane / C::PIECES, piece = lane % C::PIECES;
#pragma unroll
  for (int j = 0; j < C::LPT; ++j) {
    // idx holds -1 past the slice.  A row outside 0..pos (-1 included:
    // (g - n_heads_kv) D 2 wraps to at least 2^32 - 2^31) lies past the
    // buffer's range and reads zeros; its slot is masked anyway.
    const int32_t p = idx[s0 + q * C::LPT + j];
    const uint32_t off = ((static_cast<uint32_t>(p) * n_heads_kv + g) * D + piece * 8) * 2;
    t.k[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0));
    t.v[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0));
  }
}

// Position of piece p of tile row r in LDS: pieces are XOR-swizzled by row,
// so both the row-wise stores and the column-wise operand reads below are
// free of bank conflicts.
template <int D>
__device__ __forceinline__ int tile_at(int r, int piece) {
  return r * D + ((piece ^ (r % AttnCfg<D>::PIECES)) * 8);
}

// Online-softmax update of one tile held in LDS.  m_run / l_run / acc are
// this lane's running state (query column col; O rows = columns 4 qd + r).
// vm: bit s says whether slot s of the tile is usable for this lane's column.
template <int D>
__device__ __forceinline__ void compute_tile(const bf16x8 (&qb)[AttnCfg<D>::KS],
                                             const uint16_t* ks_lds, const uint16_t* vs_lds,
                                             uint32_t vm, float scale_log2, int lane,
                                             float& m_run, float& l_run,
                                             f32x4 (&acc)[AttnCfg<D>::DT]) {
  using C = AttnCfg<D>;
  const int col = lane & 15, qd = lane >> 4;
  // S^T tiles: rows = slots 16*sub + 4*qd + r, column = head col.  A operand:
  // slot 16*sub + col, d range [32 ks + 8 qd, +8).
  f32x4 st[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    st[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 ka = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(ks_lds + tile_at<D>(16 * sub + col, 4 * ks + qd)));
      st[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[ks], st[sub], 0, 0, 0);
    }
  }
  float z[2][4];
  float mx = -INFINITY;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = (vm >> (16 * sub + 4 * qd + r)) & 1u;
      z[sub][r] = ok ? st[sub][r] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, z[sub][r]);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  // Lazy rescaling: the reference m_run (log2 domain) moves only when some
  // head's tile maximum exceeds it by more than kRescaleLog2, so most tiles
  // skip the rescale of l and O.  Otherwise P is taken against the older
  // reference (terms up to 2^kRescaleLog2); O, l and the log-sum-exp all
  // use the same reference, so the normalised result is unchanged.
  if (__any(mx > m_run + kRescaleLog2)) {
    const float m_new = fmaxf(m_run, mx);
    const float corr = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= corr;
    m_run = m_new;
    // O rows (heads 4*qd + r) take their head's correction.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float cr = __shfl(corr, 4 * qd + r);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) acc[dt][r] *= cr;
    }
  }
  // Masked slots hold -inf, whose exp2 is 0; a reference still at -inf
  // means every slot so far was masked, and 0 then serves as well.
  const float m_use = m_run == -INFINITY ? 0.0f : m_run;
  float pr[2][4];
  float psum = 0.0f;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[sub][r] = __builtin_amdgcn_exp2f(z[sub][r] - m_use);
      psum += pr[sub][r];
    }
  l_run += psum;

  // P as the A operand: row = head col, contraction index 8*qd + i maps to
  // slot 4*qd + i (i < 4) and 16 + 4*qd + i - 4 (i >= 4); converted with
  // round-to-nearest-even.
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  typedef __bf16 bf16x8n __attribute__((ext_vector_type(8)));
  const f32x8 pf = {pr[0][0], pr[0][1], pr[0][2], pr[0][3], pr[1][0], pr[1][1], pr[1][2], pr[1][3]};
  const bf16x8 pa = __builtin_bit_cast(bf16x8, __builtin_convertvector(pf, bf16x8n));

  // B operand: column d = 16 dt + col, rows = slots 4 qd + i and 16 + 4 qd + i
  // (i < 4), the order of P's contraction.  ds_read_b64_tr_b16 transposes
  // within each 16-lane group: lane t receives element t % 4 of the 4-element
  // rows addressed by lanes t / 4 + 4 i of its group.  So lane (col, qd)
  // addresses V[4 qd + col / 4][16 dt + 4 (col % 4), +4) -- 8 contiguous
  // bytes of one row -- and receives V[4 qd + i][16 dt + col], i < 4; a
  // second read does the same 16 slots further on.
  const int tr_row = 4 * qd + (col >> 2);
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    const int d0 = dt * 16 + 4 * (col & 3);
    const int piece = d0 / 8, e = d0 % 8;
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(vs_lds + tile_at<D>(tr_row, piece) + e));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(vs_lds + tile_at<D>(16 + tr_row, piece) + e));
    const bf16x8 vb = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi),
                                              0, 1, 2, 3, 4, 5, 6, 7);
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, acc[dt], 0, 0, 0);
  }
}

// Online-softmax update of two tiles at once (64 slots: tile 0 from
// ks0/vs0 with validity vm0, tile 1 from ks1/vs1 with vm1), the same
// arithmetic as two compute_tile calls except that one reference update
// covers both: the four S sub-products are independent, and so are the two
// P V products, which gives the wave more work in flight per step.
template <int D>
__device__ __forceinline__ void compute_tile_pair(const bf16x8 (&qb)[AttnCfg<D>::KS],
                                                  const uint16_t* ks0, const uint16_t* vs0,
                                                  uint32_t vm0, const uint16_t* ks1,
                                                  const uint16_t* vs1, uint32_t vm1,
                                                  float scale_log2, int lane, float& m_run,
                                                  float& l_run, f32x4 (&acc)[AttnCfg<D>::DT]) {
  using C = AttnCfg<D>;
  const int col = lane & 15, qd = lane >> 4;
  const uint16_t* ks[2] = {ks0, ks1};
  const uint16_t* vs[2] = {vs0, vs1};
  const uint32_t vm[2] = {vm0, vm1};
  f32x4 st[2][2];
#pragma unroll
  for (int tl = 0; tl < 2; ++tl)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      st[tl][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < C::KS; ++k) {
        const bf16x8 ka = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(ks[tl] + tile_at<D>(16 * sub + col, 4 * k + qd)));
        st[tl][sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[k], st[tl][sub], 0, 0, 0);
      }
    }
  float z[2][2][4];
  float mx = -INFINITY;
#pragma unroll
  for (int tl = 0; tl < 2; ++tl)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = (vm[tl] >> (16 * sub + 4 * qd + r)) & 1u;
        z[tl][sub][r] = ok ? st[tl][sub][r] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, z[tl][sub][r]);
      }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (__any(mx > m_run + kRescaleLog2)) {
    const float m_new = fmaxf(m_run, mx);
    const float corr = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= corr;
    m_run = m_new;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float cr = __shfl(corr, 4 * qd + r);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) acc[dt][r] *= cr;
    }
  }
  const float m_use = m_run == -INFINITY ? 0.0f : m_run;
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  typedef __bf16 bf16x8n __attribute__((ext_vector_type(8)));
  bf16x8 pa[2];
  float psum = 0.0f;
#pragma unroll
  for (int tl = 0; tl < 2; ++tl) {
    float pr[2][4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[sub][r] = __builtin_amdgcn_exp2f(z[tl][sub][r] - m_use);
        psum += pr[sub][r];
      }
    const f32x8 pf = {pr[0][0], pr[0][1], pr[0][2], pr[0][3], pr[1][0], pr[1][1], pr[1][2], pr[1][3]};
    pa[tl] = __builtin_bit_cast(bf16x8, __builtin_convertvector(pf, bf16x8n));
  }
  l_run += psum;
  // B operands as in compute_tile (transposing reads), for each tile.
  const int tr_row = 4 * qd + (col >> 2);
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    const int d0 = dt * 16 + 4 * (col & 3);
    const int piece = d0 / 8, e = d0 % 8;
    typedef short v4i16 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) {
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(vs[tl] + tile_at<D>(tr_row, piece) + e));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(vs[tl] + tile_at<D>(16 + tr_row, piece) + e));
      const bf16x8 vb = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                                __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4, 5, 6, 7);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[tl], vb, acc[dt], 0, 0, 0);
    }
  }
}

// A wave's own tile: its K and V rows to its private LDS tiles, then the
// update.  LDS operations of one wave are performed in order, so the reads
// see these writes and the next tile's writes come after them.
template <int D>
__device__ __forceinline__ void attend_tile(const GatherTile<D>& t, const bf16x8 (&qb)[AttnCfg<D>::KS],
                                            uint16_t* ks_lds, uint16_t* vs_lds, uint32_t vm,
                                            float scale_log2, int lane, float& m_run,
                                            float& l_run, f32x4 (&acc)[AttnCfg<D>::DT]) {
  using C = AttnCfg<D>;
  {
    const int q = lane / C::PIECES, piece = lane % C::PIECES;
#pragma unroll
    for (int j = 0; j < C::LPT; ++j) {
      const int at = tile_at<D>(q * C::LPT + j, piece);
      *reinterpret_cast<u32x4*>(ks_lds + at) = t.k[j];
      *reinterpret_cast<u32x4*>(vs_lds + at) = t.v[j];
    }
  }
  compute_tile<D>(qb, ks_lds, vs_lds, vm, scale_log2, lane, m_run, l_run, acc);
}

// Entries of the LDS index slice: the slice rounded up to 64 plus the 64
// that the look-ahead gather reads past it, all -1 beyond the slice.
__host__ __device__ constexpr int attn_idx_entries(int per_split) {
  return (per_split + 63) / 64 * 64 + 64;
}

// LDS of one workgroup: K and V tiles of every KV head, the slice of the
// index list, and one validity word per 32 slots.
template <int D>
__host__ __device__ constexpr size_t attn_lds_bytes(int n_heads_kv, int per_split) {
  return static_cast<size_t>(2 * n_heads_kv) * AttnCfg<D>::TILE * sizeof(uint16_t) +
         static_cast<size_t>(attn_idx_entries(per_split)) * sizeof(int32_t) +
         static_cast<size_t>((per_split + 63) / 64 * 2) * sizeof(uint32_t);
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
  extern __shared__ __attribute__((aligned(16))) uint16_t lds_all[];
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
  uint16_t* ks_lds = lds_all + g * C::TILE;
  uint16_t* vs_lds = lds_all + (n_heads_kv + g) * C::TILE;
  // This slice of the row's index list, shared by all KV heads, in LDS, and
  // a bitmask of its usable slots (0 <= p <= pos), one word per 32 slots.
  const int n_idx = attn_idx_entries(per_split);
  int32_t* idx = reinterpret_cast<int32_t*>(lds_all + 2 * n_heads_kv * C::TILE);
  uint32_t* vbits = reinterpret_cast<uint32_t*>(idx + n_idx);
  const int32_t* irow = indices + local * topk + i0;
  const int n_pad = (n_slots + 63) & ~63;
  for (int base = 0; base < n_pad + 64; base += static_cast<int>(blockDim.x)) {
    const int s = base + static_cast<int>(threadIdx.x);
    const int32_t p = s < n_slots ? irow[s] : -1;
    if (s < n_pad + 64) idx[s] = p;
    const unsigned long long ok = __ballot(p >= 0 && p <= ri.pos);
    const int w0 = base + (static_cast<int>(threadIdx.x) & ~(kWave - 1));
    if (lane == 0 && w0 < n_pad) {
      vbits[w0 / 32] = static_cast<uint32_t>(ok);
      vbits[w0 / 32 + 1] = static_cast<uint32_t>(ok >> 32);
    }
  }

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
  __syncthreads();          // index list and validity words in LDS

  // Two tiles in flight: the next tile's rows are gathered while this one
  // is multiplied (the loop is unrolled by two so each tile keeps its
  // registers).  Tiles past the list gather valid rows and contribute zero.
  // The sequence's visible K and V rows (keys 0..pos; the host checks that a
  // sequence's cache fits 32-bit offsets).
  const int seq_bytes = (ri.pos + 1) * n_heads_kv * D * 2;
  const __amdgpu_buffer_rsrc_t kr = raw_buffer(k + ri.key_base * n_heads_kv * D, seq_bytes);
  const __amdgpu_buffer_rsrc_t vr = raw_buffer(v + ri.key_base * n_heads_kv * D, seq_bytes);
  GatherTile<D> ta, tb;
  gather_tile<D>(ta, idx, 0, kr, vr, n_heads_kv, g, lane);
  for (int s0 = 0; s0 < n_slots; s0 += 64) {
    gather_tile<D>(tb, idx, s0 + 32, kr, vr, n_heads_kv, g, lane);
    attend_tile<D>(ta, qb, ks_lds, vs_lds, vbits[s0 / 32], scale_log2, lane, m_run, l_run, acc);
    gather_tile<D>(ta, idx, s0 + 64, kr, vr, n_heads_kv, g, lane);
    attend_tile<D>(tb, qb, ks_lds, vs_lds, vbits[s0 / 32 + 1], scale_log2, lane, m_run, l_run, acc);
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

// ---------------------------------------------------------------- grouped prefill
//
// Adjacent query rows select largely the same positions when their queries
// are alike (page 5 section 8: the index sets of 16 adjacent queries are
// de-duplicated before attention).  A group of kGroupRows consecutive rows
// of the window is served from the union of their index sets: each K/V row
// of the union is gathered once for the group, and a per-(row, position)
// mask restricts every query to its own set, so each query's result is the
// one of its own set.
//
// Pass 1 (union_kernel, one workgroup per group, wave r holding row r's
// index list in registers): the union as packed key rows (sequence key base
// + position) with a 16-bit row mask per entry, in the caller's workspace,
// in the order described below.
// Pass 2 (grouped_attn_kernel, one workgroup per (group, KV head), one wave
// per 16 of the group's 16 * G queries): every union tile of 32 entries is
// gathered into LDS by the whole workgroup and used by the waves whose rows
// own one of its entries, with the tile update of the per-row kernel and the
// validity bits taken from the masks.
//
// The order.  Wave w of pass 2 serves rows w 16/G .. (w + 1) 16/G - 1, so an
// entry's wave byte (bit w set when one of those rows owns it) says which
// waves compute a tile holding it.  Most entries belong to few rows (on a
// workload whose 16 adjacent queries draw about 10000 distinct positions,
// 41% of them belong to one row only), so in key order nearly every tile
// holds an entry of every wave, and each wave computes every tile.  Sorted
// by the Gray-code rank of the wave byte, neighbouring entries share their
// byte or differ in one wave, and a tile is computed by the 2 to 4 waves
// that need it (measured on such groups: 950 wave-tiles instead of 2400 per
// group and KV head, against 1024 for 16 rows of 64 tiles each).  Ties keep
// key order, so the order is a function of the index sets alone.

constexpr int kGroupRows = 16;
constexpr int kUnionThreads = kGroupRows * kWave;  // wave r: row r of the group
constexpr int kUnionHeld = 2048;                   // index entries a wave holds in registers
constexpr int kUnionEntries = kGroupRows * kUnionHeld;  // masks one span can hold
constexpr int kUnionSpan = 131072;                 // packed keys per span (presence bits)
constexpr int kUnionBuckets = 256;                 // sort keys: up to 8 waves in pass 2

// Workspace of the grouped path for `groups` groups: union keys (int32), row
// masks (uint16), one count per group, then each group's keys in key order
// (staging for the union pass's scatter).
struct GroupedWorkspace {
  int32_t* keys;
  uint16_t* masks;
  int32_t* counts;
  int32_t* stage;
  int32_t* order;
};

__host__ __device__ inline size_t grouped_ws_entries(int topk) {
  return static_cast<size_t>(kGroupRows) * topk;
}

inline size_t round256(size_t n) { return (n + 255) / 256 * 256; }

inline GroupedWorkspace grouped_ws_layout(void* base, int64_t groups, int topk) {
  char* p = static_cast<char*>(base);
  GroupedWorkspace w;
  const size_t n = static_cast<size_t>(groups) * grouped_ws_entries(topk);
  w.keys = reinterpret_cast<int32_t*>(p);
  p += round256(n * sizeof(int32_t));
  w.masks = reinterpret_cast<uint16_t*>(p);
  p += round256(n * sizeof(uint16_t));
  w.counts = reinterpret_cast<int32_t*>(p);
  p += round256(static_cast<size_t>(groups) * sizeof(int32_t));
  w.stage = reinterpret_cast<int32_t*>(p);
  p += round256(n * sizeof(int32_t));
  w.order = reinterpret_cast<int32_t*>(p);
  return w;
}

// Sort key of a union entry: the Gray-code rank (prefix XOR) of its wave
// byte, for `waves` waves of 16 / waves rows each.
template <int waves>
__device__ __forceinline__ int union_bucket(uint32_t mask) {
  // The wave byte: OR each wave's rows into its lowest row bit, then pack
  // those bits (waves is 8, 4, 2 or 1: 2, 4, 8 or 16 rows a wave).
  uint32_t b;
  if constexpr (waves == 8) {
    b = (mask | (mask >> 1)) & 0x5555u;
    b = (b | (b >> 1)) & 0x3333u;
    b = (b | (b >> 2)) & 0x0F0Fu;
    b = (b | (b >> 4)) & 0x00FFu;
  } else if constexpr (waves == 4) {
    b = mask | (mask >> 1);
    b = (b | (b >> 2)) & 0x1111u;
    b = (b | (b >> 3)) & 0x0303u;
    b = (b | (b >> 6)) & 0x000Fu;
  } else if constexpr (waves == 2) {
    b = ((mask & 0x00FFu) != 0u ? 1u : 0u) | ((mask & 0xFF00u) != 0u ? 2u : 0u);
  } else {
    b = mask != 0u ? 1u : 0u;
  }
  b ^= b >> 1;
  b ^= b >> 2;
  b ^= b >> 4;
  return static_cast<int>(b);
}

// Lanes of this wave holding the same 8-bit key (among the lanes with `in`).
__device__ __forceinline__ unsigned long long same_key_lanes(int key, bool in) {
  unsigned long long peers = __ballot(in);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (key >> b) & 1;
    const unsigned long long set = __ballot(in && bit);
    peers &= bit ? set : ~set;
  }
  return peers;
}

// Exclusive prefix sum over the first `n` threads' values (n a multiple of
// kWave, at most kUnionThreads); every thread gets the total.  Two barriers;
// `wsum` holds kUnionThreads / kWave ints.
__device__ __forceinline__ int union_scan(int x, int n, int* wsum, int& total) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  int incl = tid < n ? x : 0;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1 && tid < n) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
  for (int w = 0; w < n / kWave; ++w) {
    before += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  __syncthreads();  // wsum is free again
  return before + incl - (tid < n ? x : 0);
}

// Pass 1.  The packed-key range of the group's rows is covered by spans of
// kUnionSpan keys when every row holds at most kUnionHeld entries (so a
// span's union fits the kUnionEntries masks), else of kUnionEntries keys.
// Per span: every wave marks its row's keys in a presence bitmap; a prefix
// count over the bitmap gives each key its rank within the span; every wave
// then ORs its row bit into the 16-bit mask at its keys' ranks.  Counting
// the entries of every sort key over all spans and a prefix sum over the
// sort keys give where each sort key's entries start in the output; then
// each span (rebuilt when there is more than one) is scattered in key order
// to its sort keys' next places: wave w takes a consecutive share of the
// span's entries (its counts per sort key, then the offsets over all waves,
// then the writes; an entry's key is read back by rank from a staging copy
// that the mask step writes).  Only integers are summed, so the
// result does not depend on timing, and the index lists need no order.
template <int waves>
__global__ __launch_bounds__(kUnionThreads) void union_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const int32_t* __restrict__ indices, int topk, int64_t row_begin, int64_t row_count,
    int32_t* __restrict__ ukeys, uint16_t* __restrict__ umasks,
    int32_t* __restrict__ ucount, int32_t* __restrict__ ustage) {
  constexpr int W = kUnionThreads / kWave;
  constexpr int PW = kUnionSpan / 32;      // presence words
  constexpr int WPT = PW / kUnionThreads;  // presence words per thread
  constexpr int NJ = kUnionHeld / kWave;
  static_assert(WPT * kUnionThreads == PW && kUnionBuckets <= kUnionThreads, "shapes");
  __shared__ uint32_t present[PW];
  __shared__ int32_t rank0[PW];                   // entries before each presence word
  __shared__ uint32_t mask2[kUnionEntries / 2];   // the span's masks, two per word
  __shared__ int32_t whist[W][kUnionBuckets];     // per-wave counts, then places
  __shared__ int32_t next[kUnionBuckets];         // next place of each sort key
  __shared__ int32_t wsum[W];
  __shared__ int32_t range[2];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int64_t g = blockIdx.x;
  const int64_t first = g * kGroupRows;
  const int nrows = static_cast<int>(min<int64_t>(kGroupRows, row_count - first));
  const unsigned long long below = (1ull << lane) - 1ull;
  const int span = topk <= kUnionHeld ? kUnionSpan : kUnionEntries;

  // This wave's row: packed keys of its valid entries (-1 otherwise), up to
  // kUnionHeld of them in registers; a longer list is walked in parts of
  // kUnionHeld, reloaded at every walk.
  int32_t key[NJ];
  int64_t kbase = 0;
  int32_t lim = -1;
  if (wave < nrows) {
    const RowInfo ri = row_info(cu_q, cu_k, batch, row_begin + first + wave);
    kbase = ri.key_base;
    lim = ri.pos;
  }
  const int32_t* irow = indices + (first + min(wave, nrows - 1)) * topk;
  const int parts = (topk + kUnionHeld - 1) / kUnionHeld;
  auto load_keys = [&](int part) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = part * kUnionHeld + j * kWave + lane;
      const int32_t e = wave < nrows && c < topk ? irow[c] : -1;
      key[j] = e >= 0 && e <= lim ? static_cast<int32_t>(kbase + e) : -1;
    }
  };
  // fn(key) for every valid key of this wave's row.
  auto each_key = [&](auto fn) __attribute__((always_inline)) {
    for (int part = 0; part < parts; ++part) {
      if (parts > 1) load_keys(part);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (key[j] >= 0) fn(key[j]);
    }
  };
  load_keys(0);
  // Key range of the group, [lo, hi]: the rows' visible keys (a superset of
  // the keys they list, known without waiting for the lists).
  if (lane == 0) {
    whist[wave][0] = wave < nrows ? static_cast<int32_t>(kbase) : INT32_MAX;
    whist[wave][1] = wave < nrows ? static_cast<int32_t>(kbase + lim) : -1;
  }
  if (tid < kUnionBuckets) next[tid] = 0;
  __syncthreads();
  if (tid == 0) {
    int32_t lo = INT32_MAX, hi = -1;
    for (int w = 0; w < W; ++w) {
      lo = min(lo, whist[w][0]);
      hi = max(hi, whist[w][1]);
    }
    range[0] = hi < 0 ? 0 : lo;
    range[1] = hi;
  }
  __syncthreads();
  const int32_t lo = range[0], hi = range[1];
  const int spans = hi < lo ? 0 : (hi - lo) / span + 1;
  int32_t* okeys = ukeys + g * grouped_ws_entries(topk);
  uint16_t* omasks = umasks + g * grouped_ws_entries(topk);
  int32_t* stage = ustage + g * grouped_ws_entries(topk);  // the span's keys by rank

  // The span at x0: presence bits, word ranks and masks; returns its entry count.
  auto build_span = [&](int32_t x0) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < WPT; ++k) present[tid * WPT + k] = 0u;
    __syncthreads();
    each_key([&](int32_t x) __attribute__((always_inline)) {
      const uint32_t off = static_cast<uint32_t>(x - x0);
      if (off < static_cast<uint32_t>(span)) atomicOr(&present[off >> 5], 1u << (off & 31));
    });
    __syncthreads();
    int cnt[WPT];
    int mine = 0;
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      cnt[k] = __popc(present[tid * WPT + k]);
      mine += cnt[k];
    }
    int n = 0;
    int at = union_scan(mine, kUnionThreads, wsum, n);
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      rank0[tid * WPT + k] = at;
      at += cnt[k];
    }
    for (int i = tid; i < (n + 1) / 2; i += kUnionThreads) mask2[i] = 0u;
    __syncthreads();
    each_key([&](int32_t x) __attribute__((always_inline)) {
      const uint32_t off = static_cast<uint32_t>(x - x0);
      if (off < static_cast<uint32_t>(span)) {
        const int w = static_cast<int>(off >> 5);
        const int r = rank0[w] + __popc(present[w] & ((1u << (off & 31)) - 1u));
        atomicOr(&mask2[r >> 1], (1u << wave) << (16 * (r & 1)));
        // Every row holding the key writes the same value.
        stage[r] = x;
      }
    });
    // The staged keys are complete in L2 before any wave reads them.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    return n;
  };
  auto mask_at = [&](int i) __attribute__((always_inline)) {
    return (mask2[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
  };
  auto count_span = [&](int n) __attribute__((always_inline)) {
    for (int i = tid; i < n; i += kUnionThreads) atomicAdd(&next[union_bucket<waves>(mask_at(i))], 1);
    __syncthreads();
  };
  // With `starts`, next[] holds each sort key's first place; without, the
  // span is the whole union and the places come from its own counts.
  auto scatter_span = [&](int n, bool starts) __attribute__((always_inline)) {
    for (int i = tid; i < W * kUnionBuckets; i += kUnionThreads) (&whist[0][0])[i] = 0;
    __syncthreads();
    const int per = ((n + W - 1) / W + kWave - 1) / kWave * kWave;
    const int e0 = wave * per, e1 = min(n, e0 + per);
    for (int c = e0; c < e1; c += kWave) {
      const int i = c + lane;
      const bool in = i < e1;
      const int b = in ? union_bucket<waves>(mask_at(i)) : 0;
      const unsigned long long peers = same_key_lanes(b, in);
      // One lane per sort key (the lowest) adds its count: distinct addresses.
      if (in && (peers & below) == 0ull) whist[wave][b] += __popcll(peers);
    }
    __syncthreads();
    if (!starts) {
      int tot = 0;
      if (tid < kUnionBuckets)
        for (int w = 0; w < W; ++w) tot += whist[w][tid];
      int total = 0;
      const int start = union_scan(tot, kUnionBuckets, wsum, total);
      if (tid < kUnionBuckets) next[tid] = start;
      if (tid == 0) ucount[g] = total;
    }
    if (tid < kUnionBuckets) {
      int at = next[tid];
      for (int w = 0; w < W; ++w) {
        const int c = whist[w][tid];
        whist[w][tid] = at;
        at += c;
      }
      next[tid] = at;
    }
    __syncthreads();
    for (int c = e0; c < e1; c += kWave) {
      const int i = c + lane;
      const bool in = i < e1;
      const uint32_t m = in ? mask_at(i) : 0u;
      const int b = in ? union_bucket<waves>(m) : 0;
      const unsigned long long peers = same_key_lanes(b, in);
      // Every lane reads its sort key's place before the lowest lane moves
      // it on (one wave's LDS operations are performed in order).
      const int dst = (in ? whist[wave][b] : 0) + __popcll(peers & below);
      if (in) {
        okeys[dst] = stage[i];
        omasks[dst] = static_cast<uint16_t>(m);
      }
      if (in && (peers & below) == 0ull) whist[wave][b] = dst + __popcll(peers);
    }
    __syncthreads();
  };

  // One span: built once, scattered with places from its own counts.
  // Several: every span's sort keys counted, then each rebuilt and
  // scattered at the places the counts give.
  const bool several = spans > 1;
  int n_last = 0;
  for (int sp = 0; sp < spans; ++sp) {
    n_last = build_span(lo + sp * span);
    if (several) count_span(n_last);
  }
  if (several) {
    const int cnt = tid < kUnionBuckets ? next[tid] : 0;
    int total = 0;
    const int start = union_scan(cnt, kUnionBuckets, wsum, total);
    if (tid < kUnionBuckets) next[tid] = start;
    if (tid == 0) ucount[g] = total;
    __syncthreads();
  }
  for (int sp = 0; sp < (spans > 0 ? spans : 1); ++sp)
    scatter_span(several ? build_span(lo + sp * span) : n_last, several);
}

// One workgroup per (group, KV head); wave w serves the group's queries
// 16 w .. 16 w + 15 of this KV head (query c = row c / G, head c mod G).
// Union tiles of 32 entries stream through an LDS ring of kRingG slots by
// buffer->LDS DMA, two tiles (a pair) a step: step s uses pair s while the
// copies of pairs s + 1 and s + 2 are in flight, so four tiles are on their
// way while two are used.  A pair's K and V rows (2 x 32 x D / 8 16-byte
// chunks a tile, COPIES per lane and tile: G is a power of two, so every
// wave issues the same copies) and its 64 row masks are copied by every
// wave, addressed by the pair's union keys, which come into a key slot one
// step before (a key read at copy time would stall every wave on a miss).
// Every step issues the same loads (past the union's end they read zeros),
// so one counted wait per step is exact, and one barrier per step (two
// tiles) makes every wave's copies visible and frees the slots of the pair
// before.  Six ring slots and two key slots are all the LDS the copies
// write: the compiler tells a few such targets apart (with more, or with
// the keys in registers, it waited for every copy in flight).
//
// A wave computes a pair when its rows own an entry of either tile, both
// tiles in one update (compute_tile_pair: four independent S products and
// one softmax reference update); a wave whose rows own nothing in the pair
// skips it.
constexpr int kRingG = 6;  // slots: three pairs

// Ring slot B: K tile, V tile, then 128 union masks (slot 2 p mod kRingG
// holds its pair's 64, from the pair's first entry).  One LDS variable each:
// the compiler then sees that a slot being read is not the one a copy in
// flight writes, and places no wait for those copies before the reads.
template <int D, int B>
__device__ __forceinline__ uint16_t* grouped_slot() {
  __shared__ __attribute__((aligned(16))) uint16_t buf[2 * AttnCfg<D>::TILE + 2 * kWave];
  return buf;
}
// Key slot B: the 64 union keys of a pair (one variable each, as above).
template <int B>
__device__ __forceinline__ int32_t* grouped_keyslot() {
  __shared__ __attribute__((aligned(16))) int32_t buf[kWave];
  return buf;
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N - 1, in order.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Workgroup order, longest first.  A workgroup's time follows its union's
// size (correlation 0.94-0.97 measured on correlated 2048-row windows), and
// with about two workgroups a CU the launch ends with its last long
// workgroup, so the groups are launched by descending union size
// (order_kernel, one workgroup after the union pass; ties by group index):
// workgroup i serves group order[i / n_heads_kv] with KV head
// i mod n_heads_kv.  The order decides only when each group runs, never
// what it computes.  Windows of more than kOrderMax groups keep the natural
// order.
constexpr int kOrderMax = 8192;
constexpr int kOrderThreads = 1024;

__global__ __launch_bounds__(kOrderThreads) void order_kernel(const int32_t* __restrict__ ucount,
                                                              int groups,
                                                              int32_t* __restrict__ order) {
  __shared__ uint32_t key[kOrderMax];
  const int tid = threadIdx.x;
  if (groups > kOrderMax) {
    for (int i = tid; i < groups; i += kOrderThreads) order[i] = i;
    return;
  }
  int n2 = 1;
  while (n2 < groups) n2 <<= 1;
  // Sort key: union size above, 8191 - group below (a union holds at most
  // 16 k <= 65536 entries: 17 bits, plus 13 for the group), descending.
  for (int i = tid; i < n2; i += kOrderThreads)
    key[i] = i < groups ? (static_cast<uint32_t>(ucount[i]) << 13) | static_cast<uint32_t>(kOrderMax - 1 - i)
                        : 0u;
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (n2 >> 1); t += kOrderThreads) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint32_t x = key[lo], y = key[hi];
        if ((x < y) == desc) {
          key[lo] = y;
          key[hi] = x;
        }
      }
      __syncthreads();
    }
  for (int i = tid; i < groups; i += kOrderThreads)
    order[i] = kOrderMax - 1 - static_cast<int>(key[i] & (kOrderMax - 1));
}

template <int D, int COPIES>
__global__ __launch_bounds__(8 * D / COPIES) void grouped_attn_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t total_k, int topk, int64_t row_begin,
    int64_t row_count, int n_heads_q, int n_heads_kv, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, const int32_t* __restrict__ ukeys,
    const uint16_t* __restrict__ umasks, const int32_t* __restrict__ ucount,
    const int32_t* __restrict__ order, int64_t groups) {
  using C = AttnCfg<D>;
  constexpr int CH = 32 * C::PIECES;      // 16-byte chunks of one K (or V) tile
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  constexpr int NTHREADS = 8 * D / COPIES;  // the launch's block size, 64 G
  const int G = n_heads_q / n_heads_kv;
  const int col = lane & 15, qd = lane >> 4;
  const int64_t gi = blockIdx.x / n_heads_kv;
  const int h = static_cast<int>(blockIdx.x % n_heads_kv);
  const int64_t g = groups > kOrderMax ? gi : order[gi];
  const int64_t first = g * kGroupRows;
  // This lane's query column.
  const int cq = 16 * wave + col;
  const int rl = cq / G;
  const bool active = first + rl < row_count;
  const int64_t row = row_begin + first + rl;
  const int hq = h * G + cq % G;
  bf16x8 qb[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    qb[ks] = active ? load_bf16x8(q + (row * n_heads_q + hq) * D + ks * 32 + qd * 8) : zero_bf16x8();
  // The queries have landed before the ring starts, so the ring's counted
  // waits below are the only vector-memory waits in the loop.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  // Rows of this wave's 16 columns: rl_first .. rl_first + nrw - 1.
  const int rl_first = (16 * wave) / G;
  const int nrw = (16 * wave + 15) / G - rl_first + 1;

  const int32_t count = ucount[g];
  const int32_t* keys = ukeys + g * grouped_ws_entries(topk);
  const uint16_t* masks = umasks + g * grouped_ws_entries(topk);
  const int kv_bytes = static_cast<int>(total_k * n_heads_kv * D * 2);
  // Whole words up to the union's end (a word read partly past the range
  // would come back as zero); the group's mask region always holds them.
  const __amdgpu_buffer_rsrc_t mr = raw_buffer(masks, (count * 2 + 3) & ~3);
  const __amdgpu_buffer_rsrc_t kyr = raw_buffer(keys, count * 4);
  // Union keys of pair p into a key slot (4 bytes a lane; zero past the
  // union's end).  Every wave copies the same words.
  auto copy_keys = [&](int p, int32_t* ks) __attribute__((always_inline)) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        kyr, (__attribute__((address_space(3))) void*)ks, 4, lane * 4, p * 256, 0, 0);
  };
  // Copies of pair p: tile 2 p into ring slot r0, tile 2 p + 1 into r1,
  // addressed by the keys in key slot ks; then the pair's masks (4 bytes a
  // lane, from entry 64 p) behind r0's V tile.  Copy j of this wave covers
  // chunks cbase .. cbase + 63 of a tile (cbase uniform); chunk c is piece
  // c mod PIECES of tile row c / PIECES in LDS, filled from global piece
  // (c mod PIECES) ^ (row mod PIECES) (the tile_at swizzle).
  auto issue_pair = [&](int p, uint16_t* r0, uint16_t* r1, const int32_t* ks)
                        __attribute__((always_inline)) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint16_t* rs = half == 0 ? r0 : r1;
#pragma unroll
      for (int j = 0; j < COPIES; ++j) {
        // Chunks 0 .. CH - 1 are the K tile's, CH .. 2 CH - 1 the V tile's
        // (CH is a multiple of 64, so a copy is all K or all V).
        const int cc = j * NTHREADS + kWave * wave;
        const bool is_v = cc >= CH;
        const int cbase = is_v ? cc - CH : cc;
        const int c = cbase + lane;
        const int r = c / C::PIECES;
        const int piece = (c % C::PIECES) ^ (r % C::PIECES);
        const int off = ((ks[32 * half + r] * n_heads_kv + h) * D + piece * 8) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            raw_buffer(is_v ? v : k, kv_bytes),
            (__attribute__((address_space(3))) void*)(&rs[(is_v ? C::TILE : 0) + cbase * 8]), 16,
            off, 0, 0, 0);
      }
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        mr, (__attribute__((address_space(3))) void*)(&r0[2 * C::TILE]), 4, lane * 4, p * 128, 0, 0);
  };
  // Loads per step: the keys of one pair, 2 COPIES copies, the masks.
  constexpr int L = 2 * COPIES + 2;
  static_assert(L <= 63 && kRingG == 6, "counted wait; three pairs in the ring");

  f32x4 acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  const int ntiles = (count + 31) / 32;
  const int npairs = (ntiles + 1) / 2;
  // Prologue, as steps -2 and -1 without their barriers' first purpose: the
  // keys of pair s + 3 (key slot (s + 3) mod 2) and the copies of pair s + 2
  // (keys from slot (s + 2) mod 2), after the keys of pair 0, waited for.
  // The loads in flight at step 0 are then exactly those the steps count on.
  copy_keys(0, grouped_keyslot<0>());
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  copy_keys(1, grouped_keyslot<1>());
  issue_pair(0, grouped_slot<D, 0>(), grouped_slot<D, 1>(), grouped_keyslot<0>());
  lds_barrier();  // every wave has read key slot 0 before it is refilled
  copy_keys(2, grouped_keyslot<0>());
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(L));  // the keys of pair 1
  issue_pair(1, grouped_slot<D, 2>(), grouped_slot<D, 3>(), grouped_keyslot<1>());
  // Step s (pair s in slots 2 P, 2 P + 1 with P = s mod 3): once pair s and
  // the keys of pair s + 2 have landed (only step s - 1's loads after its
  // first are younger) and every wave is past the previous step, the keys of
  // pair s + 3 (into the key slot that held pair s + 1's, read a step ago)
  // and the copies of pair s + 2 (into the slots of pair s - 1); then pair s.
  // (Issuing the copies after the pair's compute measured slower: 32.0 ms
  // against 29.9 ms on the correlated 128K prefill.)
  auto step = [&](auto tag, int s) __attribute__((always_inline)) {
    constexpr int B = decltype(tag)::value;  // s mod 6
    constexpr int P = B % 3, PI = (B + 2) % 3;
    constexpr int KR = B % 2, KW = (B + 1) % 2;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(L - 1));
    lds_barrier();
    const uint16_t* rs0 = grouped_slot<D, 2 * P>();
    const uint16_t* rs1 = grouped_slot<D, 2 * P + 1>();
    const uint32_t* mw = reinterpret_cast<const uint32_t*>(rs0 + 2 * C::TILE);
    const uint32_t mw0 = mw[(lane & 31) >> 1], mw1 = mw[16 + ((lane & 31) >> 1)];
    copy_keys(s + 3, grouped_keyslot<KW>());
    issue_pair(s + 2, grouped_slot<D, 2 * PI>(), grouped_slot<D, 2 * PI + 1>(),
               grouped_keyslot<KR>());
    // This lane's entry of each tile: the masks of its rows.
    const int e0 = 2 * s * 32 + (lane & 31);
    const uint32_t m0 = e0 >= count ? 0u : (lane & 1) ? (mw0 >> 16) : (mw0 & 0xFFFFu);
    const uint32_t m1 = e0 + 32 >= count ? 0u : (lane & 1) ? (mw1 >> 16) : (mw1 & 0xFFFFu);
    // Validity of the 64 slots for this lane's row.
    uint32_t vm0 = 0u, vm1 = 0u;
    for (int i = 0; i < nrw; ++i) {
      const uint32_t w0 = static_cast<uint32_t>(__ballot((m0 >> (rl_first + i)) & 1u));
      const uint32_t w1 = static_cast<uint32_t>(__ballot((m1 >> (rl_first + i)) & 1u));
      if (rl == rl_first + i) {
        vm0 = w0;
        vm1 = w1;
      }
    }
    // A pair holding none of this wave's rows is skipped (a fully masked
    // tile changes nothing).
    if (__any((vm0 | vm1) != 0u))
      compute_tile_pair<D>(qb, rs0, rs0 + C::TILE, vm0, rs1, rs1 + C::TILE, vm1, scale_log2, lane,
                           m_run, l_run, acc);
  };
  // Whole rounds of six pairs: a pair past the union's end has all masks
  // zero and changes nothing, and straight-line rounds keep the slots and
  // key slots static.
  for (int s = 0; s < npairs; s += 6)
    static_for<6>([&](auto b) __attribute__((always_inline)) { step(b, s + decltype(b)::value); });
  // No copy may still be writing LDS when the wave ends.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // Normalise; O rows of this lane are columns 4 qd + r.
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float lr = __shfl(l_tot, 4 * qd + r);
    const float mrun = __shfl(m_run, 4 * qd + r);
    const int c = 16 * wave + 4 * qd + r;
    const int rr = c / G;
    if (first + rr >= row_count) continue;
    const int64_t orow_i = row_begin + first + rr;
    const int ohq = h * G + c % G;
    const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
    uint16_t* orow = out + (orow_i * n_heads_q + ohq) * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
      orow[dt * 16 + col] = static_cast<uint16_t>(f32_to_bf16_bits(acc[dt][r] * inv));
    if (lse != nullptr && col == 0)
      lse[orow_i * n_heads_q + ohq] = lr > 0.0f ? (mrun + log2f(lr)) * kLn2 : -INFINITY;
  }
}

template <int D, int COPIES>
void launch_grouped_attn_d(dim3 grid, dim3 block, hipStream_t stream, const dsa_varlen& vl,
                           const uint16_t* q, const uint16_t* k, const uint16_t* v, int topk,
                           int64_t row_begin, int64_t row_count, int n_heads_q, int n_heads_kv,
                           float scale_log2, uint16_t* out, float* lse,
                           const GroupedWorkspace& ws) {
  const int64_t groups = (row_count + kGroupRows - 1) / kGroupRows;
  hipLaunchKernelGGL((grouped_attn_kernel<D, COPIES>), grid, block, 0, stream, vl.cu_seqlens_q,
                     vl.cu_seqlens_k, vl.batch, q, k, v, vl.total_k, topk, row_begin, row_count,
                     n_heads_q, n_heads_kv, scale_log2, out, lse, ws.keys, ws.masks, ws.counts,
                     ws.order, groups);
}

}  // namespace

size_t grouped_attn_workspace_bytes(int64_t row_count, int topk) {
  const int64_t groups = (row_count + kGroupRows - 1) / kGroupRows;
  const size_t n = static_cast<size_t>(groups) * grouped_ws_entries(topk);
  return 2 * round256(n * sizeof(int32_t)) + round256(n * sizeof(uint16_t)) +
         round256(static_cast<size_t>(groups) * sizeof(int32_t)) +
         static_cast<size_t>(groups) * sizeof(int32_t);
}

hipError_t launch_grouped_attn(const dsa_varlen& vl, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* indices, int topk,
                               int64_t row_begin, int64_t row_count, int n_heads_q,
                               int n_heads_kv, int head_dim, float scale, uint16_t* out,
                               float* lse, void* workspace, hipStream_t stream) {
  const int64_t groups = (row_count + kGroupRows - 1) / kGroupRows;
  const GroupedWorkspace ws = grouped_ws_layout(workspace, groups, topk);
  const int G = n_heads_q / n_heads_kv;
  auto run_union = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(groups)), dim3(kUnionThreads), 0, stream,
                       vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, indices, topk, row_begin,
                       row_count, ws.keys, ws.masks, ws.counts, ws.stage);
  };
  switch (G) {  // the attention's waves per workgroup: G in {1, 2, 4, 8}
    case 8: run_union(union_kernel<8>); break;
    case 4: run_union(union_kernel<4>); break;
    case 2: run_union(union_kernel<2>); break;
    default: run_union(union_kernel<1>); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, ws.counts,
                     static_cast<int>(groups), ws.order);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 grid(static_cast<unsigned>(groups * n_heads_kv));
  const dim3 block(kWave * G);  // 16 G queries per KV head, 16 per wave
  const float scale_log2 = scale * kLog2e;
  // Copies per lane and tile: 2 x 32 rows x head_dim / 8 chunks over 64 G
  // lanes (G in {1, 2, 4, 8}, checked by the caller): head_dim / (8 G).
  const int copies = head_dim / (8 * G);
  auto go = [&](auto d_tag, auto copies_tag) {
    launch_grouped_attn_d<decltype(d_tag)::value, decltype(copies_tag)::value>(
        grid, block, stream, vl, q, k, v, topk, row_begin, row_count, n_heads_q, n_heads_kv,
        scale_log2, out, lse, ws);
  };
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  if (head_dim == 128) {
    switch (copies) {
      case 16: go(I128{}, std::integral_constant<int, 16>{}); break;
      case 8: go(I128{}, std::integral_constant<int, 8>{}); break;
      case 4: go(I128{}, std::integral_constant<int, 4>{}); break;
      default: go(I128{}, std::integral_constant<int, 2>{}); break;
    }
  } else {
    switch (copies) {
      case 8: go(I64{}, std::integral_constant<int, 8>{}); break;
      case 4: go(I64{}, std::integral_constant<int, 4>{}); break;
      case 2: go(I64{}, std::integral_constant<int, 2>{}); break;
      default: go(I64{}, std::integral_constant<int, 1>{}); break;
    }
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- fixed scratch
//
// Device-resident scratch for the decode split partials, for callers that
// cannot allocate (code under graph capture, serving loops that forbid
// hipMalloc).  Each GPU the library runs on holds one copy until the process
// ends; host code never passes `scratch` itself to a kernel (on the host the
// name is only a stand-in), but the device address hipGetSymbolAddress
// returns for the current device, looked up once per device.
constexpr size_t kAttnScratchBytes = size_t{16} << 20;
static __device__ __align__(256) float scratch[kAttnScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch[kMaxScratchDevices] = {};
}  // namespace

size_t attn_scratch_bytes() { return kAttnScratchBytes; }

hipError_t attn_scratch(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

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
  // Up to 2 x 8 KV heads x 8 KB of tiles plus a 4096-entry index list:
  // above the default dynamic LDS limit, within the 160 KB of a CU.
  static const hipError_t lds_ok = [] {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_attn_kernel<128>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(attn_lds_bytes<128>(8, 4096)));
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_attn_kernel<64>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(attn_lds_bytes<64>(8, 4096)));
    return e;
  }();
  if (lds_ok != hipSuccess) return lds_ok;
  if (head_dim == 128) {
    const size_t lds = attn_lds_bytes<128>(n_heads_kv, (topk + splits - 1) / splits);
    hipLaunchKernelGGL(sparse_attn_kernel<128>, grid, block, lds, stream, vl.cu_seqlens_q,
                       vl.cu_seqlens_k, vl.batch, q, k, v, indices, topk, row_begin, row_count,
                       n_heads_q, n_heads_kv, scale_log2, out, lse, splits, partial);
  } else {
    const size_t lds = attn_lds_bytes<64>(n_heads_kv, (topk + splits - 1) / splits);
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
