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
// Pass 1 (union_kernel, one workgroup per group): the union as packed key
// rows (sequence key base + position, ascending) with a 16-bit row mask per
// entry, in the caller's workspace.  The index rows must be ascending with
// -1 padding after the valid entries (as dsa_topk writes them): a cursor per
// row then walks its list once while the packed-key range is swept in spans
// of kUnionSpan, each marked in an LDS bitmap and compacted in order.
// Pass 2 (grouped_attn_kernel, one workgroup per (group, KV head), one wave
// per 16 of the group's 16 * G queries): every union tile of 32 entries is
// gathered into LDS by the whole workgroup and used by every wave with the
// tile update of the per-row kernel, the validity bits taken from the masks.

constexpr int kGroupRows = 16;
constexpr int kUnionSpan = 8192;
constexpr int kUnionThreads = 256;

// Workspace of the grouped path for `groups` groups: union keys (int32), row
// masks (uint16), one count per group.
struct GroupedWorkspace {
  int32_t* keys;
  uint16_t* masks;
  int32_t* counts;
};

__host__ __device__ inline size_t grouped_ws_entries(int topk) {
  return static_cast<size_t>(kGroupRows) * topk;
}

inline GroupedWorkspace grouped_ws_layout(void* base, int64_t groups, int topk) {
  char* p = static_cast<char*>(base);
  GroupedWorkspace w;
  const size_t n = static_cast<size_t>(groups) * grouped_ws_entries(topk);
  w.keys = reinterpret_cast<int32_t*>(p);
  p += (n * sizeof(int32_t) + 255) / 256 * 256;
  w.masks = reinterpret_cast<uint16_t*>(p);
  p += (n * sizeof(uint16_t) + 255) / 256 * 256;
  w.counts = reinterpret_cast<int32_t*>(p);
  return w;
}

__global__ __launch_bounds__(kUnionThreads) void union_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const int32_t* __restrict__ indices, int topk, int64_t row_begin, int64_t row_count,
    int32_t* __restrict__ ukeys, uint16_t* __restrict__ umasks, int32_t* __restrict__ ucount) {
  constexpr int kWavesU = kUnionThreads / kWave;
  constexpr int kPer = kUnionSpan / kUnionThreads;  // bitmap entries per thread
  static_assert(kPer % 4 == 0, "bitmap entries are read 4 at a time");
  __shared__ __attribute__((aligned(16))) uint32_t bits[kUnionSpan / 2];  // 16-bit masks, paired
  __shared__ int64_t rbase[kGroupRows];
  __shared__ int32_t rlim[kGroupRows];
  __shared__ int32_t rcur[kGroupRows];
  __shared__ int32_t wsum[kWavesU];
  __shared__ int64_t span[2];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int64_t g = blockIdx.x;
  const int64_t first = g * kGroupRows;
  const int nrows = static_cast<int>(min<int64_t>(kGroupRows, row_count - first));
  if (tid < kGroupRows) {
    if (tid < nrows) {
      const RowInfo ri = row_info(cu_q, cu_k, batch, row_begin + first + tid);
      rbase[tid] = ri.key_base;
      rlim[tid] = ri.pos;
    }
    rcur[tid] = 0;
  }
  __syncthreads();
  if (tid == 0) {
    int64_t lo = rbase[0], hi = rbase[0] + rlim[0];
    for (int r = 1; r < nrows; ++r) {
      lo = min(lo, rbase[r]);
      hi = max(hi, rbase[r] + rlim[r]);
    }
    span[0] = lo;
    span[1] = hi;
  }
  __syncthreads();
  const int64_t lo = span[0], hi = span[1];
  int32_t* keys = ukeys + g * grouped_ws_entries(topk);
  uint16_t* masks = umasks + g * grouped_ws_entries(topk);
  int32_t out = 0;
  for (int64_t x0 = lo; x0 <= hi; x0 += kUnionSpan) {
    for (int i = tid; i < kUnionSpan / 2; i += kUnionThreads) bits[i] = 0u;
    __syncthreads();
    // Mark: wave w walks rows w, w + kWavesU, ... from their cursors while
    // the packed keys stay below x0 + kUnionSpan.
    for (int r = wave; r < nrows; r += kWavesU) {
      const int32_t* irow = indices + (first + r) * topk;
      const int64_t base = rbase[r];
      const int32_t lim = rlim[r];
      int32_t c = rcur[r];
      while (c < topk) {
        const int32_t e = c + lane < topk ? irow[c + lane] : -1;
        const bool valid = e >= 0 && e <= lim;
        const int64_t key = base + e;
        const bool in = valid && key < x0 + kUnionSpan;
        if (in && key >= x0) {
          const int off = static_cast<int>(key - x0);
          atomicOr(&bits[off >> 1], (1u << r) << (16 * (off & 1)));
        }
        const int n_in = __popcll(__ballot(in));
        c += n_in;
        if (n_in < kWave) break;
      }
      if (lane == 0) rcur[r] = c;
    }
    __syncthreads();
    // Compact the marked entries in key order: thread t owns entries
    // [t kPer, (t + 1) kPer).
    uint32_t m[kPer];
#pragma unroll
    for (int i = 0; i < kPer / 2; i += 2) {
      const uint2 w2 = *reinterpret_cast<const uint2*>(&bits[tid * (kPer / 2) + i]);
      m[2 * i] = w2.x & 0xFFFFu;
      m[2 * i + 1] = w2.x >> 16;
      m[2 * i + 2] = w2.y & 0xFFFFu;
      m[2 * i + 3] = w2.y >> 16;
    }
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) cnt += m[i] != 0u;
    // Exclusive prefix over the workgroup.
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWavesU; ++w) {
      before += w < wave ? wsum[w] : 0;
      total += wsum[w];
    }
    int at = out + before + incl - cnt;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (m[i] != 0u) {
        keys[at] = static_cast<int32_t>(x0 + tid * kPer + i);
        masks[at] = static_cast<uint16_t>(m[i]);
        ++at;
      }
    }
    out += total;
    __syncthreads();
  }
  if (tid == 0) ucount[g] = out;
}

// One workgroup per (group, KV head); wave w serves the group's queries
// 16 w .. 16 w + 15 of this KV head (query c = row c / G, head c mod G).
// Union tiles of 32 entries stream through an LDS ring of R slots by
// buffer->LDS DMA, so R - 1 tiles are in flight while one is used: the
// K and V rows of the tile's entries (2 x 32 x D / 8 16-byte chunks, COPIES
// per lane: G is a power of two, so every wave issues the same copies),
// while each wave loads the tile's 32 row masks into a register.  The union
// keys that address a tile's copies are loaded into registers R - 1 tiles
// earlier, so they have landed by the ring's counted wait that precedes the
// copies (a key read at copy time would stall every wave on a miss each
// tile).  Every step issues the same loads (past the union's end they read
// zeros, copied into a slot nobody reads), which keeps the counts fixed.
//
// R = grouped_ring: as many slots as leave room in LDS (at most
// kMaxRingG), bounded so that the counted wait ((R - 2) (COPIES + 2) loads)
// fits its 6-bit field.  Four slots measured as fast as eight, at fewer
// registers.
constexpr int kMaxRingG = 4;
template <int D, int COPIES>
constexpr int grouped_ring() {
  constexpr int by_wait = 2 + 63 / (COPIES + 2);
  constexpr int by_lds = (128 * 1024) / (2 * AttnCfg<D>::TILE * 2 + 512);
  constexpr int r = by_wait < by_lds ? by_wait : by_lds;
  return r < kMaxRingG ? r : kMaxRingG;
}

// Ring slot B: K tile, V tile, then 128 union masks from the tile's first
// (only its 32 are read); and key slot B: 64 union keys from a tile's first.
// One LDS variable each: the compiler then sees that a slot being read is
// not the one a copy in flight writes, and places no wait for those copies
// before the reads.
template <int D, int B>
__device__ __forceinline__ uint16_t* grouped_slot() {
  __shared__ __attribute__((aligned(16))) uint16_t buf[2 * AttnCfg<D>::TILE + 2 * kWave];
  return buf;
}
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

template <int D, int COPIES>
__global__ __launch_bounds__(8 * D / COPIES) void grouped_attn_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t total_k, int topk, int64_t row_begin,
    int64_t row_count, int n_heads_q, int n_heads_kv, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, const int32_t* __restrict__ ukeys,
    const uint16_t* __restrict__ umasks, const int32_t* __restrict__ ucount) {
  using C = AttnCfg<D>;
  constexpr int CH = 32 * C::PIECES;      // 16-byte chunks of one K (or V) tile
  constexpr int RPI = kWave / C::PIECES;  // tile rows per copy instruction
  constexpr int R = grouped_ring<D, COPIES>();
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  constexpr int NTHREADS = 8 * D / COPIES;  // the launch's block size, 64 G
  const int G = n_heads_q / n_heads_kv;
  const int col = lane & 15, qd = lane >> 4;
  const int64_t g = blockIdx.x;
  const int h = blockIdx.y;
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
  // Copies of tile t into a ring slot.  Copy j of this wave covers chunks
  // cbase .. cbase + 63 (cbase uniform); chunk c is piece c mod PIECES of
  // tile row c / PIECES in LDS, filled from global piece
  // (c mod PIECES) ^ (row mod PIECES) (the tile_at swizzle).  The tile's 32
  // row masks come with them into a register: lane l gets the word holding
  // the masks of slots 2 (l mod 32) / 2 and the one after (zero past the
  // union's end).
  const __amdgpu_buffer_rsrc_t kyr = raw_buffer(keys, count * 4);
  // Union keys u*32 .. u*32 + 63 into a key slot (4 bytes a lane; zero past
  // the union's end).  Every wave copies the same words, so every wave
  // issues the same loads.
  auto copy_keys = [&](int u, int32_t* ks) __attribute__((always_inline)) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        kyr, (__attribute__((address_space(3))) void*)ks, 4, lane * 4, u * 128, 0, 0);
  };
  // Copies of tile u into ring slot rs, addressed by the keys in key slot ks;
  // then its masks (4 bytes a lane, from entry u*32) behind the V tile.
  auto issue = [&](int u, uint16_t* rs, const int32_t* ks) __attribute__((always_inline)) {
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
      const int off = ((ks[r] * n_heads_kv + h) * D + piece * 8) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          raw_buffer(is_v ? v : k, kv_bytes),
          (__attribute__((address_space(3))) void*)(&rs[(is_v ? C::TILE : 0) + cbase * 8]), 16,
          off, 0, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        mr, (__attribute__((address_space(3))) void*)(&rs[2 * C::TILE]), 4, lane * 4, u * 64, 0, 0);
  };

  f32x4 acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  const int ntiles = (count + 31) / 32;
  // Every step issues, in order, the keys of tile u + R - 1, the copies of
  // tile u and its masks (COPIES + 2 loads); the loop's step t is such a step
  // with u = t + R - 1.  The prologue runs it for u = 0 .. R - 2 once the
  // first tiles' keys are in.
  static_for<R - 1>([&](auto b) __attribute__((always_inline)) {
    copy_keys(decltype(b)::value, grouped_keyslot<decltype(b)::value>());
  });
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  static_for<R - 1>([&](auto b) __attribute__((always_inline)) {
    constexpr int U = decltype(b)::value;
    // Key slot (U + R - 1) mod R held tile U - 1's keys: every wave has
    // read them once past this barrier.
    if constexpr (U > 0) lds_barrier();
    copy_keys(U + R - 1, grouped_keyslot<(U + R - 1) % R>());
    issue(U, grouped_slot<D, U>(), grouped_keyslot<U>());
  });
  // Tile t from ring slot B = t mod R; the copies of tile t + R - 1 go to
  // slot (B + R - 1) mod R, the one tile t - 1 used.
  auto step = [&](auto tag, int t) __attribute__((always_inline)) {
    constexpr int B = decltype(tag)::value;
    constexpr int BN = (B + R - 1) % R;
    // Tile t has landed once only the R - 2 younger steps' loads are
    // outstanding, and so have the keys of tile t + R - 1, copied before
    // tile t; the barrier makes every wave's copies visible and frees slot
    // BN and key slot (B + R - 2) mod R (all waves are done with tile t - 1).
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((R - 2) * (COPIES + 2)));
    lds_barrier();
    const uint16_t* rs = grouped_slot<D, B>();
    const uint32_t mw = reinterpret_cast<const uint32_t*>(rs + 2 * C::TILE)[(lane & 31) >> 1];
    copy_keys(t + 2 * R - 2, grouped_keyslot<(B + 2 * R - 2) % R>());
    issue(t + R - 1, grouped_slot<D, BN>(), grouped_keyslot<BN>());
    const uint32_t m16 = t * 32 + (lane & 31) >= count ? 0u
                         : (lane & 1)                   ? (mw >> 16)
                                                        : (mw & 0xFFFFu);
    // Validity of the 32 slots for this lane's row.
    uint32_t vm = 0u;
    for (int i = 0; i < nrw; ++i) {
      const uint32_t w = static_cast<uint32_t>(__ballot((m16 >> (rl_first + i)) & 1u));
      if (rl == rl_first + i) vm = w;
    }
    // The index sets come in runs of nearby positions, so a tile often holds
    // none of this wave's rows: the wave then skips it (a fully masked tile
    // changes nothing).
    if (__any(vm != 0u))
      compute_tile<D>(qb, rs, rs + C::TILE, vm, scale_log2, lane, m_run, l_run, acc);
  };
  // Whole rounds of R tiles: a tile past the union's end has all masks zero
  // and changes nothing, and straight-line rounds let the compiler see which
  // loads each register waits for.
  for (int t = 0; t < ntiles; t += R)
    static_for<R>([&](auto b) __attribute__((always_inline)) { step(b, t + decltype(b)::value); });
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
  hipLaunchKernelGGL((grouped_attn_kernel<D, COPIES>), grid, block, 0, stream, vl.cu_seqlens_q,
                     vl.cu_seqlens_k, vl.batch, q, k, v, vl.total_k, topk, row_begin, row_count,
                     n_heads_q, n_heads_kv, scale_log2, out, lse, ws.keys, ws.masks, ws.counts);
}

}  // namespace

size_t grouped_attn_workspace_bytes(int64_t row_count, int topk) {
  const int64_t groups = (row_count + kGroupRows - 1) / kGroupRows;
  const size_t n = static_cast<size_t>(groups) * grouped_ws_entries(topk);
  return (n * sizeof(int32_t) + 255) / 256 * 256 + (n * sizeof(uint16_t) + 255) / 256 * 256 +
         static_cast<size_t>(groups) * sizeof(int32_t);
}

hipError_t launch_grouped_attn(const dsa_varlen& vl, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* indices, int topk,
                               int64_t row_begin, int64_t row_count, int n_heads_q,
                               int n_heads_kv, int head_dim, float scale, uint16_t* out,
                               float* lse, void* workspace, hipStream_t stream) {
  const int64_t groups = (row_count + kGroupRows - 1) / kGroupRows;
  const GroupedWorkspace ws = grouped_ws_layout(workspace, groups, topk);
  hipLaunchKernelGGL(union_kernel, dim3(static_cast<unsigned>(groups)), dim3(kUnionThreads), 0,
                     stream, vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, indices, topk, row_begin,
                     row_count, ws.keys, ws.masks, ws.counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int G = n_heads_q / n_heads_kv;
  const dim3 grid(static_cast<unsigned>(groups), static_cast<unsigned>(n_heads_kv));
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
