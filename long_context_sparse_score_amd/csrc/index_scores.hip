// index_scores.hip -- Lightning-Indexer scores on gfx950 MFMA.
//
// I[t, s] = sum_h w[t, h] * max(0, qI[t, h, :] . kI[s, :])  for s = 0..p(t)
// (Keye-VL-2.0 report summary, page 5 section 1: a lightweight scout scores
// every position with one MQA key shared by all of its heads.)
//
// For one query row the head-by-key product is a small GEMM with M = indexer
// heads (up to 64), N = keys, K = d_idx.  Heads sit on the MFMA rows so that
// after v_mfma_f32_32x32x16_bf16 every lane holds one key column and 16 heads
// of it: the ReLU, the weight and the head sum happen in registers, and one
// exchange between the two half-waves finishes the sum.  The contraction over
// d_idx is ordered so that each half-wave covers one contiguous half of every
// qI / kI row, which keeps every load a full 16-byte vector.
//
// Two kernels share that core:
//  * index_scores_block (prefill): a 512-thread workgroup owns 8 consecutive
//    query rows of one sequence, one wave per row.  Key stages of 256 rows
//    (64 KB at d_idx = 128) are copied by buffer->LDS DMA into one of two LDS
//    buffers (16-byte chunks XOR-swizzled by key so the B-fragment reads are
//    bank-conflict free) and feed all 8 waves, so L2 traffic is 1/8 of a
//    per-wave scheme.  Inside a stage the MFMAs of one 32-key tile overlap
//    the previous tile's epilogue, and scores leave through range-checked
//    buffer stores, so a stage waits only for the next stage's DMA.
//    A workgroup whose rows straddle a sequence boundary falls back to the
//    per-wave path below.
//  * index_scores_stream (decode / few rows): each wave streams its own key
//    range of one row through a private LDS ring filled by coalesced
//    buffer->LDS DMA, three 32-key tiles in flight; long rows are split into
//    chunks so that a handful of rows still covers the whole chip.
// Every global load is issued unconditionally (addresses are clamped into
// the sequence instead): a load under a branch makes the compiler wait for
// it on the spot, which would serialise the prefetch.
#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kBlockRows = 8;        // query rows (waves) per prefill workgroup
constexpr int kStageKeys = 256;      // keys per LDS stage (2 stages: 128 KB at d_idx = 128)
constexpr int kStreamRows = 4;       // waves per stream workgroup

// Per-wave stationary state: this row's indexer queries (A operand, heads on
// MFMA rows, MT tiles of 32 heads) and its head weights laid out like the
// accumulator rows.
template <int D, int MT>
struct RowState {
  static constexpr int KS = D / 16;
  bf16x8 a[MT][KS];
  float wv[MT][16];
};

template <int D, int MT>
__device__ __forceinline__ void load_row_state(RowState<D, MT>& st,
                                               const uint16_t* __restrict__ q_idx,
                                               const float* __restrict__ w, int64_t row,
                                               int n_heads, int col, int half) {
  constexpr int KS = D / 16, HALF = D / 2;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = mt * 32 + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      st.a[mt][ks] = h < n_heads ? load_bf16x8(q_idx + (row * n_heads + h) * D + half * HALF + ks * 8)
                                 : zero_bf16x8();
    // Accumulator element v of this lane is MFMA row 8*(v/4) + 4*half + v%4.
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int hr = mt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      st.wv[mt][v] = hr < n_heads ? w[row * n_heads + hr] : 0.0f;
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

// Sum over heads of w * relu(acc); every lane ends up with the score of key
// (lane & 31).
template <int D, int MT>
__device__ __forceinline__ float tile_epilogue(const RowState<D, MT>& st,
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
  const float s = s0 + s1;
  // Add the other half-wave's partial sum.  v_permlane32_swap exchanges the
  // halves in the VALU; a shuffle would go through the LDS pipeline, whose
  // in-order counter would make this wait for the B-fragment reads just
  // issued for the next tile.
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// One wave, one row, keys [c0, c1) read straight from global memory.  Two
// register buffers alternate roles (the loop is unrolled by two tiles), so
// the next tile's load is always in flight while one is multiplied.
template <int D, int MT>
__device__ void row_direct(const RowState<D, MT>& st, const uint16_t* __restrict__ k_idx,
                           const RowInfo& ri, int32_t c0, int32_t c1,
                           float* __restrict__ out_row, int col, int half) {
  constexpr int KS = D / 16, HALF = D / 2;
  const uint16_t* kbase = k_idx + ri.key_base * D + half * HALF;
  auto fetch = [&](bf16x8 (&dst)[KS], int32_t t0) {
    const int32_t key_ld = min(t0 + col, ri.pos);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) dst[ks] = load_bf16x8(kbase + static_cast<int64_t>(key_ld) * D + ks * 8);
  };
  bf16x8 x[KS], y[KS];
  fetch(x, c0);
  fetch(y, c0 + 32);
  for (int32_t t0 = c0; t0 < c1; t0 += 64) {
    f32x16 acc[MT];
    tile_mfma<D, MT>(st, x, acc);
    fetch(x, t0 + 64);
    float s = tile_epilogue<D, MT>(st, acc);
    if (half == 0 && t0 + col < c1) out_row[t0 + col] = s;
    tile_mfma<D, MT>(st, y, acc);
    fetch(y, t0 + 96);
    s = tile_epilogue<D, MT>(st, acc);
    if (half == 0 && t0 + 32 + col < c1) out_row[t0 + 32 + col] = s;
  }
}

// ---------------------------------------------------------------- prefill kernel

template <int D, int MT>
__global__ __launch_bounds__(kBlockRows * kWave, 2) void index_scores_block(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const uint16_t* __restrict__ q_idx, const uint16_t* k_idx,
    const float* __restrict__ w, int n_heads, int64_t row_begin, int64_t row_count,
    float* __restrict__ scores, int64_t ld, int key_chunk) {
  constexpr int KS = D / 16;
  constexpr int CHUNKS = D / 8;                                     // 16-byte chunks per key row
  constexpr int DMA_PER_WAVE = kStageKeys * CHUNKS / (kBlockRows * kWave);
  constexpr int TILES = kStageKeys / 32;                            // 32-key MFMA tiles per stage
  static_assert(TILES % 2 == 0 && DMA_PER_WAVE * kBlockRows * kWave == kStageKeys * CHUNKS, "stage shape");
  __shared__ __attribute__((aligned(16))) uint16_t tile[2][kStageKeys * D];

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int col = lane & 31;
  const int half = lane >> 5;
  // Later rows have longer causal prefixes: hand them out first.
  const int64_t blk = static_cast<int64_t>(gridDim.x) - 1 - blockIdx.x;
  const int64_t first = blk * kBlockRows;
  const int64_t last = min(first + kBlockRows, row_count) - 1;
  const int64_t local = first + wave;
  const bool active = local < row_count;
  const int64_t row = row_begin + (active ? local : last);

  const RowInfo ri = row_info(cu_q, cu_k, batch, row);
  const RowInfo r_first = row_info(cu_q, cu_k, batch, row_begin + first);
  const RowInfo r_last = row_info(cu_q, cu_k, batch, row_begin + last);
  const int32_t c0 = blockIdx.y * key_chunk;

  RowState<D, MT> st;
  load_row_state<D, MT>(st, q_idx, w, row, n_heads, col, half);
  float* out_row = scores + local * ld;

  if (r_first.key_base != r_last.key_base) {
    // Rows of several sequences: every wave walks its own keys.
    const int32_t c1 = min(c0 + key_chunk, ri.pos + 1);
    if (active && c0 < c1) row_direct<D, MT>(st, k_idx, ri, c0, c1, out_row, col, half);
    return;
  }

  // All rows share one sequence; positions grow with the row.
  const int32_t c_end = min(c0 + key_chunk, r_last.pos + 1);
  if (c0 >= c_end) return;
  // Scores of keys my_end and beyond (and every score of an inactive wave)
  // fall outside the store resource and are dropped.
  const int32_t my_end = active ? min(c0 + key_chunk, ri.pos + 1) : c0;
  const uint16_t* kseq = k_idx + r_first.key_base * D;
  const __amdgpu_buffer_rsrc_t keys = raw_buffer(kseq, (r_last.pos + 1) * D * 2);
  const __amdgpu_buffer_rsrc_t outs = raw_buffer(out_row, my_end * 4);

  // Stage fill by buffer->LDS DMA: DMA instruction i of a wave writes 64
  // consecutive 16-byte LDS chunks; LDS chunk (key, s) receives global chunk
  // s ^ (key & (CHUNKS - 1)), so the B-fragment reads below are conflict free.
  // Instruction i covers keys KPI i + (key of instruction 0); the XOR term
  // repeats with period CHUNKS in the key and KPI is a multiple of it, so all
  // instructions share one per-lane offset and differ by a scalar one.
  constexpr int KPI = kBlockRows * kWave / CHUNKS;  // keys per DMA instruction of the workgroup
  static_assert(KPI % CHUNKS == 0, "the swizzle must repeat across DMA instructions");
  const int key0 = (wave * kWave + lane) / CHUNKS, s0 = lane % CHUNKS;
  const int dma_off = key0 * D * 2 + (s0 ^ (key0 & (CHUNKS - 1))) * 16;
  auto fill_stage = [&](int b, int32_t t) {
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          keys, (__attribute__((address_space(3))) void*)(&tile[b][(i * kBlockRows + wave) * kWave * 8]),
          16, dma_off, (t + i * KPI) * D * 2, 0, 0);
    }
  };
  // One score per lane of the lower half-wave (the upper half holds copies).
  auto store = [&](float v, int32_t pos) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), outs, half == 0 ? pos * 4 : 0x7FFFFFF0, 0, 0);
  };

  fill_stage(0, c0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  // Tile j's MFMAs run while tile j-1's epilogue executes on the VALU; each
  // B fragment register is refilled from LDS for tile j+1 as soon as tile
  // j's MFMAs have consumed it.
  f32x16 acc_even[MT], acc_odd[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc_odd[mt] = f32x16{};
  int32_t prev_pos = 1 << 28;  // the first epilogue has nothing to store
  int buf = 0;
  for (int32_t t0 = c0; t0 < c_end; t0 += kStageKeys) {
    if (t0 + kStageKeys < c_end) fill_stage(buf ^ 1, t0 + kStageKeys);
    const uint16_t* tb = tile[buf];
    bf16x8 b[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int slot = (half * KS + ks) ^ (col & (CHUNKS - 1));
      b[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&tb[col * D + slot * 8]));
    }
    // The first tile's fragments stay out of the interleaving pattern below.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tj = 0; tj < TILES; ++tj) {
      f32x16 (&acc)[MT] = (tj & 1) ? acc_odd : acc_even;
      f32x16 (&prev)[MT] = (tj & 1) ? acc_even : acc_odd;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(st.a[mt][ks], b[ks],
                                                            ks == 0 ? f32x16{} : acc[mt], 0, 0, 0);
        if (tj + 1 < TILES) {
          const int slot = (half * KS + ks) ^ (col & (CHUNKS - 1));  // (32 (tj+1) + col) & 15 == col & 15
          b[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&tb[((tj + 1) * 32 + col) * D + slot * 8]));
        }
      }
      store(tile_epilogue<D, MT>(st, prev), prev_pos);
      prev_pos = t0 + tj * 32 + col;
      // Interleave this tile's MFMAs with the previous tile's epilogue (4 VALU
      // after each MFMA) and refill each B fragment right after the MFMA pair
      // that frees it, a full tile before its next use.  Left alone, the
      // scheduler clusters the MFMAs and sinks the refills next to their
      // use; with two waves per SIMD nothing then covers either gap.
#pragma unroll
      for (int i = 0; i < KS * MT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        if (tj + 1 < TILES && i % MT == MT - 1)
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
      }
    }
    // Wait for the next stage's DMA only: the TILES score stores issued after
    // it may stay in flight.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(TILES));
    lds_barrier();
    buf ^= 1;
  }
  store(tile_epilogue<D, MT>(st, acc_odd), prev_pos);
}

// ---------------------------------------------------------------- decode kernel

// Each wave owns one (row, key chunk) work item and a private LDS ring of
// kRing 32-key tiles.  Tiles arrive by buffer->LDS DMA: every DMA
// instruction reads 1 KB of whole key rows (coalesced, unlike loading the
// MFMA operand layout straight from memory, which touches 32 rows per
// instruction and caps the scan well below HBM speed), and the XOR swizzle
// is applied on the global side so the B-fragment reads from LDS are
// conflict free.  kRing - 1 tiles are in flight while one is multiplied; the
// ring is private to the wave, so no workgroup barrier is needed.
constexpr int kRing = 4;

template <int D, int MT>
__global__ __launch_bounds__(kStreamRows * kWave) void index_scores_stream(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx,
    const float* __restrict__ w, int n_heads, int64_t row_begin, int64_t row_count,
    float* __restrict__ scores, int64_t ld, int key_chunk, int chunks_per_row) {
  constexpr int KS = D / 16;
  constexpr int CHUNKS = D / 8;
  constexpr int DMA_PER_TILE = 32 * CHUNKS / kWave;   // 16-byte DMA instructions per tile
  static_assert(DMA_PER_TILE * kWave == 32 * CHUNKS, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t ring[kStreamRows][kRing][32 * D];

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kStreamRows + wave;
  const int64_t local = item / chunks_per_row;
  if (local >= row_count) return;
  const int64_t row = row_begin + local;
  const RowInfo ri = row_info(cu_q, cu_k, batch, row);
  const int32_t c0 = static_cast<int32_t>(item % chunks_per_row) * key_chunk;
  const int32_t c1 = min(c0 + key_chunk, ri.pos + 1);
  if (c0 >= c1) return;
  RowState<D, MT> st;
  load_row_state<D, MT>(st, q_idx, w, row, n_heads, col, half);

  // Keys [c0, c1) only (DMA past c1 reads zeros without touching memory);
  // scores past c1 are dropped.
  const __amdgpu_buffer_rsrc_t keys = raw_buffer(k_idx + (ri.key_base + c0) * D, (c1 - c0) * D * 2);
  const __amdgpu_buffer_rsrc_t outs = raw_buffer(scores + local * ld, c1 * 4);
  auto fill = [&](int slot, int32_t t) {  // tile of keys c0 + t .. c0 + t + 31
#pragma unroll
    for (int i = 0; i < DMA_PER_TILE; ++i) {
      const int e = i * kWave + lane;
      const int key = e / CHUNKS, s = e % CHUNKS;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          keys, (__attribute__((address_space(3))) void*)(&ring[wave][slot][i * kWave * 8]), 16,
          (key * D + (s ^ (key & (CHUNKS - 1))) * 8) * 2, t * D * 2, 0, 0);
    }
  };
  auto store = [&](float v, int32_t pos) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), outs, half == 0 ? pos * 4 : 0x7FFFFFF0, 0, 0);
  };

  // Prologue: tiles 0 .. kRing-2, each followed by a dropped store so that
  // every tile's DMA is trailed by the same count of memory operations as in
  // the loop (one store, then the next tile's DMA).
#pragma unroll
  for (int p = 0; p < kRing - 1; ++p) {
    fill(p, p * 32);
    store(0.0f, 1 << 28);
  }
  f32x16 acc[MT], prev[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) prev[mt] = f32x16{};
  int32_t prev_pos = 1 << 28;
  const int ntiles = (c1 - c0 + 31) / 32;
  for (int j = 0; j < ntiles; ++j) {
    fill((j + kRing - 1) % kRing, (j + kRing - 1) * 32);
    // Tile j has landed once at most the kRing - 1 younger tiles' DMAs and
    // their trailing stores are outstanding.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kRing - 1) * (DMA_PER_TILE + 1)));
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint16_t* tb = ring[wave][j % kRing];
    bf16x8 b[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int slot = (half * KS + ks) ^ (col & (CHUNKS - 1));
      b[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&tb[col * D + slot * 8]));
    }
    tile_mfma<D, MT>(st, b, acc);
    store(tile_epilogue<D, MT>(st, prev), prev_pos);
    prev_pos = c0 + j * 32 + col;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) prev[mt] = acc[mt];
    // The slot refilled next iteration was read above: those reads must be
    // done before its DMA is issued.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  }
  store(tile_epilogue<D, MT>(st, prev), prev_pos);
  // No DMA may still be writing this wave's ring when the wave ends.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

template <int D, int MT>
hipError_t launch_dm(const dsa_varlen& vl, const uint16_t* q_idx, const uint16_t* k_idx,
                     const float* w, int n_heads, int64_t row_begin, int64_t row_count,
                     float* scores, int64_t ld, hipStream_t stream) {
  if (vl.max_seqlen_q >= kBlockRows) {
    // Prefill-like: whole rows per workgroup unless there are too few
    // workgroups to fill the chip, then split the keys.
    const int64_t blocks = (row_count + kBlockRows - 1) / kBlockRows;
    int64_t chunk = vl.max_seqlen_k;
    if (blocks < 1024) {
      const int64_t parts = (1024 + blocks - 1) / blocks;
      chunk = (vl.max_seqlen_k + parts - 1) / parts;
    }
    chunk = ((chunk + kStageKeys - 1) / kStageKeys) * kStageKeys;
    if (chunk < 512) chunk = 512;
    const int64_t chunks = (vl.max_seqlen_k + chunk - 1) / chunk;
    hipLaunchKernelGGL((index_scores_block<D, MT>), dim3(static_cast<unsigned>(blocks),
                       static_cast<unsigned>(chunks)), dim3(kBlockRows * kWave), 0, stream,
                       vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, q_idx, k_idx, w, n_heads,
                       row_begin, row_count, scores, ld, static_cast<int>(chunk));
  } else {
    // Decode-like: one wave per (row, key chunk), about 2048 work items (two
    // rounds of one 4-wave workgroup per CU; measured best among 2048-8192).
    const int64_t per_row = (2048 + row_count - 1) / row_count;
    int64_t chunk = (vl.max_seqlen_k + per_row - 1) / per_row;
    chunk = ((chunk + 31) / 32) * 32;
    if (chunk < 512) chunk = 512;
    const int64_t chunks_per_row = (vl.max_seqlen_k + chunk - 1) / chunk;
    const int64_t items = row_count * chunks_per_row;
    hipLaunchKernelGGL((index_scores_stream<D, MT>),
                       dim3(static_cast<unsigned>((items + kStreamRows - 1) / kStreamRows)),
                       dim3(kStreamRows * kWave), 0, stream, vl.cu_seqlens_q, vl.cu_seqlens_k,
                       vl.batch, q_idx, k_idx, w, n_heads, row_begin, row_count, scores, ld,
                       static_cast<int>(chunk), static_cast<int>(chunks_per_row));
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const dsa_varlen& vl, const uint16_t* q_idx, const uint16_t* k_idx,
                    const float* w, int n_heads, int64_t row_begin, int64_t row_count,
                    float* scores, int64_t ld, hipStream_t stream) {
  if (n_heads > 32)
    return launch_dm<D, 2>(vl, q_idx, k_idx, w, n_heads, row_begin, row_count, scores, ld, stream);
  return launch_dm<D, 1>(vl, q_idx, k_idx, w, n_heads, row_begin, row_count, scores, ld, stream);
}

}  // namespace

hipError_t launch_index_scores(const dsa_varlen& vl, const uint16_t* q_idx, const uint16_t* k_idx,
                               const float* w, int n_heads, int d, int64_t row_begin,
                               int64_t row_count, float* scores, int64_t ld, hipStream_t stream) {
  if (d == 128)
    return launch_d<128>(vl, q_idx, k_idx, w, n_heads, row_begin, row_count, scores, ld, stream);
  return launch_d<64>(vl, q_idx, k_idx, w, n_heads, row_begin, row_count, scores, ld, stream);
}

}  // namespace dsa
