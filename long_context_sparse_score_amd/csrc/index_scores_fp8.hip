// index_scores_fp8.hip -- Lightning-Indexer scores from fp8 inputs on
// gfx950's v_mfma_f32_32x32x64_f8f6f4, and the quantisation that makes them.
//
// The indexer of page 5 section 1 (one MQA key per position shared by all
// indexer heads) with its queries and keys held as OCP e4m3 ("e4m3fn") codes
// and one binary32 scale per vector:
//   x_j  ~  scale * e4m3(c_j),   scale = max|x| / 448,   c_j = e4m3(x_j * 448 / max|x|).
// The pages state no indexer precision; this is a declared input transform.
// Scales are non-negative, so they leave the ReLU:
//   I[t, s] = sum_h w[t,h] max(0, sq[t,h] sk[s] q8[t,h].k8[s])
//           = sk[s] * sum_h (w[t,h] sq[t,h]) max(0, q8[t,h].k8[s]).
// The code products are exact in fp32 (4-bit significands); the MFMA sums
// them in fp32.
//
// The kernels follow the bf16 indexer's plan (heads on the MFMA rows, 32-key
// tiles on the columns, epilogue in registers, one half-wave exchange) with
// one MFMA covering 64 of the d_idx products instead of 16, so a 32-key tile
// of 64 heads at d_idx = 128 is 4 MFMAs.  Key tiles arrive by buffer->LDS DMA
// with the same XOR swizzle of 16-byte chunks; the key scales travel with
// them, and each tile's scale is read with its B fragments.  The LDS swizzle
// differs from the bf16 kernels' because a key row is half as long.
#include <type_traits>

#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kBlockRows8 = 8;    // query rows (waves) per prefill workgroup
constexpr int kStageKeys8 = 512;  // keys per LDS stage
constexpr int kStreamRows8 = 4;   // waves per decode workgroup
constexpr int kRing8 = 4;         // 32-key tiles in a decode wave's LDS ring

// LDS layout of a key tile: 16-byte chunk s of key row r sits in slot
// s ^ swz(r).  LDS serves 16 lanes (256 bytes, all 64 banks) per cycle; rows
// are D bytes, so 256 / D consecutive rows share one bank pattern and the
// swizzle must differ between rows 256 / D apart: swz(r) = (r / (256 / D)) mod
// (D / 16).  The 16 rows read together then cover all 64 banks once.
template <int D>
__host__ __device__ constexpr int swz(int r) {
  return (r / (256 / D)) & (D / 16 - 1);
}

__device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi) {
  return i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
               static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
               static_cast<int>(hi[2]), static_cast<int>(hi[3])};
}

// 32 consecutive code bytes from global memory (16-byte aligned).
__device__ __forceinline__ i32x8 load_codes32(const uint8_t* p) {
  const u32x4* v = reinterpret_cast<const u32x4*>(p);
  return join(v[0], v[1]);
}

// Per-wave stationary state: this row's query codes (A operand, heads on
// MFMA rows, MT tiles of 32 heads, KS MFMAs of 64 products per tile) and the
// head weights times the query scales, laid out like the accumulator rows.
// The contraction index of lane half `half`, MFMA ks, byte j is
// half * D/2 + 32 ks + j for queries and keys alike.
template <int D, int MT>
struct RowState8 {
  static constexpr int KS = D / 64;
  i32x8 a[MT][KS];
  float wv[MT][16];
};

template <int D, int MT>
__device__ __forceinline__ void load_row_state8(RowState8<D, MT>& st,
                                                const uint8_t* __restrict__ q8,
                                                const float* __restrict__ q_scale,
                                                const float* __restrict__ w, int64_t row,
                                                int n_heads, int col, int half) {
  constexpr int KS = D / 64, HALF = D / 2;
  // Loads are issued unconditionally from clamped heads and masked after, so
  // that they are all in flight together.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = mt * 32 + col;
    const int hl = min(h, n_heads - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const i32x8 v = load_codes32(q8 + (row * n_heads + hl) * D + half * HALF + ks * 32);
      st.a[mt][ks] = h < n_heads ? v : i32x8{};
    }
    // Accumulator element v of this lane is MFMA row 8*(v/4) + 4*half + v%4.
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int hr = mt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      const int hc = min(hr, n_heads - 1);
      const float wq = w[row * n_heads + hc] * q_scale[row * n_heads + hc];
      st.wv[mt][v] = hr < n_heads ? wq : 0.0f;
    }
  }
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // Format selectors 0/0: both operands e4m3; no block scales.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D, int MT>
__device__ __forceinline__ void tile_mfma8(const RowState8<D, MT>& st, const i32x8 (&b)[D / 64],
                                           f32x16 (&acc)[MT]) {
  constexpr int KS = D / 64;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    acc[mt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc[mt] = mfma_fp8(st.a[mt][ks], b[ks], acc[mt]);
  }
}

// sum_h wv * relu(acc) over the 32 heads of each tile; every lane ends up with
// the (unscaled) score of key (lane & 31).
template <int D, int MT>
__device__ __forceinline__ float tile_epilogue8(const RowState8<D, MT>& st,
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
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// One wave, one row, keys [c0, c1) read straight from global memory (rows of
// a workgroup that straddles sequences).
template <int D, int MT>
__device__ void row_direct8(const RowState8<D, MT>& st, const uint8_t* __restrict__ k8,
                            const float* __restrict__ k_scale, const RowInfo& ri, int32_t c0,
                            int32_t c1, float* __restrict__ out_row, int col, int half) {
  constexpr int KS = D / 64, HALF = D / 2;
  const uint8_t* kbase = k8 + ri.key_base * D + half * HALF;
  for (int32_t t0 = c0; t0 < c1; t0 += 32) {
    const int32_t key = min(t0 + col, ri.pos);
    i32x8 b[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) b[ks] = load_codes32(kbase + static_cast<int64_t>(key) * D + ks * 32);
    const float sk = k_scale[ri.key_base + key];
    f32x16 acc[MT];
    tile_mfma8<D, MT>(st, b, acc);
    const float s = sk * tile_epilogue8<D, MT>(st, acc);
    if (half == 0 && t0 + col < c1) out_row[t0 + col] = s;
  }
}

// ---------------------------------------------------------------- prefill kernel

// LDS stage buffers of the prefill kernel, one variable per (array, buffer):
// with each stage's buffer known at compile time, the compiler can tell the
// buffer an in-flight DMA copy fills from the one being read and places no
// wait for the copy before reads of the other.
template <typename T, int ELEMS, int ID, int B>
__device__ __forceinline__ T* stage_lds8() {
  __shared__ __attribute__((aligned(16))) T buf[ELEMS];
  return buf;
}

// A zero the compiler cannot see through, added to a stage buffer's address
// at every stage: both buffers' per-lane read addresses are then not held in
// registers across the stage loop.
__device__ __forceinline__ int32_t opaque_zero8() {
  int32_t z = 0;
  asm volatile("" : "+s"(z));
  return z;
}

template <int D, int MT>
__global__ __launch_bounds__(kBlockRows8 * kWave, 2) void index_scores_fp8_block(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale, const uint8_t* k8,
    const float* k_scale, const float* __restrict__ w, int n_heads, int64_t row_begin,
    int64_t row_count, float* __restrict__ scores, int64_t ld, int key_chunk) {
  constexpr int KS = D / 64;
  constexpr int CHUNKS = D / 16;                                     // 16-byte chunks per key
  constexpr int DMA_PER_WAVE = kStageKeys8 * CHUNKS / (kBlockRows8 * kWave);
  constexpr int TILES = kStageKeys8 / 32;
  static_assert(TILES % 2 == 0 && DMA_PER_WAVE * kBlockRows8 * kWave == kStageKeys8 * CHUNKS,
                "stage shape");
  static_assert(kStageKeys8 == kBlockRows8 * kWave, "every lane carries one key scale");
  // Stage buffers (key codes, key scales), one LDS variable each.
  auto tile = [](auto bb) { return stage_lds8<uint8_t, kStageKeys8 * D, 0, decltype(bb)::value>(); };
  auto tscale = [](auto bb) { return stage_lds8<float, kStageKeys8, 1, decltype(bb)::value>(); };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int col = lane & 31;
  const int half = lane >> 5;
  // Later rows have longer causal prefixes: hand them out first.
  const int64_t blk = static_cast<int64_t>(gridDim.x) - 1 - blockIdx.x;
  const int64_t first = blk * kBlockRows8;
  const int64_t last = min(first + kBlockRows8, row_count) - 1;
  const int64_t local = first + wave;
  const bool active = local < row_count;
  const int64_t row = row_begin + (active ? local : last);

  const RowInfo ri = row_info(cu_q, cu_k, batch, row);
  const RowInfo r_first = row_info(cu_q, cu_k, batch, row_begin + first);
  const RowInfo r_last = row_info(cu_q, cu_k, batch, row_begin + last);
  const int32_t c0 = blockIdx.y * key_chunk;

  RowState8<D, MT> st;
  load_row_state8<D, MT>(st, q8, q_scale, w, row, n_heads, col, half);
  float* out_row = scores + local * ld;

  if (r_first.key_base != r_last.key_base) {
    const int32_t c1 = min(c0 + key_chunk, ri.pos + 1);
    if (active && c0 < c1) row_direct8<D, MT>(st, k8, k_scale, ri, c0, c1, out_row, col, half);
    return;
  }

  const int32_t c_end = min(c0 + key_chunk, r_last.pos + 1);
  if (c0 >= c_end) return;
  const int32_t my_end = active ? min(c0 + key_chunk, ri.pos + 1) : c0;
  const __amdgpu_buffer_rsrc_t keys = raw_buffer(k8 + r_first.key_base * D, (r_last.pos + 1) * D);
  const __amdgpu_buffer_rsrc_t kscl = raw_buffer(k_scale + r_first.key_base, (r_last.pos + 1) * 4);
  const __amdgpu_buffer_rsrc_t outs = raw_buffer(out_row, my_end * 4);

  // Stage fill: DMA instruction i of a wave writes 64 consecutive 16-byte LDS
  // chunks; LDS chunk (key, s) receives global chunk s ^ swz(key).  Every
  // lane also copies one of the stage's key scales (4 bytes).
  constexpr int KPI = kBlockRows8 * kWave / CHUNKS;
  static_assert((KPI / (256 / D)) % CHUNKS == 0 && KPI % (256 / D) == 0,
                "the swizzle must repeat across DMA instructions");
  const int key0 = (wave * kWave + lane) / CHUNKS, s0 = lane % CHUNKS;
  const int dma_off = key0 * D + (s0 ^ swz<D>(key0)) * 16;
  auto fill_stage = [&](auto b, int32_t t) __attribute__((always_inline)) {
    uint8_t* td = tile(b);
    float* sd = tscale(b);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          keys, (__attribute__((address_space(3))) void*)(&td[(i * kBlockRows8 + wave) * kWave * 16]),
          16, dma_off, (t + i * KPI) * D, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
          kscl, (__attribute__((address_space(3))) void*)(&sd[wave * kWave]), 4, lane * 4,
          (t + wave * kWave) * 4, 0, 0);
  };
  auto store = [&](float v, int32_t pos) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), outs, half == 0 ? pos * 4 : 0x7FFFFFF0, 0, 0);
  };
  // B fragment ks of key row r = 32 tj + col of a stage: chunks c and c + 1 of
  // this lane's half of the row (swz(32 tj + col) == swz(col)).
  const int sw = swz<D>(col);
  auto read_b = [&](const uint8_t* tb, int r, int ks) {
    const int c = half * (CHUNKS / 2) + 2 * ks;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(&tb[r * D + ((c ^ sw) * 16)]);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(&tb[r * D + (((c + 1) ^ sw) * 16)]);
    return join(lo, hi);
  };

  fill_stage(B0{}, c0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  f32x16 acc_even[MT], acc_odd[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc_odd[mt] = f32x16{};
  float sk_even = 0.0f, sk_odd = 0.0f;
  int32_t prev_pos = 1 << 28;  // the first epilogue has nothing to store
  // One stage: keys [t0, t0 + kStageKeys8) from buffer bsel, the next
  // stage's copy into the other buffer.
  auto stage = [&](auto bsel, int32_t t0) __attribute__((always_inline)) {
    constexpr int BS = decltype(bsel)::value;
    if (t0 + kStageKeys8 < c_end) fill_stage(std::integral_constant<int, 1 - BS>{}, t0 + kStageKeys8);
    const uint8_t* tb = tile(bsel) + opaque_zero8();
    const float* ts = tscale(bsel);
    i32x8 b[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) b[ks] = read_b(tb, col, ks);
    sk_even = ts[col];
    // The first tile's fragments stay out of the interleaving pattern below.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tj = 0; tj < TILES; ++tj) {
      f32x16 (&acc)[MT] = (tj & 1) ? acc_odd : acc_even;
      f32x16 (&prev)[MT] = (tj & 1) ? acc_even : acc_odd;
      const float sk_prev = (tj & 1) ? sk_even : sk_odd;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = mfma_fp8(st.a[mt][ks], b[ks], ks == 0 ? f32x16{} : acc[mt]);
        // Refill the fragment these MFMAs consumed, a full tile ahead.
        if (tj + 1 < TILES) b[ks] = read_b(tb, (tj + 1) * 32 + col, ks);
      }
      if (tj + 1 < TILES) {
        if (tj & 1) sk_even = ts[(tj + 1) * 32 + col];
        else sk_odd = ts[(tj + 1) * 32 + col];
      }
      store(sk_prev * tile_epilogue8<D, MT>(st, prev), prev_pos);
      prev_pos = t0 + tj * 32 + col;
      // Interleave this tile's MFMAs with the previous tile's epilogue (VALU)
      // and issue each fragment's two LDS reads right after the MFMAs that
      // free it.
#pragma unroll
      for (int i = 0; i < KS * MT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        if (tj + 1 < TILES && i % MT == MT - 1) {
          if (i == KS * MT - 1)
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // fragment and scale reads
          else
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // fragment reads
        }
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);  // VALU
      }
    }
    // Wait for the next stage's DMA only: the TILES score stores issued after
    // it may stay in flight.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(TILES));
    lds_barrier();
  };
  for (int32_t t0 = c0; t0 < c_end; t0 += 2 * kStageKeys8) {
    stage(B0{}, t0);
    if (t0 + kStageKeys8 < c_end) stage(B1{}, t0 + kStageKeys8);
  }
  store(((TILES - 1) & 1 ? sk_odd : sk_even) * tile_epilogue8<D, MT>(st, acc_odd), prev_pos);
}

// ---------------------------------------------------------------- decode kernel

// Each wave owns one (row, key chunk) work item and a private LDS ring of
// kRing8 32-key tiles (codes and scales), filled by coalesced buffer->LDS DMA.
template <int D, int MT>
__global__ __launch_bounds__(kStreamRows8 * kWave) void index_scores_fp8_stream(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k8, const float* __restrict__ k_scale,
    const float* __restrict__ w, int n_heads, int64_t row_begin, int64_t row_count,
    float* __restrict__ scores, int64_t ld, int key_chunk, int chunks_per_row) {
  constexpr int KS = D / 64;
  constexpr int CHUNKS = D / 16;
  constexpr int DMA_PER_TILE = 32 * CHUNKS / kWave;
  static_assert(DMA_PER_TILE * kWave == 32 * CHUNKS, "tile shape");
  __shared__ __attribute__((aligned(16))) uint8_t ring[kStreamRows8][kRing8][32 * D];
  __shared__ float sring[kStreamRows8][kRing8][kWave];

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kStreamRows8 + wave;
  const int64_t local = item / chunks_per_row;
  if (local >= row_count) return;
  const int64_t row = row_begin + local;
  const RowInfo ri = row_info(cu_q, cu_k, batch, row);
  const int32_t c0 = static_cast<int32_t>(item % chunks_per_row) * key_chunk;
  const int32_t c1 = min(c0 + key_chunk, ri.pos + 1);
  if (c0 >= c1) return;
  RowState8<D, MT> st;
  load_row_state8<D, MT>(st, q8, q_scale, w, row, n_heads, col, half);

  const __amdgpu_buffer_rsrc_t keys = raw_buffer(k8 + (ri.key_base + c0) * D, (c1 - c0) * D);
  const __amdgpu_buffer_rsrc_t kscl = raw_buffer(k_scale + ri.key_base + c0, (c1 - c0) * 4);
  const __amdgpu_buffer_rsrc_t outs = raw_buffer(scores + local * ld, c1 * 4);
  // Tile of keys c0 + t .. c0 + t + 31: DMA_PER_TILE code copies, then one
  // scale copy (both half-waves fetch the same 32 scales).
  auto fill = [&](int slot, int32_t t) {
#pragma unroll
    for (int i = 0; i < DMA_PER_TILE; ++i) {
      const int e = i * kWave + lane;
      const int key = e / CHUNKS, s = e % CHUNKS;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          keys, (__attribute__((address_space(3))) void*)(&ring[wave][slot][i * kWave * 16]), 16,
          key * D + (s ^ ((key / (256 / D)) & (CHUNKS - 1))) * 16, t * D, 0, 0);  // s ^ swz(key)
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        kscl, (__attribute__((address_space(3))) void*)(&sring[wave][slot][0]), 4, col * 4, t * 4,
        0, 0);
  };
  auto store = [&](float v, int32_t pos) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), outs, half == 0 ? pos * 4 : 0x7FFFFFF0, 0, 0);
  };

#pragma unroll
  for (int p = 0; p < kRing8 - 1; ++p) {
    fill(p, p * 32);
    store(0.0f, 1 << 28);
  }
  f32x16 acc[MT], prev[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) prev[mt] = f32x16{};
  float sk_prev = 0.0f;
  int32_t prev_pos = 1 << 28;
  const int ntiles = (c1 - c0 + 31) / 32;
  for (int j = 0; j < ntiles; ++j) {
    fill((j + kRing8 - 1) % kRing8, (j + kRing8 - 1) * 32);
    // Tile j has landed once at most the kRing8 - 1 younger tiles' copies and
    // their trailing stores are outstanding.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kRing8 - 1) * (DMA_PER_TILE + 2)));
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint8_t* tb = ring[wave][j % kRing8];
    i32x8 b[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = half * (CHUNKS / 2) + 2 * ks;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(&tb[col * D + ((c ^ swz<D>(col)) * 16)]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(&tb[col * D + (((c + 1) ^ swz<D>(col)) * 16)]);
      b[ks] = join(lo, hi);
    }
    const float sk = sring[wave][j % kRing8][col];
    tile_mfma8<D, MT>(st, b, acc);
    store(sk_prev * tile_epilogue8<D, MT>(st, prev), prev_pos);
    prev_pos = c0 + j * 32 + col;
    sk_prev = sk;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) prev[mt] = acc[mt];
    // The slot refilled next iteration was read above.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  }
  store(sk_prev * tile_epilogue8<D, MT>(st, prev), prev_pos);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

template <int D, int MT>
hipError_t launch_fp8_dm(const dsa_varlen& vl, const uint8_t* q8, const float* qs,
                         const uint8_t* k8, const float* ks, const float* w, int n_heads,
                         int64_t row_begin, int64_t row_count, float* scores, int64_t ld,
                         hipStream_t stream) {
  if (vl.max_seqlen_q >= kBlockRows8) {
    const int64_t blocks = (row_count + kBlockRows8 - 1) / kBlockRows8;
    int64_t chunk = vl.max_seqlen_k;
    if (blocks < 1024) {
      const int64_t parts = (1024 + blocks - 1) / blocks;
      chunk = (vl.max_seqlen_k + parts - 1) / parts;
    }
    chunk = ((chunk + kStageKeys8 - 1) / kStageKeys8) * kStageKeys8;
    if (chunk < 512) chunk = 512;
    const int64_t chunks = (vl.max_seqlen_k + chunk - 1) / chunk;
    hipLaunchKernelGGL((index_scores_fp8_block<D, MT>), dim3(static_cast<unsigned>(blocks),
                       static_cast<unsigned>(chunks)), dim3(kBlockRows8 * kWave), 0, stream,
                       vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, q8, qs, k8, ks, w, n_heads,
                       row_begin, row_count, scores, ld, static_cast<int>(chunk));
  } else {
    const int64_t per_row = (2048 + row_count - 1) / row_count;
    int64_t chunk = (vl.max_seqlen_k + per_row - 1) / per_row;
    chunk = ((chunk + 31) / 32) * 32;
    if (chunk < 512) chunk = 512;
    const int64_t chunks_per_row = (vl.max_seqlen_k + chunk - 1) / chunk;
    const int64_t items = row_count * chunks_per_row;
    hipLaunchKernelGGL((index_scores_fp8_stream<D, MT>),
                       dim3(static_cast<unsigned>((items + kStreamRows8 - 1) / kStreamRows8)),
                       dim3(kStreamRows8 * kWave), 0, stream, vl.cu_seqlens_q, vl.cu_seqlens_k,
                       vl.batch, q8, qs, k8, ks, w, n_heads, row_begin, row_count, scores, ld,
                       static_cast<int>(chunk), static_cast<int>(chunks_per_row));
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_fp8_d(const dsa_varlen& vl, const uint8_t* q8, const float* qs,
                        const uint8_t* k8, const float* ks, const float* w, int n_heads,
                        int64_t row_begin, int64_t row_count, float* scores, int64_t ld,
                        hipStream_t stream) {
  if (n_heads > 32)
    return launch_fp8_dm<D, 2>(vl, q8, qs, k8, ks, w, n_heads, row_begin, row_count, scores, ld,
                               stream);
  return launch_fp8_dm<D, 1>(vl, q8, qs, k8, ks, w, n_heads, row_begin, row_count, scores, ld,
                             stream);
}

// ---------------------------------------------------------------- quantisation

// Vectors of D bf16 values -> D e4m3 codes and one scale.  D / 8 lanes share a
// vector (16 bytes each); every step is binary32: amax, inv = 448 / amax
// (correctly rounded division), code = e4m3(x * inv) rounded to nearest even
// by v_cvt_pk_fp8_f32 (which saturates at 448), scale = amax / 448.
template <int D>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t* __restrict__ x,
                                                           int64_t rows,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ scales) {
  constexpr int LPR = D / 8;      // lanes per vector
  constexpr int RPW = kWave / LPR;  // vectors per wave and step
  const int lane = lane_id();
  const int sub = lane % LPR;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * blockDim.x / kWave;
  for (int64_t r0 = wave * RPW; r0 < rows; r0 += waves * RPW) {
    const int64_t r = r0 + lane / LPR;
    const bool ok = r < rows;
    u32x4 u = ok ? *reinterpret_cast<const u32x4*>(x + r * D + sub * 8) : u32x4{0u, 0u, 0u, 0u};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    uint32_t lo = 0u, hi = 0u;
    if (m > 0.0f) {
      const float inv = 448.0f / m;
      lo = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(v[0] * inv, v[1] * inv, 0, false));
      lo = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(v[2] * inv, v[3] * inv, static_cast<int>(lo), true));
      hi = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(v[4] * inv, v[5] * inv, 0, false));
      hi = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(v[6] * inv, v[7] * inv, static_cast<int>(hi), true));
    }
    if (ok) {
      *reinterpret_cast<uint2*>(codes + r * D + sub * 8) = make_uint2(lo, hi);
      if (sub == 0) scales[r] = m / 448.0f;
    }
  }
}

}  // namespace

hipError_t launch_index_scores_fp8(const dsa_varlen& vl, const uint8_t* q8, const float* q_scale,
                                   const uint8_t* k8, const float* k_scale, const float* w,
                                   int n_heads, int d, int64_t row_begin, int64_t row_count,
                                   float* scores, int64_t ld, hipStream_t stream) {
  if (d == 128)
    return launch_fp8_d<128>(vl, q8, q_scale, k8, k_scale, w, n_heads, row_begin, row_count,
                             scores, ld, stream);
  return launch_fp8_d<64>(vl, q8, q_scale, k8, k_scale, w, n_heads, row_begin, row_count, scores,
                          ld, stream);
}

hipError_t launch_quantize_fp8(const uint16_t* x, int64_t rows, int d, uint8_t* codes,
                               float* scales, hipStream_t stream) {
  // Grid-stride over vectors: enough waves to keep every CU streaming.
  const int64_t per_block = 4 * (kWave / (d / 8));
  int64_t blocks = (rows + per_block - 1) / per_block;
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (d == 128)
    hipLaunchKernelGGL(quantize_fp8_kernel<128>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, x, rows, codes, scales);
  else
    hipLaunchKernelGGL(quantize_fp8_kernel<64>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, x, rows, codes, scales);
  return hipGetLastError();
}

}  // namespace dsa
