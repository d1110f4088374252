// indexer_kl.hip -- the indexer's warm-up loss and its gradient on gfx950.
//
// Page 5 (Keye-VL-2.0 report summary), section 1, on the two training
// stages: in the dense warm-up the rest of the model is frozen and only the
// indexer is trained, so that its distribution over positions approaches
// the full attention's, the gap measured by KL divergence.  For query row t
// at position p (keys s = 0..p), with G = Hq / Hkv:
//   A_h[s]   = softmax_s(scale * Q[t,h] . K[s, h / G])       dense attention of head h
//   P[s]     = (1 / Hq) sum_h A_h[s]                         the target, heads averaged
//   Pi[s]    = softmax_s(I[t,s])                             the indexer's distribution
//   loss[t]  = sum_s P[s] (ln P[s] - ln Pi[s])               KL(P || Pi)
//   grad[t,s] = Pi[s] - P[s]                                 d loss[t] / d I[t,s]
//
// One workgroup serves 16 consecutive query rows; they are the 16 columns
// of mfma_f32_16x16x32_bf16 (B operand: one query head of the 16 rows), so
// no MFMA column is wasted whatever Hq / Hkv is.  W waves split the Hq
// heads (HPW = Hq / W each).  Key tiles of 32 positions with all KV heads
// are staged in LDS (XOR-swizzled like the attention tiles) and shared by
// all waves: two LDS buffers, the next tile copied into one by
// buffer->LDS DMA while the other is used.
//   Pass 1: the dense logits of every head, for the running max and sum of
//           each (row, head) softmax, and the rows' indexer scores, for the
//           max and sum of theirs.
//   Pass 2: the logits again; each wave sums exp(z - m) / l over its heads
//           for every (key, row) into LDS, and one thread per (row, key)
//           adds the waves' sums (/ Hq = P), forms Pi from the score and the
//           row's normaliser, accumulates the KL term and writes the
//           gradient.
// Rows of several sequences in one workgroup are served one sequence at a
// time, the other rows' columns masked.
#include <type_traits>

#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kKlRows = 16;  // query rows per workgroup (MFMA columns)
constexpr int kKlKeys = 32;  // positions per tile
constexpr float kKlLog2e = 1.4426950408889634f;
constexpr float kKlLn2 = 0.6931471805599453f;
// Growth of a (row, head) maximum (log2 units) that pass 1's running
// reference absorbs before it is moved: terms of the running sum stay below
// 2^8, and most half tiles skip the rescale's exponential.
constexpr float kKlRescaleLog2 = 8.0f;

template <int D>
struct KlCfg {
  static constexpr int KS = D / 32;      // k-steps of one logit tile
  static constexpr int PIECES = D / 8;   // 16-byte pieces of one K row
};

// LDS element of piece `piece` of KV head g of tile key `key`.
template <int D>
__device__ __forceinline__ int kl_at(int key, int g, int n_heads_kv, int piece) {
  return (key * n_heads_kv + g) * D + ((piece ^ (key % KlCfg<D>::PIECES)) * 8);
}

// LDS: two K tile buffers of ELEMS bf16 (the copies of one tile, at least
// 32 keys x Hkv x D; one static variable apiece, so that the compiler sees
// which buffer a copy in flight writes and places no wait for it before
// reads of the other), the waves' partial sums [W][16 rows][kPStride] fp32
// (32 keys, padded) and the per-row words.
constexpr int kPStride = kKlKeys + 1;
// s_waitcnt immediate: lgkmcnt(0), vmcnt and expcnt left unconstrained.
constexpr int kLgkmcnt0 = 0xF | (3 << 14) | 0x70;
// Scheduling of a block that issues one tile's MFMAs beside independent
// VALU work: the K-fragment reads first, then NVALU VALU instructions
// after each of the NMFMA MFMAs, so the wave's exponentials issue while its
// matrix products run instead of after the last of them.
template <int NMFMA, int NVALU>
__device__ __forceinline__ void interleave_mfma_valu() {
  __builtin_amdgcn_sched_group_barrier(0x100, NMFMA / 4, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);  // VALU
  }
}

template <int ELEMS, int B>
__device__ __forceinline__ uint16_t* kl_kbuf() {
  __shared__ __attribute__((aligned(16))) uint16_t buf[ELEMS];
  return buf;
}

template <int D, int HPW, int W, int CPT>
__global__ __launch_bounds__(W * kWave) void indexer_kl_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ scores, int64_t ld, int64_t row_begin, int64_t row_count,
    int n_heads_q, int n_heads_kv, float scale_log2, float* __restrict__ loss,
    float* __restrict__ grad, int64_t ld_grad) {
  using C = KlCfg<D>;
  constexpr int NT = W * kWave;
  constexpr int RI = kKlRows * kKlKeys / NT;  // (row, key) entries per thread
  static_assert(RI * NT == kKlRows * kKlKeys, "entries split evenly");
  __shared__ float ppart[W * kKlRows * kPStride];
  __shared__ int32_t rowkb[kKlRows];   // key base per row
  __shared__ int32_t rowpos[kKlRows];  // position per row

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 15, qd = lane >> 4;
  const int G = n_heads_q / n_heads_kv;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * kKlRows;
  const int n_rows = static_cast<int>(min<int64_t>(kKlRows, row_count - first));

  if (tid < kKlRows) {
    const int64_t lr = first + min(tid, n_rows - 1);
    const RowInfo ri = row_info(cu_q, cu_k, batch, row_begin + lr);
    rowkb[tid] = tid < n_rows ? static_cast<int32_t>(ri.key_base) : -1;
    rowpos[tid] = tid < n_rows ? ri.pos : -1;
  }
  __syncthreads();

  // This lane's query column and this thread's (row, key) entries.
  const int my_kb = rowkb[col], my_pos = rowpos[col];
  int e_row[RI], e_key[RI];
#pragma unroll
  for (int i = 0; i < RI; ++i) {
    const int e = tid + NT * i;
    e_row[i] = e / kKlKeys;
    e_key[i] = e % kKlKeys;
  }

  // Q of this wave's heads for the 16 rows (B operands).
  bf16x8 qb[HPW][C::KS];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int h = wave * HPW + j;
    const int64_t lr = first + min(col, n_rows - 1);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qb[j][ks] = load_bf16x8(q + ((row_begin + lr) * n_heads_q + h) * D + ks * 32 + qd * 8);
  }

  // 16-byte chunks of one K tile, CPT per thread (the launcher picks CPT =
  // ceil(chunks / NT)), copied from global memory to LDS by buffer->LDS
  // DMA: copy i of a wave fills LDS chunks cbase .. cbase + 63 (cbase
  // uniform), chunk cb being physical piece cb mod PIECES of LDS row
  // cb / PIECES (key * Hkv + g), filled from global piece
  // (cb mod PIECES) ^ (key mod PIECES) (kl_at's swizzle).  Chunks past the
  // tile read a clamped valid chunk into the buffer's unused part.
  constexpr int KB = CPT * NT * 8;  // bf16 per buffer
  const int chunks = kKlKeys * n_heads_kv * C::PIECES;

  // Serve the rows one sequence at a time (key bases ascend with the row).
  int32_t seg_kb = rowkb[0];
  while (true) {
    int32_t pmax = -1;
    for (int r = 0; r < n_rows; ++r)
      if (rowkb[r] == seg_kb) pmax = max(pmax, rowpos[r]);
    const bool col_in = my_kb == seg_kb;
    const int ntiles = (pmax + kKlKeys) / kKlKeys;
    const uint16_t* kseq = k + static_cast<int64_t>(seg_kb) * n_heads_kv * D;

    // Starts the copy of tile t into kt.  The tile's visible K rows (keys
    // t * 32 .. min(t * 32 + 31, pmax)) form one range-checked buffer; a
    // key past pmax is clamped to the last of them.
    auto issue_tile = [&](int t, uint16_t* kt) __attribute__((always_inline)) {
      const int rows = min(kKlKeys, pmax + 1 - t * kKlKeys);
      const __amdgpu_buffer_rsrc_t krs =
          raw_buffer(kseq + static_cast<int64_t>(t) * kKlKeys * n_heads_kv * D,
                     rows * n_heads_kv * D * 2);
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int cbase = i * NT + kWave * wave;
        const int cc = min(cbase + lane, chunks - 1);
        const int rowg = cc / C::PIECES;
        const int key = rowg / n_heads_kv, g = rowg % n_heads_kv;
        const int piece = (cc % C::PIECES) ^ (key % C::PIECES);
        const int off = ((min(key, rows - 1) * n_heads_kv + g) * D + piece * 8) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            krs, (__attribute__((address_space(3))) void*)(kt + cbase * 8), 16, off, 0, 0, 0);
      }
    };
    // The two buffers; tile t is staged in buffer t mod 2.
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    // Scores of this thread's entries of the tile at t (-inf when not
    // visible); the address is clamped into the row, so the load carries no
    // branch.
    auto load_scores = [&](int t, float (&sv)[RI]) {
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        const int r = min(e_row[i], n_rows - 1);
        const int s = t * kKlKeys + e_key[i];
        const bool vis = e_row[i] < n_rows && rowkb[r] == seg_kb && s <= rowpos[r];
        const float x = scores[(first + r) * ld + min(s, max(rowpos[r], 0))];
        sv[i] = vis ? x : -INFINITY;
      }
    };
    // Raw dot products of the tile in kt for all HPW heads: st[sub][j][r]
    // is head j's product with key 16 sub + 4 qd + r of this lane's row.
    // The wave's heads share one KV head (Hq = 2^n <= 64 split over
    // W = min(8, Hq) waves, Hkv in {1, 2, 4, 8} dividing Hq: G = Hq / Hkv
    // is a multiple of HPW), so each K fragment is read from LDS once for
    // all of them.
    const int g_w = wave * HPW / G;
    auto tile_dots = [&](const uint16_t* kt, f32x4 (&st)[2][HPW]) __attribute__((always_inline)) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int j = 0; j < HPW; ++j) st[sub][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const bf16x8 ka = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(
                          kt + kl_at<D>(16 * sub + col, g_w, n_heads_kv, 4 * ks + qd)));
#pragma unroll
          for (int j = 0; j < HPW; ++j)
            st[sub][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[j][ks], st[sub][j], 0, 0, 0);
        }
      }
    };
    // Logits (log2 domain) of head j for tile t from its products, -inf
    // where not visible.
    auto logits = [&](const f32x4 (&st)[2][HPW], int t, int j, float (&z)[2][4])
        __attribute__((always_inline)) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = t * kKlKeys + 16 * sub + 4 * qd + r;
          z[sub][r] = col_in && s <= my_pos ? st[sub][j][r] * scale_log2 : -INFINITY;
        }
    };
    // A tile is full when all 16 rows belong to this sequence and see all
    // of its keys: no masking then, and the scale folds into the exponent's
    // FMA (softmax_scale > 0, which the caller checks).
    bool all_in = n_rows == kKlRows;
    int32_t min_pos = pmax;
    for (int r = 0; r < kKlRows; ++r) {
      all_in = all_in && rowkb[r] == seg_kb;
      min_pos = min(min_pos, rowpos[r]);
    }
    const int full_tiles = all_in ? (min_pos + 1) / kKlKeys : 0;

    // Both passes are software-pipelined by one tile: step t issues tile
    // t's MFMAs and then does the exponential work of tile t - 1, whose
    // products the step before left in registers.  In the steps whose
    // previous tile is full, that work and the MFMAs form one basic block,
    // scheduled so that each wave's VALU work runs beside its own matrix
    // products.  Tile t sits in K buffer t % 2 and its products in stA (t
    // even) or stB (t odd).
    f32x4 stA[2][HPW], stB[2][HPW];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int j = 0; j < HPW; ++j) stA[sub][j] = stB[sub][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Step t: once tile t has landed for every wave (and every wave is done
    // with tile t - 1, whose buffer is refilled next), the copy of tile t + 1
    // and the load of its scores are started, unconditionally (the last
    // tile copies itself again), and tile t is used while they are in
    // flight.  One drain and one barrier per tile.
    auto begin_step = [&](auto b, int t, float (&sv)[RI], float (&sv_next)[RI])
        __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      lds_barrier();
#pragma unroll
      for (int i = 0; i < RI; ++i) sv[i] = sv_next[i];
      issue_tile(min(t + 1, ntiles - 1), kl_kbuf<KB, 1 - decltype(b)::value>());
      load_scores(min(t + 1, ntiles - 1), sv_next);
    };
    // A pass's steps: step(b, t, cur, next) with cur the products of tile
    // t - 1 and next the set for tile t's.  Steps 0 and 1 and the steps
    // after the full tiles take the generic step, the pairs of steps in
    // between the fast one; the last tile's values follow the loop.
    auto run_pass = [&](auto fast_step, auto generic_step, auto last_values)
        __attribute__((always_inline)) {
      generic_step(B0{}, 0, stB, stA);
      int t = 1;
      if (ntiles > 1) {
        generic_step(B1{}, 1, stA, stB);
        t = 2;
      }
      const int tf = min(full_tiles, ntiles - 1);  // last step whose previous tile is full
      for (; t + 1 <= tf; t += 2) {
        fast_step(B0{}, t, stB, stA);
        fast_step(B1{}, t + 1, stA, stB);
      }
      for (; t < ntiles; t += 2) {
        generic_step(B0{}, t, stB, stA);
        if (t + 1 < ntiles) generic_step(B1{}, t + 1, stA, stB);
      }
      if ((ntiles - 1) & 1) last_values(stB, ntiles - 1);
      else last_values(stA, ntiles - 1);
    };

    // ---- pass 1: per-(row, head) softmax statistics, per-row indexer ones.
    float hm[HPW], hl[HPW];
#pragma unroll
    for (int j = 0; j < HPW; ++j) { hm[j] = -INFINITY; hl[j] = 0.0f; }
    float im[RI], il[RI];
#pragma unroll
    for (int i = 0; i < RI; ++i) { im[i] = -INFINITY; il[i] = 0.0f; }
    // Full tiles: the reference hm moves only when a lane's term would pass
    // 2^kKlRescaleLog2 (lazy rescaling; the first tile always moves it from
    // -inf), so the sum's terms are taken against a reference up to 2^8
    // below the maximum, and the final reduction, which rescales every
    // lane's sum from its own reference, is unchanged.  The sums h are
    // taken against the current reference first; where a lane's tile sum
    // passes 2^8 (the only way one of its terms can), the tile is redone
    // with the lane maxima (redo1), which moves exactly the lanes whose
    // maximum passed the reference by more than 2^8.
    auto sums1 = [&](const f32x4 (&st)[2][HPW], float (&h)[HPW], bool& redo)
        __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        h[j] = hl[j];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            h[j] += __builtin_amdgcn_exp2f(__builtin_fmaf(st[sub][j][r], scale_log2, -hm[j]));
        redo = redo | !(h[j] <= hl[j] + 256.0f);
      }
    };
    auto redo1 = [&](const f32x4 (&st)[2][HPW], float (&h)[HPW]) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const float mx = fmaxf(fmaxf(fmaxf(st[0][j][0], st[0][j][1]), fmaxf(st[0][j][2], st[0][j][3])),
                               fmaxf(fmaxf(st[1][j][0], st[1][j][1]), fmaxf(st[1][j][2], st[1][j][3]))) *
                         scale_log2;
        const bool move = mx > hm[j] + kKlRescaleLog2;
        const float mn = move ? mx : hm[j];
        h[j] = hl[j] * __builtin_amdgcn_exp2f(hm[j] - mn);
        hm[j] = mn;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            h[j] += __builtin_amdgcn_exp2f(__builtin_fmaf(st[sub][j][r], scale_log2, -hm[j]));
      }
    };
    // Tiles with masked entries: the exact running max and sum.
    auto masked1 = [&](const f32x4 (&st)[2][HPW], int t) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        float z[2][4];
        logits(st, t, j, z);
        float mx = -INFINITY;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, z[sub][r]);
        const float mn = fmaxf(hm[j], mx);
        if (mn != -INFINITY) {
          float sum = 0.0f;
#pragma unroll
          for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int r = 0; r < 4; ++r) sum += __builtin_amdgcn_exp2f(z[sub][r] - mn);
          hl[j] = hl[j] * __builtin_amdgcn_exp2f(hm[j] - mn) + sum;
          hm[j] = mn;
        }
      }
    };
    // Statistics of tile t (nothing for t < 0).
    auto values1 = [&](const f32x4 (&st)[2][HPW], int t) __attribute__((always_inline)) {
      float h[HPW];
      bool redo = false;
      if (static_cast<unsigned>(t) < static_cast<unsigned>(full_tiles)) {
        sums1(st, h, redo);
      } else {
        if (t >= 0) masked1(st, t);
#pragma unroll
        for (int j = 0; j < HPW; ++j) h[j] = hl[j];
      }
      if (__any(redo)) redo1(st, h);
#pragma unroll
      for (int j = 0; j < HPW; ++j) hl[j] = h[j];
    };
    // The indexer's own running statistics over the tile's scores.
    auto score_stats = [&](const float (&sv)[RI]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        if (sv[i] != -INFINITY) {
          const float x = sv[i] * kKlLog2e;
          const float mn = fmaxf(im[i], x);
          il[i] = il[i] * __builtin_amdgcn_exp2f(im[i] - mn) + __builtin_amdgcn_exp2f(x - mn);
          im[i] = mn;
        }
      }
    };
    float sv_next[RI];
    auto step1 = [&](auto b, int t, f32x4 (&cur)[2][HPW], f32x4 (&next)[2][HPW])
        __attribute__((always_inline)) {
      float sv[RI];
      begin_step(b, t, sv, sv_next);
      tile_dots(kl_kbuf<KB, decltype(b)::value>(), next);
      values1(cur, t - 1);
      score_stats(sv);
    };
    auto fast1 = [&](auto b, int t, f32x4 (&cur)[2][HPW], f32x4 (&next)[2][HPW])
        __attribute__((always_inline)) {
      float sv[RI];
      begin_step(b, t, sv, sv_next);
      float h[HPW];
      bool redo = false;
      tile_dots(kl_kbuf<KB, decltype(b)::value>(), next);
      sums1(cur, h, redo);
      interleave_mfma_valu<2 * HPW * C::KS, 3>();
      if (__any(redo)) redo1(cur, h);
#pragma unroll
      for (int j = 0; j < HPW; ++j) hl[j] = h[j];
      score_stats(sv);
    };
    load_scores(0, sv_next);
    issue_tile(0, kl_kbuf<KB, 0>());
    run_pass(fast1, step1, values1);
    // Whole-row statistics: the four lane quarters hold one row's keys.
    // hb[j] = log2 of the normaliser of head j: A = exp2(z - hb[j]).
    float hb[HPW];
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      float m = fmaxf(hm[j], __shfl_xor(hm[j], 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      float l = hm[j] == -INFINITY ? 0.0f : hl[j] * exp2f(hm[j] - m);
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      hb[j] = l > 0.0f ? m + log2f(l) : INFINITY;  // no visible key: A = 0
    }
    // The 32 entries of one row sit in 32 consecutive lanes.
    float lnorm[RI];
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      float m = im[i];
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
      float l = im[i] == -INFINITY ? 0.0f : il[i] * exp2f(im[i] - m);
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) l += __shfl_xor(l, o);
      lnorm[i] = (m + log2f(l)) * kKlLn2;  // ln sum_s exp(I[s])
    }

    // ---- pass 2: the target, the KL terms and the gradient.
    float kl[RI];
#pragma unroll
    for (int i = 0; i < RI; ++i) kl[i] = 0.0f;
    const float inv_hq = 1.0f / static_cast<float>(n_heads_q);
    // Tile t's gradient is stored in step t + 2, after that step's loads
    // are issued, so the drain that opens the next step finds the stores
    // long done instead of waiting for them right after they were issued.
    float gval[RI], sv_prev[RI];
    bool gok[RI];
#pragma unroll
    for (int i = 0; i < RI; ++i) { gval[i] = 0.0f; gok[i] = false; sv_prev[i] = -INFINITY; }
    auto store_grads = [&](int t) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < RI; ++i)
        if (gok[i]) grad[(first + e_row[i]) * ld_grad + t * kKlKeys + e_key[i]] = gval[i];
    };
    // Each wave sums A = exp2(z - hb) over its heads for every (key, row)
    // of the tile.
    auto sums2 = [&](const f32x4 (&st)[2][HPW], float (&acc)[2][4]) __attribute__((always_inline)) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int j = 0; j < HPW; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[sub][r] += __builtin_amdgcn_exp2f(__builtin_fmaf(st[sub][j][r], scale_log2, -hb[j]));
    };
    auto masked2 = [&](const f32x4 (&st)[2][HPW], int t, float (&acc)[2][4])
        __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        float z[2][4];
        logits(st, t, j, z);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[sub][r] += __builtin_amdgcn_exp2f(z[sub][r] - hb[j]);
      }
    };
    // The waves' sums go through LDS; after a barrier one thread per (row,
    // key) adds them (/ Hq = P), forms ln Pi from the score and the row's
    // normaliser, accumulates the KL term and keeps Pi - P for the store.
    auto finish2 = [&](const float (&acc)[2][4], const float (&sv_t)[RI]) __attribute__((always_inline)) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          ppart[(wave * kKlRows + col) * kPStride + 16 * sub + 4 * qd + r] = acc[sub][r];
      // LDS writes done, nothing else: a workgroup fence here would also
      // wait for the next tile's copy.
      __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
      lds_barrier();
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        const int r = e_row[i];
        gok[i] = grad != nullptr && sv_t[i] != -INFINITY;
        if (sv_t[i] != -INFINITY) {
          float psum = 0.0f;
#pragma unroll
          for (int w = 0; w < W; ++w) psum += ppart[(w * kKlRows + r) * kPStride + e_key[i]];
          const float P = psum * inv_hq;
          const float lpi = sv_t[i] - lnorm[i];
          const float pi = __builtin_amdgcn_exp2f(lpi * kKlLog2e);
          if (P > 0.0f) kl[i] += P * (__builtin_amdgcn_logf(P) * kKlLn2 - lpi);
          gval[i] = pi - P;
        }
      }
    };
    // Tile t (nothing for t < 0), its scores in sv_prev.
    auto values2 = [&](const f32x4 (&st)[2][HPW], int t) __attribute__((always_inline)) {
      if (t < 0) return;
      float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      if (t < full_tiles) sums2(st, acc);
      else masked2(st, t, acc);
      finish2(acc, sv_prev);
    };
    // Every step starts with: every wave is done reading the partial sums.
    auto step2 = [&](auto b, int t, f32x4 (&cur)[2][HPW], f32x4 (&next)[2][HPW])
        __attribute__((always_inline)) {
      float sv[RI];
      begin_step(b, t, sv, sv_next);
      store_grads(t - 2);
      tile_dots(kl_kbuf<KB, decltype(b)::value>(), next);
      values2(cur, t - 1);
#pragma unroll
      for (int i = 0; i < RI; ++i) sv_prev[i] = sv[i];
    };
    auto fast2 = [&](auto b, int t, f32x4 (&cur)[2][HPW], f32x4 (&next)[2][HPW])
        __attribute__((always_inline)) {
      float sv[RI];
      begin_step(b, t, sv, sv_next);
      store_grads(t - 2);
      float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      tile_dots(kl_kbuf<KB, decltype(b)::value>(), next);
      sums2(cur, acc);
      interleave_mfma_valu<2 * HPW * C::KS, 3>();
      finish2(acc, sv_prev);
#pragma unroll
      for (int i = 0; i < RI; ++i) sv_prev[i] = sv[i];
    };
    // The last tile: once every wave is done with tile ntiles - 2's partial
    // sums.
    auto last2 = [&](const f32x4 (&st)[2][HPW], int t) __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
      lds_barrier();
      store_grads(t - 1);
      values2(st, t);
      store_grads(t);
    };
    // Every wave is done with pass 1's last tile before tile 0 is copied
    // again.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
    load_scores(0, sv_next);
    issue_tile(0, kl_kbuf<KB, 0>());
    run_pass(fast2, step2, last2);
    // Per-row loss: the row's 32 lanes.
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      float v = kl[i];
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) v += __shfl_xor(v, o);
      const int r = e_row[i];
      if (e_key[i] == 0 && r < n_rows && rowkb[r] == seg_kb) loss[first + r] = v;
    }

    // Next sequence among the rows, if any.
    int32_t next = -1;
    for (int r = 0; r < n_rows; ++r)
      if (rowkb[r] > seg_kb) { next = rowkb[r]; break; }
    if (next < 0) break;
    seg_kb = next;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the last step's copy has landed
    __syncthreads();
  }
}

template <int D, int HPW, int W, int CPT>
hipError_t launch_kl_d(const dsa_varlen& vl, const uint16_t* q, const uint16_t* k,
                       const float* scores, int64_t ld, int64_t row_begin, int64_t row_count,
                       int n_heads_q, int n_heads_kv, float scale, float* loss, float* grad,
                       int64_t ld_grad, hipStream_t stream) {
  const unsigned blocks = static_cast<unsigned>((row_count + kKlRows - 1) / kKlRows);
  hipLaunchKernelGGL((indexer_kl_kernel<D, HPW, W, CPT>), dim3(blocks), dim3(W * kWave), 0, stream,
                     vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, q, k, scores, ld, row_begin,
                     row_count, n_heads_q, n_heads_kv, scale * kKlLog2e, loss, grad, ld_grad);
  return hipGetLastError();
}

template <int D>
hipError_t launch_kl_heads(const dsa_varlen& vl, const uint16_t* q, const uint16_t* k,
                           const float* scores, int64_t ld, int64_t row_begin, int64_t row_count,
                           int n_heads_q, int n_heads_kv, float scale, float* loss, float* grad,
                           int64_t ld_grad, hipStream_t stream) {
  // W = min(8, Hq) waves, Hq / W heads each (the caller checks Hq in
  // {1, 2, 4, 8, 16, 32, 64}); CPT = the K-tile chunks each thread moves,
  // 32 Hkv D / 8 over 64 W threads (Hkv <= min(Hq, 8): 1, 2, 4 or 8).
  const int waves = n_heads_q < 8 ? n_heads_q : 8;
  const int cpt = (kKlKeys * n_heads_kv * (D / 8) + kWave * waves - 1) / (kWave * waves);
#define DSA_KL(HPW, W)                                                                        \
  switch (cpt) {                                                                              \
    case 1: return launch_kl_d<D, HPW, W, 1>(vl, q, k, scores, ld, row_begin, row_count,      \
                                             n_heads_q, n_heads_kv, scale, loss, grad,        \
                                             ld_grad, stream);                                \
    case 2: return launch_kl_d<D, HPW, W, 2>(vl, q, k, scores, ld, row_begin, row_count,      \
                                             n_heads_q, n_heads_kv, scale, loss, grad,        \
                                             ld_grad, stream);                                \
    case 4: return launch_kl_d<D, HPW, W, 4>(vl, q, k, scores, ld, row_begin, row_count,      \
                                             n_heads_q, n_heads_kv, scale, loss, grad,        \
                                             ld_grad, stream);                                \
    default: return launch_kl_d<D, HPW, W, 8>(vl, q, k, scores, ld, row_begin, row_count,     \
                                              n_heads_q, n_heads_kv, scale, loss, grad,       \
                                              ld_grad, stream);                               \
  }
  switch (n_heads_q) {
    case 1: DSA_KL(1, 1);
    case 2: DSA_KL(1, 2);
    case 4: DSA_KL(1, 4);
    case 8: DSA_KL(1, 8);
    case 16: DSA_KL(2, 8);
    case 32: DSA_KL(4, 8);
    default: DSA_KL(8, 8);
  }
#undef DSA_KL
}

}  // namespace

hipError_t launch_indexer_kl(const dsa_varlen& vl, const uint16_t* q, const uint16_t* k,
                             const float* scores, int64_t ld, int64_t row_begin,
                             int64_t row_count, int n_heads_q, int n_heads_kv, int head_dim,
                             float scale, float* loss, float* grad, int64_t ld_grad,
                             hipStream_t stream) {
  if (head_dim == 128)
    return launch_kl_heads<128>(vl, q, k, scores, ld, row_begin, row_count, n_heads_q,
                                n_heads_kv, scale, loss, grad, ld_grad, stream);
  return launch_kl_heads<64>(vl, q, k, scores, ld, row_begin, row_count, n_heads_q, n_heads_kv,
                             scale, loss, grad, ld_grad, stream);
}

}  // namespace dsa
