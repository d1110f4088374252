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
// all waves; the next tile is loaded into registers while one is used.
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
#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kKlRows = 16;  // query rows per workgroup (MFMA columns)
constexpr int kKlKeys = 32;  // positions per tile
constexpr float kKlLog2e = 1.4426950408889634f;
constexpr float kKlLn2 = 0.6931471805599453f;

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

// LDS layout (dynamic): the K tile (32 keys x Hkv x D bf16), a 1 KB dump
// for the stores of lanes without a chunk, the waves' partial sums
// [W][16 rows][kPStride] fp32 (32 keys, padded), then per-row words.
constexpr int kPStride = kKlKeys + 1;
__host__ __device__ constexpr size_t kl_lds_bytes(int d, int n_heads_kv, int waves) {
  return static_cast<size_t>(kKlKeys) * n_heads_kv * d * 2 + kWave * 16 +
         static_cast<size_t>(waves) * kKlRows * kPStride * 4 + 4 * kKlRows * 4;
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
  extern __shared__ __attribute__((aligned(16))) uint16_t kl_lds[];
  uint16_t* ktile = kl_lds;
  uint16_t* dump = kl_lds + kKlKeys * n_heads_kv * D;
  float* ppart = reinterpret_cast<float*>(dump + kWave * 8);
  int32_t* rowkb = reinterpret_cast<int32_t*>(ppart + W * kKlRows * kPStride);  // key base per row
  int32_t* rowpos = rowkb + kKlRows;                                           // position per row

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
  // ceil(chunks / NT)).  Load indices past the
  // tile are clamped to its last chunk, so the loads carry no branch and
  // stay in flight during the tile's products (a wave's lanes then share
  // one address, one request); their stores go to a per-lane dump slot
  // (a branch there would again make the compiler drain the loads).
  const int chunks = kKlKeys * n_heads_kv * C::PIECES;
  constexpr int kMaxCpt = CPT;

  // Serve the rows one sequence at a time (key bases ascend with the row).
  int32_t seg_kb = rowkb[0];
  while (true) {
    int32_t pmax = -1;
    for (int r = 0; r < n_rows; ++r)
      if (rowkb[r] == seg_kb) pmax = max(pmax, rowpos[r]);
    const bool col_in = my_kb == seg_kb;
    const int ntiles = (pmax + kKlKeys) / kKlKeys;
    const uint16_t* kseq = k + static_cast<int64_t>(seg_kb) * n_heads_kv * D;

    u32x4 pre[kMaxCpt];
    auto load_tile = [&](int t) {
#pragma unroll
      for (int i = 0; i < kMaxCpt; ++i) {
        const int c = min(tid + NT * i, chunks - 1);
        const int key = c / (n_heads_kv * C::PIECES);
        const int s = min(t * kKlKeys + key, pmax);  // past the prefix: any visible row
        const int rest = c % (n_heads_kv * C::PIECES);
        pre[i] = *reinterpret_cast<const u32x4*>(kseq + static_cast<int64_t>(s) * n_heads_kv * D +
                                                 rest * 8);
      }
    };
    auto store_tile = [&]() {
#pragma unroll
      for (int i = 0; i < kMaxCpt; ++i) {
        const int c = tid + NT * i;
        const int cc = min(c, chunks - 1);
        const int key = cc / (n_heads_kv * C::PIECES);
        const int rest = cc % (n_heads_kv * C::PIECES);
        const int at = c < chunks ? kl_at<D>(key, rest / C::PIECES, n_heads_kv, rest % C::PIECES)
                                  : kKlKeys * n_heads_kv * D + lane * 8;
        *reinterpret_cast<u32x4*>(kl_lds + at) = pre[i];
      }
    };
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
    // Logits (log2 domain) of head j for the tile at t: z[sub][r] is key
    // 16 sub + 4 qd + r of this lane's row, -inf when not visible.
    // Raw dot products of head j for the tile: st[sub][r] is key
    // 16 sub + 4 qd + r of this lane's row.
    auto dots = [&](int j, f32x4 (&st)[2]) {
      const int g = (wave * HPW + j) / G;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        st[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const bf16x8 ka = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(
                          ktile + kl_at<D>(16 * sub + col, g, n_heads_kv, 4 * ks + qd)));
          st[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[j][ks], st[sub], 0, 0, 0);
        }
      }
    };
    // Raw dot products of all HPW heads for half sub of the tile (keys
    // 16 sub + 4 qd + r): when the heads share one KV head (G a multiple of
    // HPW) each K fragment is read from LDS once for all of them.
    auto dots_sub = [&](int sub, bool one_g, f32x4 (&st)[HPW]) {
#pragma unroll
      for (int j = 0; j < HPW; ++j) st[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (one_g) {
        const int g = (wave * HPW) / G;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const bf16x8 ka = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(
                          ktile + kl_at<D>(16 * sub + col, g, n_heads_kv, 4 * ks + qd)));
#pragma unroll
          for (int j = 0; j < HPW; ++j)
            st[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[j][ks], st[j], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          const int g = (wave * HPW + j) / G;
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) {
            const bf16x8 ka = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(
                            ktile + kl_at<D>(16 * sub + col, g, n_heads_kv, 4 * ks + qd)));
            st[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[j][ks], st[j], 0, 0, 0);
          }
        }
      }
    };
    const bool one_g = G % HPW == 0;
    // Logits (log2 domain) of head j for the tile at t, -inf when not
    // visible.
    auto logits = [&](int t, int j, float (&z)[2][4]) {
      f32x4 st[2];
      dots(j, st);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = t * kKlKeys + 16 * sub + 4 * qd + r;
          z[sub][r] = col_in && s <= my_pos ? st[sub][r] * scale_log2 : -INFINITY;
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

    // ---- pass 1: per-(row, head) softmax statistics, per-row indexer ones.
    float hm[HPW], hl[HPW];
#pragma unroll
    for (int j = 0; j < HPW; ++j) { hm[j] = -INFINITY; hl[j] = 0.0f; }
    float im[RI], il[RI];
#pragma unroll
    for (int i = 0; i < RI; ++i) { im[i] = -INFINITY; il[i] = 0.0f; }
    // The scores and the K rows of tile t + 1 are loaded while tile t is
    // used, unconditionally (the last tile reloads itself): a branch would
    // make the compiler drain the loads at the first use of any of them.
    float sv_next[RI];
    load_scores(0, sv_next);
    load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
      __syncthreads();  // every wave is done with the previous tile
      store_tile();
      __syncthreads();
      float sv[RI];
#pragma unroll
      for (int i = 0; i < RI; ++i) sv[i] = sv_next[i];
      load_scores(min(t + 1, ntiles - 1), sv_next);
      load_tile(min(t + 1, ntiles - 1));
      if (t < full_tiles) {
        // Each half tile of 16 keys updates the running statistics.
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          f32x4 st[HPW];
          dots_sub(sub, one_g, st);
#pragma unroll
          for (int j = 0; j < HPW; ++j) {
            const float mx = fmaxf(fmaxf(st[j][0], st[j][1]), fmaxf(st[j][2], st[j][3]));
            const float mn = fmaxf(hm[j], mx * scale_log2);
            float sum = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              sum += __builtin_amdgcn_exp2f(__builtin_fmaf(st[j][r], scale_log2, -mn));
            hl[j] = hl[j] * __builtin_amdgcn_exp2f(hm[j] - mn) + sum;
            hm[j] = mn;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          float z[2][4];
          logits(t, j, z);
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
      }
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        if (sv[i] != -INFINITY) {
          const float x = sv[i] * kKlLog2e;
          const float mn = fmaxf(im[i], x);
          il[i] = il[i] * exp2f(im[i] - mn) + exp2f(x - mn);
          im[i] = mn;
        }
      }
    }
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
    load_scores(0, sv_next);
    load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
      __syncthreads();  // tile t-1's reads of K and of the partial sums are done
      store_tile();
      __syncthreads();
      float sv[RI];
#pragma unroll
      for (int i = 0; i < RI; ++i) sv[i] = sv_next[i];
      load_scores(min(t + 1, ntiles - 1), sv_next);
      load_tile(min(t + 1, ntiles - 1));
      float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      if (t < full_tiles) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          f32x4 st[HPW];
          dots_sub(sub, one_g, st);
#pragma unroll
          for (int j = 0; j < HPW; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[sub][r] += __builtin_amdgcn_exp2f(__builtin_fmaf(st[j][r], scale_log2, -hb[j]));
        }
      } else {
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          float z[2][4];
          logits(t, j, z);
#pragma unroll
          for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[sub][r] += __builtin_amdgcn_exp2f(z[sub][r] - hb[j]);
        }
      }
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          ppart[(wave * kKlRows + col) * kPStride + 16 * sub + 4 * qd + r] = acc[sub][r];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        const int r = e_row[i];
        const int s = t * kKlKeys + e_key[i];
        if (sv[i] != -INFINITY) {
          float psum = 0.0f;
#pragma unroll
          for (int w = 0; w < W; ++w) psum += ppart[(w * kKlRows + r) * kPStride + e_key[i]];
          const float P = psum * inv_hq;
          const float lpi = sv[i] - lnorm[i];
          const float pi = __expf(lpi);
          if (P > 0.0f) kl[i] += P * (__logf(P) - lpi);
          if (grad != nullptr) grad[(first + r) * ld_grad + s] = pi - P;
        }
      }
    }
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
    __syncthreads();
  }
}

template <int D, int HPW, int W, int CPT>
hipError_t launch_kl_d(const dsa_varlen& vl, const uint16_t* q, const uint16_t* k,
                       const float* scores, int64_t ld, int64_t row_begin, int64_t row_count,
                       int n_heads_q, int n_heads_kv, float scale, float* loss, float* grad,
                       int64_t ld_grad, hipStream_t stream) {
  const size_t lds = kl_lds_bytes(D, n_heads_kv, W);
  // Up to 64 KB of K tile (8 KV heads at d = 128) plus the partial sums:
  // above the default dynamic LDS limit, within the 160 KB of a CU.  Set
  // once per instantiation (thread-safe static initialisation).
  static const hipError_t lds_ok = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&indexer_kl_kernel<D, HPW, W, CPT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kl_lds_bytes(D, 8, W)));
  if (lds_ok != hipSuccess) return lds_ok;
  const unsigned blocks = static_cast<unsigned>((row_count + kKlRows - 1) / kKlRows);
  hipLaunchKernelGGL((indexer_kl_kernel<D, HPW, W, CPT>), dim3(blocks), dim3(W * kWave), lds, stream,
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
