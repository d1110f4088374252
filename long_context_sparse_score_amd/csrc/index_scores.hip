// index_scores.hip -- Lightning-Indexer scores on gfx950 MFMA.
//
// I[t, s] = sum_h w[t, h] * max(0, qI[t, h, :] . kI[s, :])  for s = 0..p(t)
// (Keye-VL-2.0 report summary, page 5 section 1: a lightweight scout scores
// every position with one MQA key shared by all of its heads).  The per-row
// MFMA core (heads on the MFMA rows, ReLU / weight / head sum in registers)
// is in index_core.h.
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
//    per-wave path of index_core.h.
//  * index_scores_stream (decode / few rows): each wave streams its own key
//    range of one row through a private LDS ring filled by coalesced
//    buffer->LDS DMA, three 32-key tiles in flight; long rows are split into
//    chunks so that a handful of rows still covers the whole chip.
// Every global load is issued unconditionally (addresses are clamped into
// the sequence instead): a load under a branch makes the compiler wait for
// it on the spot, which would serialise the prefetch.
//
// Both kernels have a candidate mode for the fused indexer -> top-k: instead
// of writing every score, the epilogue keeps the scores at or above the
// row's threshold.  The two tiles of a pair finish their head sums together
// (index_core.h), so each 64-key step ranks its survivors with one ballot.
// The prefill kernel runs its rows whole (one key chunk), so a wave owns its
// row's list and writes each step's survivors straight to it: one
// range-checked 8-byte store per lane and step, the same store count as
// score mode, no branch and no atomics.  The decode kernel splits rows into
// chunks: survivors go to the wave's LDS staging area (one LDS write per
// lane, no branch), and each group of 8 tiles reserves room in the row's
// list with one atomic whose result is used a group later.  In score mode
// both kernels can also score only every key_stride-th key (the fused path's
// sample).
#include <type_traits>

#include "dsa_common.h"
#include "dsa_internal.h"
#include "index_core.h"

namespace dsa {

namespace {

using namespace core;

constexpr int kBlockRows = 8;        // query rows (waves) per prefill workgroup
constexpr int kStageKeys = 256;      // keys per LDS stage (2 stages: 128 KB at d_idx = 128)
constexpr int kStreamRows = 4;       // waves per stream workgroup
constexpr int kStreamGroup = 8;      // stream-kernel tiles per candidate reservation
// One wave's candidate staging: N halves of HALF entries, each followed by
// one dump slot per lane.  With two halves (stream kernel) the survivors of
// the current tile group go to half `cur` while the other half waits for
// its reservation.
template <int HALF, int N>
struct CandStage {
  static constexpr int kSlots = HALF + kWave;
  uint2 e[N][kSlots];
};

// Appends the survivors among 64 consecutive keys (lane l: the score v of
// key pos; a survivor has v >= tau and pos < end) to half `cur` of the
// staging area: survivors rank by ballot, every other lane writes its own
// dump slot -- one LDS write per lane, no branch.  The ballot itself is the
// lane condition (inverse ballot), so the append is two compares, the rank
// and one select.
// RING: the half is a ring (slot = count mod HALF, HALF a power of two) that
// the caller drains as it goes; otherwise slots count up from 0.
template <bool RING = false, int HALF, int N>
__device__ __forceinline__ void cand_append(CandStage<HALF, N>& cs, int cur, uint32_t& fill, float v,
                                            int32_t pos, int32_t end, float tau, int lane) {
  static_assert(!RING || (HALF & (HALF - 1)) == 0, "ring size");
  const unsigned long long m =
      __builtin_amdgcn_ballot_w64(pos < end) & __builtin_amdgcn_ballot_w64(v >= tau);
  const bool ok = __builtin_amdgcn_inverse_ballot_w64(m);
  const uint32_t rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
  const uint32_t at = RING ? (fill + rank) & (HALF - 1) : fill + rank;
  cs.e[cur][ok ? at : HALF + static_cast<uint32_t>(lane)] =
      make_uint2(__float_as_uint(v), static_cast<uint32_t>(pos));
  fill += static_cast<uint32_t>(__popcll(m));
}

// Copies n staged entries of half h to the row's list at `base` (entries
// past the list's capacity are dropped; the count records them).
template <int HALF, int N>
__device__ __forceinline__ void cand_copy(const CandStage<HALF, N>& cs, int h, uint32_t n,
                                          uint32_t base, uint2* __restrict__ list, int cap,
                                          int lane) {
  for (uint32_t i = lane; i < n; i += kWave)
    if (base + i < static_cast<uint32_t>(cap)) list[base + i] = cs.e[h][i];
}

// Reserves n entries of the row's list (returns the old count; lane 0 only).
__device__ __forceinline__ uint32_t cand_reserve(uint32_t* count, uint32_t n, int lane) {
  uint32_t base = 0;
  if (lane == 0 && n != 0) base = atomicAdd(count, n);
  return base;
}

// ---------------------------------------------------------------- prefill kernel

// LDS key stage B of a prefill workgroup (ELEMS bf16).  Each stage buffer is
// a variable of its own, so the compiler can tell the buffer a DMA is
// filling from the one being read, and places no wait for the copy in
// flight before reads of the other.
template <int ELEMS, int B>
__device__ __forceinline__ uint16_t* stage_buf() {
  __shared__ __attribute__((aligned(16))) uint16_t buf[ELEMS];
  return buf;
}

// SK keys per LDS stage; CAND selects the candidate mode (no score rows).
// Candidate mode runs with one key chunk (gridDim.y == 1): each wave then
// owns its row's list and counter, so no atomics are needed.  The 8 waves'
// staging areas (SK entries plus 64 dump slots each, 20 KB at SK = 256, beside
// the 128 KB of key stages at d_idx = 128) serve only workgroups whose rows
// span several sequences.
template <int D, int MT, int SK, bool CAND>
__global__ __launch_bounds__(kBlockRows * kWave, 2) void index_scores_block(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const uint16_t* __restrict__ q_idx, const uint16_t* k_idx,
    const float* __restrict__ w, int n_heads, int64_t row_begin, int64_t row_count,
    IndexOut o, int key_chunk) {
  constexpr int KS = D / 16;
  constexpr int CHUNKS = D / 8;                                     // 16-byte chunks per key row
  constexpr int DMA_PER_WAVE = SK * CHUNKS / (kBlockRows * kWave);
  constexpr int TILES = SK / 32;                                    // 32-key MFMA tiles per stage
  static_assert(TILES % 2 == 0 && DMA_PER_WAVE * kBlockRows * kWave == SK * CHUNKS, "stage shape");
  __shared__ CandStage<CAND ? SK : 1, 1> cstage[CAND ? kBlockRows : 1];
  static_assert(!CAND || TILES * 32 <= SK, "a stage's survivors fit one half");

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
  const int stride = o.key_stride;

  const RowInfo ri = row_info(cu_q, cu_k, batch, row);
  const RowInfo r_first = row_info(cu_q, cu_k, batch, row_begin + first);
  const RowInfo r_last = row_info(cu_q, cu_k, batch, row_begin + last);
  const int32_t c0 = blockIdx.y * key_chunk;
  const int32_t nv = visible_keys(ri.pos, stride);

  RowState<D, MT> st;
  load_row_state<D, MT>(st, q_idx, w, row, n_heads, col, half);
  float* out_row = CAND ? nullptr : o.scores + local * o.ld;
  const float tau = CAND && active ? o.tau[local] : 0.0f;
  uint2* list = CAND ? o.cand + local * o.cap : nullptr;
  uint32_t* counter = CAND ? o.count + local : nullptr;

  if (r_first.key_base != r_last.key_base) {
    // Rows of several sequences: every wave walks its own keys.
    const int32_t c1 = min(c0 + key_chunk, nv);
    if (!active || c0 >= c1) return;
    if constexpr (CAND) {
      // One staging half, copied to the row's list whenever a further 64
      // survivors might not fit.
      CandStage<SK, 1>& cs = cstage[wave];
      uint32_t fill = 0, written = 0;
      auto flush = [&]() {
        cand_copy(cs, 0, fill, written, list, o.cap, lane);
        written += fill;
        fill = 0;
      };
      row_direct<D, MT>(st, k_idx, ri, stride, c0, c1, col, half,
                        [&](float v, int32_t pos) {
                          cand_append(cs, 0, fill, v, pos, c1, tau, lane);
                        },
                        [&]() {
                          if (fill > static_cast<uint32_t>(SK - 64)) flush();
                        });
      flush();
      if (lane == 0) *counter = written;
    } else {
      row_direct<D, MT>(st, k_idx, ri, stride, c0, c1, col, half,
                        [&](float v, int32_t pos) {
                          if (pos < c1) out_row[pos] = v;
                        },
                        []() {});
    }
    return;
  }

  // All rows share one sequence; positions grow with the row.
  const int32_t c_end = min(c0 + key_chunk, visible_keys(r_last.pos, stride));
  if (c0 >= c_end) return;
  // Scores of keys my_end and beyond (and every score of an inactive wave)
  // fall outside the store resource and are dropped (candidate mode: fail
  // the admission test).
  const int32_t my_end = active ? min(c0 + key_chunk, nv) : c0;
  const uint16_t* kseq = k_idx + r_first.key_base * D;
  const __amdgpu_buffer_rsrc_t keys = raw_buffer(kseq, (r_last.pos + 1) * D * 2);
  const __amdgpu_buffer_rsrc_t outs = raw_buffer(out_row, CAND ? 0 : my_end * 4);

  // Stage fill by buffer->LDS DMA: DMA instruction i of a wave writes 64
  // consecutive 16-byte LDS chunks; LDS chunk (key, s) receives global chunk
  // s ^ (key & (CHUNKS - 1)), so the B-fragment reads below are conflict free.
  // Instruction i covers keys KPI i + (key of instruction 0); the XOR term
  // repeats with period CHUNKS in the key and KPI is a multiple of it, so all
  // instructions share one per-lane offset and differ by a scalar one.
  constexpr int KPI = kBlockRows * kWave / CHUNKS;  // keys per DMA instruction of the workgroup
  static_assert(KPI % CHUNKS == 0, "the swizzle must repeat across DMA instructions");
  const int key0 = (wave * kWave + lane) / CHUNKS, s0 = lane % CHUNKS;
  const int key_bytes = stride * D * 2;  // distance between consecutive keys of this launch
  const int dma_off = key0 * key_bytes + (s0 ^ (key0 & (CHUNKS - 1))) * 16;
  auto fill_stage = [&](uint16_t* dst, int32_t t) {
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          keys, (__attribute__((address_space(3))) void*)(&dst[(i * kBlockRows + wave) * kWave * 8]),
          16, dma_off, (t + i * KPI) * key_bytes, 0, 0);
    }
  };
  // Candidate mode launches one key chunk, so the wave owns its row's list
  // and its count: each 64-key step stores its survivors straight to the
  // list, ranked by ballot, with one range-checked 8-byte store per lane
  // (lanes without a survivor, and entries past the list's capacity, get
  // an offset outside the buffer and store nothing).  That is one store per
  // 64 keys, as in score mode.
  uint32_t fill = 0;
  const __amdgpu_buffer_rsrc_t lrs = raw_buffer(list, CAND ? o.cap * 8 : 0);
  // The scores of 64 consecutive keys, key pos at this lane.
  auto emit = [&](float v, int32_t pos) {
    if constexpr (CAND) {
      const unsigned long long m =
          __builtin_amdgcn_ballot_w64(pos < my_end) & __builtin_amdgcn_ballot_w64(v >= tau);
      const uint32_t at = __builtin_amdgcn_mbcnt_hi(
          static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), fill));
      const u32x2 ev = {__float_as_uint(v), static_cast<uint32_t>(pos)};
      __builtin_amdgcn_raw_buffer_store_b64(
          ev, lrs, __builtin_amdgcn_inverse_ballot_w64(m) ? at * 8u : 0x7FFFFFF0u, 0, 0);
      fill += static_cast<uint32_t>(__popcll(m));
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), outs, pos * 4, 0, 0);
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  fill_stage(stage_buf<SK * D, 0>(), c0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  // Tile j's MFMAs run while tile j-1's epilogue executes on the VALU; each
  // B fragment register is refilled from LDS for tile j+1 as soon as tile
  // j's MFMAs have consumed it.  Tiles pair up (0, 1), (2, 3), ...: the
  // partial head sums of a pair's first tile are held until its second
  // tile's are ready, and one swap finishes both tiles' 64 scores.
  f32x16 acc_even[MT], acc_odd[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc_odd[mt] = f32x16{};
  int32_t prev_pos = 1 << 28;  // key 0 of the previous tile (the first has none)
  int32_t pair_pos = 1 << 28;  // key 0 of the pending pair (the first emit is dropped)
  float held = 0.0f;           // partials of the pending pair's first tile
  // One stage: keys [t0, t0 + SK) from stage buffer B, the next stage's DMA
  // into the other buffer.
  auto stage = [&](auto bsel, int32_t t0) __attribute__((always_inline)) {
    constexpr int B = decltype(bsel)::value;
    if (t0 + SK < c_end) fill_stage(stage_buf<SK * D, 1 - B>(), t0 + SK);
    // The buffer's address is rebuilt every stage (a zero the compiler cannot
    // see through): held across the loop, both buffers' per-lane read
    // addresses would cost eight more registers.
    int32_t zero = 0;
    asm volatile("" : "+s"(zero));
    const uint16_t* tb = stage_buf<SK * D, B>() + zero;
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
      const float part = tile_partial<D, MT>(st, prev);
      if (tj & 1) {  // tile tj - 1 opens a pair
        held = part;
        pair_pos = prev_pos;
      } else {       // tile tj - 1 closes one
        emit(pair_scores(held, part), pair_pos + lane);
      }
      prev_pos = t0 + tj * 32;
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
    // Wait for the next stage's DMA only: the stage's TILES / 2 score (or
    // candidate) stores issued after it may stay in flight.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(TILES / 2));
    lds_barrier();
  };
  for (int32_t t0 = c0; t0 < c_end; t0 += 2 * SK) {
    stage(B0{}, t0);
    if (t0 + SK < c_end) stage(B1{}, t0 + SK);
  }
  // The last stage's last tile (odd) closes the last pair.
  emit(pair_scores(held, tile_partial<D, MT>(st, acc_odd)), pair_pos + lane);
  if constexpr (CAND) {
    if (active && lane == 0) *counter = fill;  // above cap: entries were dropped
  }
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

template <int D, int MT, bool CAND>
__global__ __launch_bounds__(kStreamRows * kWave) void index_scores_stream(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx,
    const float* __restrict__ w, int n_heads, int64_t row_begin, int64_t row_count,
    IndexOut o, int key_chunk, int chunks_per_row) {
  constexpr int KS = D / 16;
  constexpr int CHUNKS = D / 8;
  constexpr int DMA_PER_TILE = 32 * CHUNKS / kWave;   // 16-byte DMA instructions per tile
  constexpr int GROUP_KEYS = kStreamGroup * 32;       // keys per candidate reservation
  static_assert(DMA_PER_TILE * kWave == 32 * CHUNKS, "tile shape");
  static_assert(kRing == 4, "the tile loop below is unrolled by the ring depth");
  __shared__ CandStage<CAND ? GROUP_KEYS : 1, 2> cstage[CAND ? kStreamRows : 1];
  static_assert(kStreamGroup % 2 == 0, "groups of whole tile pairs");
  static_assert(!CAND || kStreamGroup * 32 <= GROUP_KEYS, "a group's survivors fit one half");

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kStreamRows + wave;
  const int64_t local = item / chunks_per_row;
  if (local >= row_count) return;
  const int64_t row = row_begin + local;
  const int stride = o.key_stride;
  const RowInfo ri = row_info(cu_q, cu_k, batch, row);
  const int32_t c0 = static_cast<int32_t>(item % chunks_per_row) * key_chunk;
  const int32_t c1 = min(c0 + key_chunk, visible_keys(ri.pos, stride));
  if (c0 >= c1) return;
  const float tau = CAND ? o.tau[local] : 0.0f;
  RowState<D, MT> st;
  load_row_state<D, MT>(st, q_idx, w, row, n_heads, col, half);

  // Keys [c0, c1) only (DMA past c1 reads zeros without touching memory);
  // scores past c1 are dropped.  Key j of this launch is position j * stride.
  const int key_bytes = stride * D * 2;
  const __amdgpu_buffer_rsrc_t keys =
      raw_buffer(k_idx + (ri.key_base + static_cast<int64_t>(c0) * stride) * D,
                 ((c1 - c0 - 1) * stride + 1) * D * 2);
  const __amdgpu_buffer_rsrc_t outs = raw_buffer(CAND ? nullptr : o.scores + local * o.ld, CAND ? 0 : c1 * 4);
  // Ring slot B of this wave.  Each slot is an LDS variable of its own and
  // is picked at compile time, so the compiler sees that reading one slot
  // does not wait for the DMA into another.
  auto slot_buf = [&](auto bsel) -> uint16_t* {
    return stage_buf<kStreamRows * 32 * D, decltype(bsel)::value>() + wave * (32 * D);
  };
  auto fill = [&](auto bsel, int32_t t) {  // tile of keys c0 + t .. c0 + t + 31
    uint16_t* dst = slot_buf(bsel);
#pragma unroll
    for (int i = 0; i < DMA_PER_TILE; ++i) {
      const int e = i * kWave + lane;
      const int key = e / CHUNKS, s = e % CHUNKS;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          keys, (__attribute__((address_space(3))) void*)(dst + i * kWave * 8), 16,
          key * key_bytes + (s ^ (key & (CHUNKS - 1))) * 16, t * key_bytes, 0, 0);
    }
  };
  // Candidate staging (cand_append): groups of kStreamGroup tiles.
  CandStage<CAND ? GROUP_KEYS : 1, 2>& cs = cstage[CAND ? wave : 0];
  uint2* list = CAND ? o.cand + local * o.cap : nullptr;
  uint32_t* counter = CAND ? o.count + local : nullptr;
  int cur = 0;
  uint32_t cfill = 0, pend = 0, pend_base = 0;
  // The scores of 64 consecutive keys, key pos at this lane.
  auto emit = [&](float v, int32_t pos) {
    if constexpr (CAND) {
      cand_append(cs, cur, cfill, v, pos, c1, tau, lane);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), outs, pos * 4, 0, 0);
    }
  };
  auto group_end = [&]() {
    if constexpr (CAND) {
      if (pend != 0u)
        cand_copy(cs, cur ^ 1, pend, __builtin_amdgcn_readfirstlane(pend_base), list, o.cap, lane);
      pend_base = cand_reserve(counter, cfill, lane);
      pend = cfill;
      cfill = 0;
      cur ^= 1;
    }
  };
  // Vector-memory operations that trail each tile's DMA: one store (score
  // mode: the closing tile of a pair stores the pair's 64 scores, the
  // opening tile a dropped store) or none (candidate mode; its reservations
  // and copies only add operations, which makes the waits below stricter,
  // never weaker).
  constexpr int TRAIL = CAND ? 0 : 1;

  // Prologue: tiles 0 .. kRing-2, each followed by a dropped store (score
  // mode) so that every tile's DMA is trailed by the same count of memory
  // operations as in the loop.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  auto prologue = [&](auto bsel) {
    fill(bsel, decltype(bsel)::value * 32);
    if constexpr (!CAND) __builtin_amdgcn_raw_buffer_store_b32(0, outs, 0x7FFFFFF0, 0, 0);
  };
  prologue(S0{});
  prologue(S1{});
  prologue(S2{});
  f32x16 acc[MT], prev[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) prev[mt] = f32x16{};
  // Tiles pair up (0, 1), (2, 3), ... as in the prefill kernel.
  int32_t prev_pos = 1 << 28;  // key 0 of the previous tile (the first has none)
  int32_t pair_pos = 1 << 28;  // key 0 of the pending pair (the first emit is dropped)
  float held = 0.0f;
  // Wave-uniform, so the loop exits below are scalar branches.
  const int ntiles = __builtin_amdgcn_readfirstlane((c1 - c0 + 31) / 32);
  // Tile j sits in slot j % kRing; the step for tile j refills slot
  // (j - 1) % kRing, read by the step before, with tile j + kRing - 1.
  auto step = [&](auto bsel, int j) {
    constexpr int B = decltype(bsel)::value;
    fill(std::integral_constant<int, (B + kRing - 1) % kRing>{}, (j + kRing - 1) * 32);
    // Tile j has landed once at most the kRing - 1 younger tiles' DMAs and
    // their trailing stores are outstanding.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kRing - 1) * (DMA_PER_TILE + TRAIL)));
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint16_t* tb = slot_buf(bsel);
    bf16x8 b[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int slot = (half * KS + ks) ^ (col & (CHUNKS - 1));
      b[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&tb[col * D + slot * 8]));
    }
    tile_mfma<D, MT>(st, b, acc);
    const float part = tile_partial<D, MT>(st, prev);
    if constexpr (B & 1) {  // tile j - 1 opens a pair
      held = part;
      pair_pos = prev_pos;
      if constexpr (!CAND) __builtin_amdgcn_raw_buffer_store_b32(0, outs, 0x7FFFFFF0, 0, 0);
    } else {                // tile j - 1 closes one
      emit(pair_scores(held, part), pair_pos + lane);
      // A group's worth of tiles emitted (the epilogue lags one tile).
      if (CAND && j % kStreamGroup == 0 && j > 0) group_end();
    }
    prev_pos = c0 + j * 32;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) prev[mt] = acc[mt];
    // The slot refilled by the next step was read above: those reads must be
    // done before its DMA is issued.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  };
  // Whole groups of kRing tiles, then the 0 .. kRing - 1 left: the loop has
  // one exit, so its only way back to slot 0 is through slot 3 (the
  // compiler's waits follow every control path).
  int j = 0;
  for (; j + kRing <= ntiles; j += kRing) {
    step(S0{}, j);
    step(S1{}, j + 1);
    step(S2{}, j + 2);
    step(S3{}, j + 3);
  }
  if (j < ntiles) step(S0{}, j);
  if (j + 1 < ntiles) step(S1{}, j + 1);
  if (j + 2 < ntiles) step(S2{}, j + 2);
  // The last tile closes a pair (ntiles even) or opens one (ntiles odd,
  // closed by an empty tile past c1).
  {
    const float part = tile_partial<D, MT>(st, prev);
    if (ntiles & 1) {
      emit(pair_scores(part, 0.0f), prev_pos + lane);
    } else {
      emit(pair_scores(held, part), pair_pos + lane);
    }
  }
  if constexpr (CAND) {
    group_end();
    if (pend != 0u)
      cand_copy(cs, cur ^ 1, pend, __builtin_amdgcn_readfirstlane(pend_base), list, o.cap, lane);
  }
  // No DMA may still be writing this wave's ring when the wave ends.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

template <int D, int MT, bool CAND>
hipError_t launch_dm(const dsa_varlen& vl, const uint16_t* q_idx, const uint16_t* k_idx,
                     const float* w, int n_heads, int64_t row_begin, int64_t row_count,
                     const IndexOut& o, hipStream_t stream) {
  // Keys of the longest row in this launch's units.
  const int64_t max_keys = (vl.max_seqlen_k - 1) / o.key_stride + 1;
  if (vl.max_seqlen_q >= kBlockRows) {
    // Prefill-like: whole rows per workgroup unless there are too few
    // workgroups to fill the chip, then split the keys.
    constexpr int SK = kStageKeys;
    const int64_t blocks = (row_count + kBlockRows - 1) / kBlockRows;
    int64_t chunk = max_keys;
    // Candidate mode runs one chunk (a wave owns its row); so does a sampled
    // pass (key_stride > 1), whose rows are short.
    if (blocks < 1024 && !CAND && o.key_stride == 1) {
      const int64_t parts = (1024 + blocks - 1) / blocks;
      chunk = (max_keys + parts - 1) / parts;
    }
    chunk = ((chunk + SK - 1) / SK) * SK;
    if (chunk < 2 * SK) chunk = 2 * SK;
    const int64_t chunks = (max_keys + chunk - 1) / chunk;
    hipLaunchKernelGGL((index_scores_block<D, MT, SK, CAND>), dim3(static_cast<unsigned>(blocks),
                       static_cast<unsigned>(chunks)), dim3(kBlockRows * kWave), 0, stream,
                       vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, q_idx, k_idx, w, n_heads,
                       row_begin, row_count, o, static_cast<int>(chunk));
  } else {
    // Decode-like: one wave per (row, key chunk), about 2048 work items (two
    // rounds of one 4-wave workgroup per CU; measured best among 2048-8192).
    const int64_t per_row = (2048 + row_count - 1) / row_count;
    int64_t chunk = (max_keys + per_row - 1) / per_row;
    chunk = ((chunk + 31) / 32) * 32;
    if (chunk < 512) chunk = 512;
    const int64_t chunks_per_row = (max_keys + chunk - 1) / chunk;
    const int64_t items = row_count * chunks_per_row;
    hipLaunchKernelGGL((index_scores_stream<D, MT, CAND>),
                       dim3(static_cast<unsigned>((items + kStreamRows - 1) / kStreamRows)),
                       dim3(kStreamRows * kWave), 0, stream, vl.cu_seqlens_q, vl.cu_seqlens_k,
                       vl.batch, q_idx, k_idx, w, n_heads, row_begin, row_count, o,
                       static_cast<int>(chunk), static_cast<int>(chunks_per_row));
  }
  return hipGetLastError();
}

template <int D, bool CAND>
hipError_t launch_d(const dsa_varlen& vl, const uint16_t* q_idx, const uint16_t* k_idx,
                    const float* w, int n_heads, int64_t row_begin, int64_t row_count,
                    const IndexOut& o, hipStream_t stream) {
  if (n_heads > 32)
    return launch_dm<D, 2, CAND>(vl, q_idx, k_idx, w, n_heads, row_begin, row_count, o, stream);
  return launch_dm<D, 1, CAND>(vl, q_idx, k_idx, w, n_heads, row_begin, row_count, o, stream);
}

}  // namespace

hipError_t launch_index_scores_to(const dsa_varlen& vl, const uint16_t* q_idx,
                                  const uint16_t* k_idx, const float* w, int n_heads, int d,
                                  int64_t row_begin, int64_t row_count, const IndexOut& out,
                                  bool candidates, hipStream_t stream) {
  if (candidates) {
    if (d == 128)
      return launch_d<128, true>(vl, q_idx, k_idx, w, n_heads, row_begin, row_count, out, stream);
    return launch_d<64, true>(vl, q_idx, k_idx, w, n_heads, row_begin, row_count, out, stream);
  }
  if (d == 128)
    return launch_d<128, false>(vl, q_idx, k_idx, w, n_heads, row_begin, row_count, out, stream);
  return launch_d<64, false>(vl, q_idx, k_idx, w, n_heads, row_begin, row_count, out, stream);
}

hipError_t launch_index_scores(const dsa_varlen& vl, const uint16_t* q_idx, const uint16_t* k_idx,
                               const float* w, int n_heads, int d, int64_t row_begin,
                               int64_t row_count, float* scores, int64_t ld, hipStream_t stream) {
  IndexOut o;
  o.scores = scores;
  o.ld = ld;
  return launch_index_scores_to(vl, q_idx, k_idx, w, n_heads, d, row_begin, row_count, o, false,
                                stream);
}

}  // namespace dsa
