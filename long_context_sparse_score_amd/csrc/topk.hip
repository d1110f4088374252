// topk.hip -- deterministic per-row top-k of indexer scores.
//
// For each query row keep the n = min(k, p + 1) positions with the largest
// score, ties towards the lower position, and write them in ascending
// position order padded with -1 (Keye-VL-2.0 report summary, page 5: section
// 1 keeps the k = 2048 best positions per query token; section 8 needs the
// selection to be deterministic so training and inference agree).
//
// One workgroup owns one row and reads it from HBM once, in position order,
// with three steps of loads in flight.  Two configurations: windows of many
// rows use 256 threads, steps of 1024 scores and ~37 KB of LDS, so four rows
// share a CU and hide each other's latencies; few long rows (decode) use 512
// threads, steps of 4096 scores and a candidate buffer twice as large, so one
// row alone keeps 48 KB in flight.
//
// A score survives only if it beats the running threshold, which for finite
// scores is one float compare against the smallest float whose
// order-preserving key is above it.  Survivors (raw bits and position) are
// appended to a candidate buffer in LDS: each wave to its own segment, slots
// by ballot and mbcnt, lanes without a survivor writing to a dump slot, so
// the append has no divergent branch and an element group without survivors
// costs one compare and one scalar test.  Long rows start from a threshold
// read off a spread sample of the row, at the rank where a set multiple of k
// scores of the whole row are expected above it, so the buffer is rarely
// cut before the end.  The estimate only decides speed: if fewer than k
// scores beat it, the row is streamed again from threshold zero, so the
// result is exact for any input.  When the buffer could overflow on the
// next step it is cut to exactly k entries by a radix select whose digits
// are taken relative to the range of the candidates' keys (min..max): the
// bins spread over the values actually present, so atomics rarely collide
// and each level shrinks the range by the bin count.  Ties at the k-th key
// are cut by a second select on the position.  The new threshold is the
// k-th key: the stream resumes right after the step that called for the
// cut, so later scores equal to it sit at higher positions and can never
// displace the kept ties, and the test stays a strict "greater than".  At
// the end the kept positions are marked in an LDS bitmask and written in
// ascending order by a prefix count over its words (a bitonic sort serves
// rows too long for the bitmask).  Every decision depends only on key and
// position values, never on the order in which lanes appended, so the
// output is bitwise repeatable.
//
// The select itself (topk_core.h) also serves the fused indexer -> top-k
// (index_topk.hip): its exact fallback streams a recomputed score row, and
// its candidate select reuses the radix select.
#include "dsa_common.h"
#include "dsa_internal.h"
#include "topk_core.h"

namespace dsa {

namespace {

using namespace topk;

// One workgroup per row: the whole row streamed once, k positions out.
template <class Impl>
__global__ __launch_bounds__(Impl::kThreads) void topk_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const float* __restrict__ scores, int64_t ld, int64_t row_begin, int64_t row_count, int k,
    int32_t* __restrict__ indices) {
  __shared__ typename Impl::Shared sh;
  const int tid = threadIdx.x;
  // Later rows are longer: hand them out first.
  const int64_t local = row_count - 1 - static_cast<int64_t>(blockIdx.x);
  const RowInfo ri = row_info(cu_q, cu_k, batch, row_begin + local);
  const int32_t n = ri.pos + 1;
  int32_t* orow = indices + local * k;
  if (n <= k) {
    for (int j = tid; j < k; j += Impl::kThreads) orow[j] = j < n ? j : -1;
    return;
  }
  typename Impl::FillT fl;
  Impl::select_row(sh, ScoreSource{scores + local * ld, n, 0}, n, k, fl);
  Impl::emit_sorted(sh, fl, k, n, orow);
  // Fewer than k held only for non-finite input: pad like a short row.
  for (int j = static_cast<int>(fl.total()) + tid; j < k; j += Impl::kThreads) orow[j] = -1;
}

template <class Impl>
hipError_t launch_rows(const dsa_varlen& vl, const float* scores, int64_t ld, int64_t row_begin,
                       int64_t row_count, int k, int32_t* indices, hipStream_t stream) {
  hipLaunchKernelGGL((topk_kernel<Impl>), dim3(static_cast<unsigned>(row_count)),
                     dim3(Impl::kThreads), 0, stream, vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch,
                     scores, ld, row_begin, row_count, k, indices);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const dsa_varlen& vl, const float* scores, int64_t ld, int64_t row_begin,
                       int64_t row_count, int k, int32_t* indices, hipStream_t stream) {
  // With fewer rows than two per CU, rows cannot hide each other's
  // latencies: give each row the wide configuration, with a denser sample
  // (4096 scores) so that a start threshold aimed at 1.5 k survivors
  // almost never leaves fewer than k (a restart doubles that row's time,
  // and the launch waits for its slowest row).
  if (row_count < 512)
    return launch_rows<TopkImpl<2, 8192, 512, 1024, 3, 2>>(vl, scores, ld, row_begin, row_count,
                                                           k, indices, stream);
  // Many rows: steps of 1024 scores, four rows per CU; a 2048-score sample
  // aimed at 1.5 k survivors (a rare restart costs only its own row here);
  // 9-bit radix digits (a 512-bin histogram was 1-4% faster per window than
  // 1024 bins on the 128K prefill).
  return launch_rows<TopkImpl<1, 4096, 256, 512, 3, 2>>(vl, scores, ld, row_begin, row_count, k,
                                                        indices, stream);
}

}  // namespace dsa
