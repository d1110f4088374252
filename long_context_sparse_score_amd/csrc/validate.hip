// validate.hip -- device-side checks of the preconditions the entry points do
// not verify on the host: the packed-batch offsets (cu_seqlens) and the
// contents of index lists and score rows.  Opt-in (dsa_check_* calls, or the
// DSA_CHECK environment flag); each check waits for its stream.
#include <mutex>

#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kMaxDevices = 64;
constexpr int kCheckThreads = 256;
// Positions covered by one pass of the duplicate bitmap (32 KiB of LDS).
constexpr int kBitmapWords = 8192;
constexpr int32_t kBitmapSpan = kBitmapWords * 32;

// A finding is packed as (item << 8) | code; the smallest one wins, so the
// report names the first offending sequence or row, whatever the schedule.
__device__ __forceinline__ void report(unsigned long long* rep, int64_t item, int code) {
  atomicMin(rep, (static_cast<unsigned long long>(item) << 8) | static_cast<unsigned>(code));
}

__global__ void check_offsets_kernel(const int32_t* __restrict__ cu_q,
                                     const int32_t* __restrict__ cu_k, int batch,
                                     int64_t total_q, int64_t total_k, int32_t max_q,
                                     int32_t max_k, unsigned long long* rep) {
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < batch; b += gridDim.x * blockDim.x) {
    const int32_t q0 = cu_q[b], q1 = cu_q[b + 1], k0 = cu_k[b], k1 = cu_k[b + 1];
    if (b == 0 && (q0 != 0 || k0 != 0)) report(rep, b, kCheckOffsetStart);
    if (q1 < q0 || k1 < k0) {
      report(rep, b, kCheckOffsetOrder);
    } else {
      if (q1 - q0 > k1 - k0) report(rep, b, kCheckMoreQueriesThanKeys);
      if (q1 - q0 > max_q || k1 - k0 > max_k) report(rep, b, kCheckAboveMax);
    }
    if (b == batch - 1 && (q1 != total_q || k1 != total_k)) report(rep, b, kCheckTotal);
  }
}

// One workgroup per row of the window: every entry is -1 or a position in
// 0..p (unless empty_outside: then any entry outside 0..p is an empty slot,
// as the attention kernels treat it), and no position appears twice.
// Duplicates are found with an LDS bitmap, one span of positions per pass.
__global__ __launch_bounds__(kCheckThreads) void check_indices_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const int32_t* __restrict__ indices, int topk, int64_t row_begin, int empty_outside,
    unsigned long long* rep) {
  __shared__ uint32_t bits[kBitmapWords];
  __shared__ int found;
  const int64_t local = blockIdx.x;
  const RowInfo ri = row_info(cu_q, cu_k, batch, row_begin + local);
  const int32_t* irow = indices + local * topk;
  if (threadIdx.x == 0) found = 0;
  __syncthreads();
  for (int j = threadIdx.x; j < topk; j += kCheckThreads) {
    const int32_t p = irow[j];
    if (!empty_outside && p != -1 && (p < 0 || p > ri.pos)) found = 1;
  }
  __syncthreads();
  if (found) {
    if (threadIdx.x == 0) report(rep, local, kCheckIndexRange);
    return;
  }
  for (int64_t span0 = 0; span0 <= ri.pos; span0 += kBitmapSpan) {
    const int words = static_cast<int>(min<int64_t>(kBitmapWords, (ri.pos - span0) / 32 + 1));
    for (int i = threadIdx.x; i < words; i += kCheckThreads) bits[i] = 0u;
    __syncthreads();
    for (int j = threadIdx.x; j < topk; j += kCheckThreads) {
      if (irow[j] < 0 || irow[j] > ri.pos) continue;  // empty slot (empty_outside only)
      const int64_t p = irow[j] - span0;
      if (p < 0 || p >= kBitmapSpan) continue;
      const uint32_t bit = 1u << (p & 31);
      if (atomicOr(&bits[p >> 5], bit) & bit) found = 1;
    }
    __syncthreads();
    if (found) break;
  }
  if (found && threadIdx.x == 0) report(rep, local, kCheckIndexDuplicate);
}

// One workgroup per row of the window: columns 0..p are finite.
__global__ __launch_bounds__(kCheckThreads) void check_scores_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch,
    const float* __restrict__ scores, int64_t ld, int64_t row_begin, unsigned long long* rep) {
  const int64_t local = blockIdx.x;
  const RowInfo ri = row_info(cu_q, cu_k, batch, row_begin + local);
  const float* srow = scores + local * ld;
  bool bad = false;
  for (int32_t s = threadIdx.x; s <= ri.pos; s += kCheckThreads) bad |= !isfinite(srow[s]);
  if (__any(bad) && lane_id() == 0) report(rep, local, kCheckScoreNotFinite);
}

std::mutex g_report_mutex;
unsigned long long* g_report[kMaxDevices] = {};

// Caller holds g_report_mutex.
hipError_t report_buffer(unsigned long long** rep) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (g_report[dev] == nullptr) {
    e = hipMalloc(reinterpret_cast<void**>(&g_report[dev]), 256);
    if (e != hipSuccess) return e;
  }
  *rep = g_report[dev];
  return hipSuccess;
}

// Clears the report, enqueues `launch`, waits for the stream and reads the
// smallest finding back (~0 when there is none).  One report word serves a
// device, so checks run one at a time: the lock is held until the finding
// has been read back, and checks from several host threads or streams
// queue behind each other instead of mixing their findings.
template <class Launch>
hipError_t run_check(hipStream_t stream, unsigned long long* finding, Launch launch) {
  std::lock_guard<std::mutex> lock(g_report_mutex);
  unsigned long long* rep = nullptr;
  hipError_t e = report_buffer(&rep);
  if (e != hipSuccess) return e;
  if ((e = hipMemsetAsync(rep, 0xff, sizeof *rep, stream)) != hipSuccess) return e;
  launch(rep);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = hipMemcpyAsync(finding, rep, sizeof *rep, hipMemcpyDeviceToHost, stream)) != hipSuccess)
    return e;
  return hipStreamSynchronize(stream);
}

}  // namespace

hipError_t check_offsets(const dsa_varlen& vl, hipStream_t stream, unsigned long long* finding) {
  return run_check(stream, finding, [&](unsigned long long* rep) {
    const int blocks = (vl.batch + kCheckThreads - 1) / kCheckThreads;
    hipLaunchKernelGGL(check_offsets_kernel, dim3(blocks), dim3(kCheckThreads), 0, stream,
                       vl.cu_seqlens_q, vl.cu_seqlens_k, vl.batch, vl.total_q, vl.total_k,
                       vl.max_seqlen_q, vl.max_seqlen_k, rep);
  });
}

hipError_t check_indices(const dsa_varlen& vl, const int32_t* indices, int topk,
                         int64_t row_begin, int64_t row_count, bool empty_outside,
                         hipStream_t stream, unsigned long long* finding) {
  return run_check(stream, finding, [&](unsigned long long* rep) {
    hipLaunchKernelGGL(check_indices_kernel, dim3(static_cast<unsigned>(row_count)),
                       dim3(kCheckThreads), 0, stream, vl.cu_seqlens_q, vl.cu_seqlens_k,
                       vl.batch, indices, topk, row_begin, empty_outside ? 1 : 0, rep);
  });
}

hipError_t check_scores(const dsa_varlen& vl, const float* scores, int64_t ld, int64_t row_begin,
                        int64_t row_count, hipStream_t stream, unsigned long long* finding) {
  return run_check(stream, finding, [&](unsigned long long* rep) {
    hipLaunchKernelGGL(check_scores_kernel, dim3(static_cast<unsigned>(row_count)),
                       dim3(kCheckThreads), 0, stream, vl.cu_seqlens_q, vl.cu_seqlens_k,
                       vl.batch, scores, ld, row_begin, rep);
  });
}

}  // namespace dsa
