// mfma_peak.hip -- bench-only calibration: the bf16 MFMA throughput the chip
// sustains with every SIMD issuing v_mfma_f32_32x32x16_bf16 back to back
// (no loads, no other work), to set beside the published dense peak.  The
// sustained engine clock under full matrix-core load is below the boost
// clock the published figure assumes.
//
// Each wave keeps four independent accumulators and rotates four operand
// pairs, so that neither a dependency nor constant operands (which switch
// fewer bits) make the loop easier than real work.  Built into its own
// library, apart from the DSA entry points.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__device__ __forceinline__ bf16x8 pattern(uint32_t seed) {
  uint32_t v[4];
  for (int i = 0; i < 4; ++i) {
    seed = seed * 1664525u + 1013904223u;
    // bf16 pairs with exponents near 1.0 and varying mantissas and signs
    v[i] = ((seed & 0x807Fu) | 0x3F00u) | (((seed >> 16) & 0x807Fu) | 0x3F00u) << 16;
  }
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(v));
}

__global__ __launch_bounds__(256) void mfma_loop(int64_t iters, float* out) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8 a[4], b[4];
  for (int i = 0; i < 4; ++i) {
    a[i] = pattern(t * 8 + i);
    b[i] = pattern(t * 8 + 4 + i);
  }
  f32x16 c[4] = {};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(i + j) & 3], b[(i + 2 * j) & 3], c[j], 0, 0, 0);
    }
  }
  float s = 0.0f;
  for (int j = 0; j < 4; ++j)
    for (int v = 0; v < 16; ++v) s += c[j][v];
  out[t] = s;
}

}  // namespace

// Launches `blocks` workgroups of 256 threads running `iters` rounds of 16
// MFMAs per wave; returns the HIP status.  flops = blocks * 4 waves * iters
// * 16 * 32768.  `out` holds blocks * 256 floats.
extern "C" int dsa_calib_mfma_bf16(int64_t iters, int blocks, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(256), 0, stream, iters, out);
  return static_cast<int>(hipGetLastError());
}

namespace {

// Streaming read: every thread reads 16-byte vectors in a grid-stride loop
// (four in flight) and folds them into one word, so only the reads count.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_loop(const u32x4* __restrict__ src, int64_t n,
                                                 uint32_t* out) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  uint32_t acc = 0;
  int64_t i = t;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n; i += stride) {
    const u32x4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  out[t] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from `src` with `blocks` workgroups of 256
// threads; `out` holds blocks * 256 words.
extern "C" int dsa_calib_read(const void* src, int64_t bytes, int blocks, uint32_t* out,
                              hipStream_t stream) {
  hipLaunchKernelGGL(read_loop, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, out);
  return static_cast<int>(hipGetLastError());
}
