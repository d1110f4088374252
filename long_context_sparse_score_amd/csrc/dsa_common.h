// dsa_common.h -- device-side helpers shared by the DSA kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Operand and accumulator types of the gfx950 bf16 MFMA instructions.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
// Native 16-byte vector (HIP's uint4 is a union-based struct that register
// promotion of local arrays does not always see through).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// 16 bytes (8 bf16) from global memory as an MFMA operand.
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, u);
}

// Raw buffer resource over [base, base + bytes) (gfx9-family word 3): loads
// past the end return zero and stores past it are dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           0x00020000);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  uint4 u = make_uint4(0u, 0u, 0u, 0u);
  return __builtin_bit_cast(bf16x8, u);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// s_waitcnt immediate: vmcnt(n), expcnt and lgkmcnt left unconstrained.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// Workgroup barrier for LDS hand-off.  The waits it needs are explicit
// (s_waitcnt before it); the wavefront-scope fences only keep the compiler
// from moving LDS accesses across it, without the vmcnt(0) a workgroup
// fence would add (that would also wait for outstanding global stores).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sequence owning packed query row `row` (cu_q non-decreasing, cu_q[0] == 0).
__device__ __forceinline__ int find_sequence(const int32_t* __restrict__ cu_q, int batch,
                                             int64_t row) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (static_cast<int64_t>(cu_q[mid]) <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Position and key offset of a packed query row inside its sequence.
struct RowInfo {
  int64_t key_base;  // packed index of local key 0
  int32_t pos;       // causal position p (keys 0..p visible)
  int32_t seq_len_k;
};

__device__ __forceinline__ RowInfo row_info(const int32_t* __restrict__ cu_q,
                                            const int32_t* __restrict__ cu_k, int batch,
                                            int64_t row) {
  int b = find_sequence(cu_q, batch, row);
  int32_t q0 = cu_q[b], q1 = cu_q[b + 1], k0 = cu_k[b], k1 = cu_k[b + 1];
  RowInfo r;
  r.key_base = k0;
  r.seq_len_k = k1 - k0;
  r.pos = (k1 - k0) - (q1 - q0) + static_cast<int32_t>(row - q0);
  return r;
}

}  // namespace dsa
