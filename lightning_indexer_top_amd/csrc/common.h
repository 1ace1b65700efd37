// Shared device helpers of the gfx950 kernels (wave64, MFMA operand vectors,
// orderable keys for selection).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

namespace li {

constexpr int WAVE = 64;

// Cache-policy operand of global_load_lds for data read once per launch: nt
// (non-temporal).  Such lines are inserted for early eviction instead of
// displacing reused ones; on a read-once HBM stream it raised the measured read
// rate of the same access pattern from 6.1 to 6.95-7.1 TB/s.
constexpr int CPOL_STREAM = 2;

// Orderable unsigned images of floating-point values: a > b (as numbers, -0 == +0
// excluded) iff ord(a) > ord(b).  NaNs with the sign bit clear order above +inf.
__device__ __forceinline__ uint32_t ord_f32(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t ord_f64(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  if (u == 0x8000000000000000ull) u = 0;
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ double unord_f64(uint64_t k) {
  uint64_t u = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)u);
}

// bf16 bits -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS):
// shifts by 1, 2, 4, 8 inside each row of 16 lanes, then the last lane of each
// row is added into the rows above it (row_bcast:15, row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] in [15:14]).
#define LI_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
#define LI_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4))

// s_waitcnt vmcnt(n) for a run-time n in [0, 23] (the count is an immediate).
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define LI_CASE(c) \
  case c:          \
    LI_WAIT_VMCNT(c); \
    break;
    LI_CASE(0) LI_CASE(1) LI_CASE(2) LI_CASE(3) LI_CASE(4) LI_CASE(5) LI_CASE(6) LI_CASE(7)
    LI_CASE(8) LI_CASE(9) LI_CASE(10) LI_CASE(11) LI_CASE(12) LI_CASE(13) LI_CASE(14) LI_CASE(15)
    LI_CASE(16) LI_CASE(17) LI_CASE(18) LI_CASE(19) LI_CASE(20) LI_CASE(21) LI_CASE(22)
#undef LI_CASE
    default:
      LI_WAIT_VMCNT(23);
      break;
  }
}

// LDS pointers and their 32-bit LDS addresses (for inline assembly and the
// LDS destination of global_load_lds).
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_u8*)p; }

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads() it
// does not wait for the wave's outstanding global loads, so prefetches issued
// before it stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum over the 64 lanes of a wave (result in every lane).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, WAVE));
  return v;
}

}  // namespace li
