// Roofline probes for gfx950 (liblightning_indexer_probe.so): the measured
// ceilings reported beside the datasheet peaks.  Not part of the indexer path.
//
//   li_probe_read  -- a read-only HBM stream: every byte of a device buffer is read
//                     once with 16-byte loads, the sum of the words folded into one
//                     value per workgroup (so nothing is dead code); no stores in
//                     the stream.
//   li_probe_mfma_bf16 -- a register-resident loop of v_mfma_f32_32x32x16_bf16:
//                     four independent accumulator chains per wave, operands held
//                     in VGPRs, either constant bits or pseudo-random normal-range
//                     bf16 values (the chip's clock falls with operand bit
//                     activity, so both are measured).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/li_probe.h"

typedef __bf16 pbf16x8 __attribute__((ext_vector_type(8)));
typedef float pf32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int RD_THREADS = 256;
constexpr int RD_UNROLL = 8;  // 16-byte loads in flight per thread per step

__global__ __launch_bounds__(RD_THREADS) void probe_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                                uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * RD_THREADS;
  int64_t i = (int64_t)blockIdx.x * RD_THREADS + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (RD_UNROLL - 1) * stride < n16; i += RD_UNROLL * stride) {
    uint4 v[RD_UNROLL];
#pragma unroll
    for (int u = 0; u < RD_UNROLL; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < RD_UNROLL; ++u) acc += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc += v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[RD_THREADS / 64];
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int wv = 0; wv < RD_THREADS / 64; ++wv) s += red[wv];
    sink[blockIdx.x] = s;
  }
}

__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// bf16 bit pattern of a normal-range value in [-4, 4): random sign, exponent in
// [2^-4, 2^2), random mantissa
__device__ __forceinline__ uint16_t rnd_bf16(uint32_t h) {
  const uint32_t sign = (h >> 31) << 15;
  const uint32_t ex = 123u + ((h >> 7) % 6u);
  return (uint16_t)(sign | (ex << 7) | (h & 0x7Fu));
}

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, int random, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const uint32_t seed = (uint32_t)(blockIdx.x * 256 + threadIdx.x) * 2654435761u;
  pbf16x8 a[2], b[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    uint16_t va[8], vb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      va[e] = random ? rnd_bf16(hash32(seed + 16u * r + e)) : (uint16_t)0x3F80;
      vb[e] = random ? rnd_bf16(hash32(seed ^ (0x9e3779b9u + 16u * r + e))) : (uint16_t)0x3F80;
    }
    a[r] = __builtin_bit_cast(pbf16x8, *(const uint4*)va);
    b[r] = __builtin_bit_cast(pbf16x8, *(const uint4*)vb);
  }
  pf32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[0], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[1], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], c3, 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

int cus() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 256;
  return v;
}

}  // namespace

extern "C" {

int li_probe_read_blocks(void) { return cus() * 8; }

int li_probe_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || ((uintptr_t)buf & 15u) || (bytes & 15u)) return 1;
  probe_read_kernel<<<li_probe_read_blocks(), RD_THREADS, 0, stream>>>((const uint4*)buf, (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int li_probe_mfma_blocks(void) { return cus() * 2; }

double li_probe_mfma_flop(int iters) {
  // 16 MFMAs of 32 x 32 x 16 per iteration per wave, 4 waves per workgroup
  return (double)li_probe_mfma_blocks() * 4.0 * iters * 16.0 * (32.0 * 32.0 * 16.0 * 2.0);
}

int li_probe_mfma_bf16(int iters, int random, float* sink, hipStream_t stream) {
  if (!sink || iters < 1) return 1;
  probe_mfma_kernel<<<li_probe_mfma_blocks(), 256, 0, stream>>>(iters, random, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
