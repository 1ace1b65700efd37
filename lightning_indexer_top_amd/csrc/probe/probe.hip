// Roofline probes for gfx950 (liblightning_indexer_probe.so): the measured
// ceilings reported beside the datasheet peaks.  Not part of the indexer path.
//
//   li_probe_read  -- a read-only HBM stream: every byte of a device buffer is read
//                     once with 16-byte loads (no stores in the stream but one word
//                     per workgroup), in one of five access patterns: grid-stride
//                     register loads, a contiguous range per wave into registers,
//                     a contiguous range per wave by DMA into LDS, the same with
//                     the non-temporal cache policy, or the decode scoring kernel's
//                     own pattern (a contiguous range per workgroup whose four waves
//                     take 4 KB tiles in turn, three in flight per wave, DMA into
//                     LDS, non-temporal).
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

__device__ __forceinline__ uint32_t fold(const uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__device__ __forceinline__ void sink_block(uint32_t acc, uint32_t* sink) {
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

// Mode 0: grid-stride 16-byte loads, U in flight per thread, consumed in registers.
template <int U>
__global__ __launch_bounds__(RD_THREADS) void probe_read_stride(const uint4* __restrict__ p, int64_t n16,
                                                                uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * RD_THREADS;
  int64_t i = (int64_t)blockIdx.x * RD_THREADS + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc += fold(v[u]);
  }
  for (; i < n16; i += stride) acc += fold(p[i]);
  sink_block(acc, sink);
}

// Mode 1: every wave streams its own contiguous range, U consecutive 1 KB wave
// loads in flight, consumed in registers.
template <int U>
__global__ __launch_bounds__(RD_THREADS) void probe_read_chunk(const uint4* __restrict__ p, int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (RD_THREADS / 64);
  const int64_t wid = (int64_t)blockIdx.x * (RD_THREADS / 64) + (threadIdx.x >> 6);
  const int64_t per = ((n16 + waves - 1) / waves + 63) / 64 * 64;
  const int64_t lo = wid * per, hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  int64_t i = lo;
  for (; i + 64 * U <= hi; i += 64 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + 64 * u + lane];
#pragma unroll
    for (int u = 0; u < U; ++u) acc += fold(v[u]);
  }
  for (i += lane; i < hi; i += 64) acc += fold(p[i]);
  sink_block(acc, sink);
}

// Modes 2 and 3: every wave streams its own contiguous range into LDS by DMA
// (global_load_lds, 1 KB per wave load), U loads in flight, never read back;
// CPOL 0 (default cache policy) or 2 (non-temporal).
template <int U, int CPOL>
__global__ __launch_bounds__(RD_THREADS) void probe_read_dma(const uint4* __restrict__ p, int64_t n16,
                                                             uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[RD_THREADS / 64][U][1024];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t waves = (int64_t)gridDim.x * (RD_THREADS / 64);
  const int64_t wid = (int64_t)blockIdx.x * (RD_THREADS / 64) + w;
  const int64_t per = ((n16 + waves - 1) / waves + 63) / 64 * 64;
  const int64_t lo = wid * per, hi = lo + per < n16 ? lo + per : n16;
  int slot = 0;
  for (int64_t i = lo; i + 64 <= hi; i += 64) {
    __builtin_amdgcn_global_load_lds((const void*)(p + i + lane),
                                     (__attribute__((address_space(3))) void*)&ring[w][slot][0], 16, 0, CPOL);
    slot = slot + 1 == U ? 0 : slot + 1;
    // keep U loads in flight: the slot issued next is free once the load U back has landed
    __builtin_amdgcn_s_waitcnt((U - 1) | (7 << 4) | (15 << 8));
  }
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  sink_block(lane == 0 ? (uint32_t)hi : 0u, sink);
}

// Mode 4: the decode scoring kernel's stream.  A workgroup owns a contiguous range
// (a multiple of 16 KB); its four waves take 4 KB tiles in turn (wave w reads tiles
// w, w + 4, ...), four 1 KB DMA loads a tile, NST tiles in flight per wave,
// non-temporal.
template <int NST>
__global__ __launch_bounds__(RD_THREADS) void probe_read_tiles(const uint8_t* __restrict__ p, int64_t bytes,
                                                               int64_t per_block, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[NST][RD_THREADS / 64][4096];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t lo = blockIdx.x * per_block;
  const int64_t hi = lo + per_block < bytes ? lo + per_block : bytes;
  int st = 0;
  for (int64_t t = lo + w * 4096; t + 4096 <= hi; t += 4 * 4096) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(p + t + j * 1024 + lane * 16),
                                       (__attribute__((address_space(3))) void*)&ring[st][w][j * 1024], 16, 0, 2);
    st = st + 1 == NST ? 0 : st + 1;
    // keep NST tiles in flight: the stage issued next is free once the tile NST back has landed
    __builtin_amdgcn_s_waitcnt((4 * (NST - 1)) | (7 << 4) | (15 << 8));
  }
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  sink_block(lane == 0 ? (uint32_t)hi : 0u, sink);
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

int li_probe_read_blocks(int blocks_per_cu) { return cus() * blocks_per_cu; }

int li_probe_read(const void* buf, size_t bytes, uint32_t* sink, int mode, int blocks_per_cu, hipStream_t stream) {
  if (!buf || !sink || ((uintptr_t)buf & 15u) || (bytes & 15u) || mode < 0 || mode > 4 || blocks_per_cu < 1 ||
      blocks_per_cu > 16)
    return 1;
  if (mode == 4 && (bytes & 16383u)) return 1;  // whole 16 KB groups of tiles
  const int g = li_probe_read_blocks(blocks_per_cu);
  const uint4* p = (const uint4*)buf;
  const int64_t n = (int64_t)(bytes / 16);
  if (mode == 0)
    probe_read_stride<8><<<g, RD_THREADS, 0, stream>>>(p, n, sink);
  else if (mode == 1)
    probe_read_chunk<8><<<g, RD_THREADS, 0, stream>>>(p, n, sink);
  else if (mode == 2)
    probe_read_dma<12, 0><<<g, RD_THREADS, 0, stream>>>(p, n, sink);
  else if (mode == 3)
    probe_read_dma<12, 2><<<g, RD_THREADS, 0, stream>>>(p, n, sink);
  else {
    int64_t per = ((int64_t)bytes + g - 1) / g;
    per = (per + 16383) / 16384 * 16384;
    probe_read_tiles<3><<<(int)(((int64_t)bytes + per - 1) / per), RD_THREADS, 0, stream>>>((const uint8_t*)buf,
                                                                                      (int64_t)bytes, per, sink);
  }
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
