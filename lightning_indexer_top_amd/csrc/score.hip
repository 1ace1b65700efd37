// Lightning-indexer scoring kernels for gfx950.
//
// score(r, s) = sum_h w[r, h] * max(q[r, h] . k[b, s], 0)  for s < nv[r]
// ("Long context", llm-serving.xyz lecture 03, section "The Architectural Answer:
// Read Less of the Past", paragraph "Stage 1, the lightning indexer"; the 128 B FP8
// key + 4 B scale layout and the 64 x 128 x 2 FLOP per key of Derivation 4).
//
// score_stream_kernel: bf16 queries against fp8 (or bf16) keys.  Decode is a pure
// stream over the key cache, so each wave owns one query row's 64 x 128 query
// block in VGPRs (the MFMA A operand, loaded once) and streams 32-key tiles
// through v_mfma_f32_32x32x16_bf16 as the B operand.  fp8 codes are widened to
// bf16 in registers (exact: every E4M3 value is a bf16 value); the per-key scale is
// positive, so it commutes with the ReLU and is applied once after the head sum.
//
// MFMA layout used (32x32x16, wave64): lane l supplies row/column (l & 31) of the
// A/B operands and 8 consecutive K elements chosen by l >> 5; the accumulator
// element (i, j) lives in lane j + 32 * ((i / 4) & 1), register (i & 3) + 4 * (i / 8).
// The dot product does not depend on which K positions a lane carries as long as A
// and B agree, so lane half hf carries key dimensions [64 hf, 64 hf + 64), eight
// per K step: each lane then reads 64 (fp8) or 128 (bf16) contiguous bytes of its
// key row.
#include "common.h"
#include "launch.h"

namespace li {

template <int HT, bool FP8>
__global__ __launch_bounds__(256) void score_stream_kernel(const uint16_t* __restrict__ q,
                                                           const float* __restrict__ w,
                                                           const uint8_t* __restrict__ k,
                                                           const float* __restrict__ ks,
                                                           const int32_t* __restrict__ nv, int T, int S, int H,
                                                           int keys_per_block, float* __restrict__ scores) {
  const int r = blockIdx.y;
  const int b = r / T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hf = lane >> 5, col = lane & 31;
  int nvis = S;
  if (nv) nvis = min(max(nv[r], 0), S);

  const int key0 = blockIdx.x * keys_per_block;
  const int key_end = min(key0 + keys_per_block, S);
  float* out_row = scores + (int64_t)r * S;

  // A operand: query heads t*32 + col, dims [64 hf, 64 hf + 64).
  bf16x8 a[HT][8];
  float wv[HT][16];
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const int h = t * 32 + col;
    const uint4* qp = (const uint4*)(q + ((int64_t)r * H + (h < H ? h : 0)) * 128 + 64 * hf);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      uint4 v = h < H ? qp[kk] : make_uint4(0, 0, 0, 0);
      a[t][kk] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hh = t * 32 + (i & 3) + 8 * (i >> 2) + 4 * hf;
      wv[t][i] = hh < H ? w[(int64_t)r * H + hh] : 0.0f;
    }
  }

  const int row_bytes = FP8 ? 128 : 256;
  const uint8_t* kbase = k + (int64_t)b * S * row_bytes;

  for (int tile = key0 + wave * 32; tile < key_end; tile += 4 * 32) {
    const int key = tile + col;
    if (tile >= nvis) {  // whole tile invisible
      if (hf == 0 && key < key_end) out_row[key] = -INFINITY;
      continue;
    }
    const int kld = key < S ? key : S - 1;  // clamp the tail tile's loads in bounds
    const uint8_t* kp = kbase + (int64_t)kld * row_bytes + (FP8 ? 64 : 128) * hf;
    bf16x8 bop[8];
    if constexpr (FP8) {
      uint4 raw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[i] = ((const uint4*)kp)[i];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const uint32_t lo = (kk & 1) ? raw[kk >> 1].z : raw[kk >> 1].x;
        const uint32_t hi = (kk & 1) ? raw[kk >> 1].w : raw[kk >> 1].y;
        bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
        bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
        bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
        bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
        bop[kk] = (bf16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) bop[kk] = __builtin_bit_cast(bf16x8, ((const uint4*)kp)[kk]);
    }
    float part = 0.0f;
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t][kk], bop[kk], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) part = fmaf(wv[t][i], fmaxf(acc[i], 0.0f), part);
    }
    part += __shfl_xor(part, 32, 64);
    if (hf == 0 && key < key_end) {
      float sc = part;
      if constexpr (FP8) sc *= ks[(int64_t)b * S + kld];
      out_row[key] = key < nvis ? sc : -INFINITY;
    }
  }
}

// Generic fp32 path (fp32 queries or keys): one thread per key, fp32 FMAs, the
// query row staged in LDS.  dot_h accumulates over the key dimension in ascending
// order, the head sum over h in ascending order, then the key scale.
template <typename QT, int KT>
__global__ __launch_bounds__(256) void score_valu_kernel(const QT* __restrict__ q, const float* __restrict__ w,
                                                         const void* __restrict__ k, const float* __restrict__ ks,
                                                         const int32_t* __restrict__ nv, int T, int S, int H,
                                                         float* __restrict__ scores) {
  extern __shared__ float sq[];  // [H * 128 + H]
  const int r = blockIdx.y;
  const int b = r / T;
  for (int i = threadIdx.x; i < H * 128; i += blockDim.x) {
    if constexpr (sizeof(QT) == 4)
      sq[i] = q[(int64_t)r * H * 128 + i];
    else
      sq[i] = bf16_to_f32(q[(int64_t)r * H * 128 + i]);
  }
  for (int i = threadIdx.x; i < H; i += blockDim.x) sq[H * 128 + i] = w[(int64_t)r * H + i];
  __syncthreads();
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= S) return;
  int nvis = S;
  if (nv) nvis = min(max(nv[r], 0), S);
  if (s >= nvis) {
    scores[(int64_t)r * S + s] = -INFINITY;
    return;
  }
  float kv[128];
  const int64_t row = (int64_t)b * S + s;
  if constexpr (KT == 0) {
    const float4* kp = (const float4*)((const float*)k + row * 128);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      float4 v = kp[j];
      kv[4 * j] = v.x; kv[4 * j + 1] = v.y; kv[4 * j + 2] = v.z; kv[4 * j + 3] = v.w;
    }
  } else if constexpr (KT == 1) {
    const uint16_t* kp = (const uint16_t*)k + row * 128;
#pragma unroll
    for (int j = 0; j < 128; ++j) kv[j] = bf16_to_f32(kp[j]);
  } else {
    const uint32_t* kp = (const uint32_t*)((const uint8_t*)k + row * 128);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t v = kp[j];
      auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8(v, false);
      auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8(v, true);
      kv[4 * j] = p0[0]; kv[4 * j + 1] = p0[1]; kv[4 * j + 2] = p1[0]; kv[4 * j + 3] = p1[1];
    }
  }
  float acc = 0.0f;
  for (int h = 0; h < H; ++h) {
    float dot = 0.0f;
#pragma unroll
    for (int j = 0; j < 128; ++j) dot = fmaf(sq[h * 128 + j], kv[j], dot);
    acc = fmaf(sq[H * 128 + h], fmaxf(dot, 0.0f), acc);
  }
  if (ks) acc *= ks[row];
  scores[(int64_t)r * S + s] = acc;
}

hipError_t launch_score(const void* q, int q_type, const float* w, const void* k, int k_type, const float* ks,
                        const int32_t* nv, int B, int T, int S, int H, float* scores, hipStream_t st) {
  const int R = B * T;
  if (q_type == DT_BF16 && (k_type == DT_FP8 || k_type == DT_BF16)) {
    const int kpb = 1024;
    dim3 grid((S + kpb - 1) / kpb, R);
    const bool f8 = k_type == DT_FP8;
    const uint16_t* qq = (const uint16_t*)q;
    const uint8_t* kk = (const uint8_t*)k;
    if (H <= 32) {
      if (f8) score_stream_kernel<1, true><<<grid, 256, 0, st>>>(qq, w, kk, ks, nv, T, S, H, kpb, scores);
      else score_stream_kernel<1, false><<<grid, 256, 0, st>>>(qq, w, kk, ks, nv, T, S, H, kpb, scores);
    } else if (H <= 64) {
      if (f8) score_stream_kernel<2, true><<<grid, 256, 0, st>>>(qq, w, kk, ks, nv, T, S, H, kpb, scores);
      else score_stream_kernel<2, false><<<grid, 256, 0, st>>>(qq, w, kk, ks, nv, T, S, H, kpb, scores);
    } else {
      if (f8) score_stream_kernel<4, true><<<grid, 256, 0, st>>>(qq, w, kk, ks, nv, T, S, H, kpb, scores);
      else score_stream_kernel<4, false><<<grid, 256, 0, st>>>(qq, w, kk, ks, nv, T, S, H, kpb, scores);
    }
    return hipGetLastError();
  }
  dim3 grid((S + 255) / 256, R);
  const size_t lds = sizeof(float) * (size_t)H * 129;
  static const bool attr_set = [] {
    // H <= 128 needs up to 66 KB of dynamic LDS
    (void)hipFuncSetAttribute((const void*)score_valu_kernel<float, 0>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              96 * 1024);
    (void)hipFuncSetAttribute((const void*)score_valu_kernel<float, 1>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              96 * 1024);
    (void)hipFuncSetAttribute((const void*)score_valu_kernel<float, 2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              96 * 1024);
    (void)hipFuncSetAttribute((const void*)score_valu_kernel<uint16_t, 0>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    return true;
  }();
  (void)attr_set;
  if (q_type == DT_F32) {
    const float* qq = (const float*)q;
    if (k_type == DT_F32) score_valu_kernel<float, 0><<<grid, 256, lds, st>>>(qq, w, k, ks, nv, T, S, H, scores);
    else if (k_type == DT_BF16) score_valu_kernel<float, 1><<<grid, 256, lds, st>>>(qq, w, k, ks, nv, T, S, H, scores);
    else score_valu_kernel<float, 2><<<grid, 256, lds, st>>>(qq, w, k, ks, nv, T, S, H, scores);
  } else {
    const uint16_t* qq = (const uint16_t*)q;
    score_valu_kernel<uint16_t, 0><<<grid, 256, lds, st>>>(qq, w, k, ks, nv, T, S, H, scores);
  }
  return hipGetLastError();
}

}  // namespace li
