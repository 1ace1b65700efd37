// Pooled indexer keys (IndexPool) for gfx950: blocks of `pool` token keys are
// pooled into one fp8 key with a per-key scale when the block completes, the
// indexer scores the pooled keys, and the selected blocks are expanded back to
// the token indices the sparse attention reads ("Long context", llm-serving.xyz
// lecture 03, section "The 2025-2026 Hybrid Turn: Linear Attention Returns":
// four indexer keys pooled into one, index_kpool = 4, quartering the indexer
// cache; "Latent Sparse Attention", section "Where the time goes": 32 heads x 128
// dims over keys pooled four at a time, top-512 blocks).
//
// pool_keys_kernel: one wave per four pooled keys (all their token loads in
// flight before the first is used).  Lane l owns dimensions 2l and 2l+1
// (one 32-bit word of each bf16 token row, so every token row is read as one
// coalesced 256-byte wave load); the mean is summed in fp32 in token order and
// scaled by 1/pool (a power of two: exact), the wave's largest magnitude sets the
// scale (amax / 448), and each value is rounded to E4M3 (nearest, ties to even,
// saturating) after an fp32 division by the scale.  Those fp32 steps decide the
// codes, in that order.  HBM-bound: pool x 256 B read and 132 B written per key.
#include "common.h"
#include "launch.h"

namespace li {

// fp32 -> OCP E4M3FN code: round to nearest, ties to even, saturating at +-448
// (bias 7, three mantissa bits; exponent field 0 holds the subnormals n * 2^-9).
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __uint_as_float(u & 0x7FFFFFFFu);
  if (!(a < 448.0f)) return sign | 0x7Eu;
  if (a < 0.015625f) {  // below 2^-6: subnormal codes n * 2^-9, n in [0, 8] (8 = smallest normal)
    const float n = __builtin_rintf(a * 512.0f);  // exact scaling; rint rounds ties to even
    return sign | (uint32_t)n;
  }
  const uint32_t ua = u & 0x7FFFFFFFu;
  uint32_t keep = ua >> 20;  // exponent field (8 bits) and the top three mantissa bits
  const uint32_t rest = ua & 0xFFFFFu, half = 0x80000u;
  if (rest > half || (rest == half && (keep & 1u))) keep += 1u;  // a carry bumps the exponent
  const int e = (int)(keep >> 3) - 127;
  const uint32_t m = keep & 7u;
  if (e > 8 || (e == 8 && m > 6u)) return sign | 0x7Eu;
  return sign | ((uint32_t)(e + 7) << 3) | m;
}

constexpr int POOL_KPW = 4;  // pooled keys per wave: all their token loads are issued before any is used

__global__ __launch_bounds__(256) void pool_keys_kernel(const uint32_t* __restrict__ k, int64_t L, int64_t Sp,
                                                        int pool, float inv_pool, int64_t n_keys,
                                                        uint16_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t key0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * POOL_KPW;
  if (key0 >= n_keys) return;
  uint32_t v[POOL_KPW][8];
#pragma unroll
  for (int u = 0; u < POOL_KPW; ++u) {
    const int64_t key = key0 + u < n_keys ? key0 + u : n_keys - 1;
    const int64_t b = key / Sp, j = key - b * Sp;
    const uint32_t* row = k + ((b * L + j * pool) * 64) + lane;
#pragma unroll
    for (int t = 0; t < 8; ++t) v[u][t] = t < pool ? row[(int64_t)t * 64] : 0u;
  }
#pragma unroll
  for (int u = 0; u < POOL_KPW; ++u) {
    const int64_t key = key0 + u;
    float s0 = __uint_as_float(v[u][0] << 16), s1 = __uint_as_float(v[u][0] & 0xFFFF0000u);
#pragma unroll
    for (int t = 1; t < 8; ++t) {
      if (t < pool) {
        s0 = s0 + __uint_as_float(v[u][t] << 16);
        s1 = s1 + __uint_as_float(v[u][t] & 0xFFFF0000u);
      }
    }
    const float m0 = s0 * inv_pool, m1 = s1 * inv_pool;
    const float amax = wave_max(fmaxf(fabsf(m0), fabsf(m1)));
    const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
    const uint32_t c0 = e4m3_code(m0 / sc), c1 = e4m3_code(m1 / sc);
    if (key < n_keys) {
      codes[key * 64 + lane] = (uint16_t)(c0 | (c1 << 8));
      if (lane == 0) scales[key] = sc;
    }
  }
}

hipError_t launch_pool_keys(const uint16_t* k, int B, int L, int pool, uint8_t* codes, float* scales,
                            hipStream_t st) {
  const int64_t Sp = L / pool;
  const int64_t n = (int64_t)B * Sp;
  if (n == 0) return hipSuccess;
  const int64_t waves = (n + POOL_KPW - 1) / POOL_KPW;
  const int64_t blocks = (waves + 3) / 4;
  pool_keys_kernel<<<(unsigned)blocks, 256, 0, st>>>((const uint32_t*)k, L, Sp, pool, 1.0f / (float)pool, n,
                                                     (uint16_t*)codes, scales);
  return hipGetLastError();
}

// Visible complete blocks of each row: floor(nv_tokens / pool), at most Sp.
__global__ void pooled_nv_kernel(const int32_t* __restrict__ nv_tokens, int R, int pool, int Sp,
                                 int32_t* __restrict__ nvb) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int n = max(nv_tokens[r], 0) / pool;
  nvb[r] = min(n, Sp);
}

// Selected block j of a row -> its tokens pool*j .. pool*j + pool - 1 (ascending,
// since the blocks are listed in ascending order); a padded block gives -1s.
__global__ void expand_blocks_kernel(const int32_t* __restrict__ blk, int64_t n_out, int pool,
                                     int32_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_out) return;
  const int32_t bj = blk[i / pool];
  out[i] = bj < 0 ? -1 : bj * pool + (int32_t)(i % pool);
}

static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t pooled_topk_ws_bytes(int B, int T, int Sp, int H, int topk) {
  const size_t R = (size_t)B * T;
  return a256(R * 4) + a256(R * (size_t)topk * 4) + indexer_topk_ws_bytes(DT_BF16, DT_FP8, B, T, Sp, H, topk);
}

hipError_t launch_pooled_topk(const uint16_t* q, const float* w, const uint8_t* codes, const float* scales,
                              const int32_t* nv_tokens, int B, int T, int Sp, int H, int pool, int topk,
                              int32_t* idx_tokens, float* val_blocks, void* ws, hipStream_t st) {
  const int R = B * T;
  uint8_t* p = (uint8_t*)ws;
  int32_t* nvb = (int32_t*)p;
  p += a256((size_t)R * 4);
  int32_t* blk = (int32_t*)p;
  p += a256((size_t)R * topk * 4);
  if (nv_tokens) {
    pooled_nv_kernel<<<(R + 255) / 256, 256, 0, st>>>(nv_tokens, R, pool, Sp, nvb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch_indexer_topk(q, DT_BF16, w, codes, DT_FP8, scales, nv_tokens ? nvb : nullptr, B, T, Sp, H,
                                     topk, blk, val_blocks, p, st);
  if (e != hipSuccess) return e;
  const int64_t n_out = (int64_t)R * topk * pool;
  expand_blocks_kernel<<<(unsigned)((n_out + 255) / 256), 256, 0, st>>>(blk, n_out, pool, idx_tokens);
  return hipGetLastError();
}

}  // namespace li
