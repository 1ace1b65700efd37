// Sparse attention over the selected latent rows for gfx950.
//
// "Long context", llm-serving.xyz lecture 03, section "The Architectural Answer",
// paragraph "Stage 2, sparse main attention": exact attention over only the top-k
// selected entries; section "Sparsity Is a Systems Feature: The Blast Radius",
// "Kernel layer": an MQA-shaped kernel that gathers the rows by token index.  Each
// selected row is a 576-element latent shared by every query head; keys use all 576
// elements and values the first 512.
//
// One workgroup (4 waves) handles one sequence and 32 query heads.  Selected rows
// are gathered 32 at a time into LDS; the logits are formed transposed,
// S^T[row, head] = K . Q^T with v_mfma_f32_32x32x16_bf16 (the 36 K-steps of 16 dims
// split over the 4 waves and summed through LDS), so that each lane owns one head
// and the softmax statistics are lane-local.  The probabilities, already in the
// accumulator layout, serve directly as the B operand of O^T[dv, head] = V^T . P^T
// (rounded to bf16), with V^T read from the LDS copy of the same rows.  An online
// softmax carries the running max and sum across the chunks.
#include "common.h"
#include "launch.h"

namespace li {

constexpr int AT_DQK = 576;
constexpr int AT_DV = 512;
constexpr int AT_CH = 32;      // rows per chunk
constexpr int AT_ROWB = 1168;  // LDS bytes per row (1152 + 16 padding)

__global__ __launch_bounds__(256) void sparse_attn_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ kv,
                                                          const int32_t* __restrict__ idx, int B, int Hq, int S, int k,
                                                          float tau, uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint8_t skv[AT_CH * AT_ROWB];
  __shared__ float spart[4][16][64];
  __shared__ int svalid[AT_CH];

  // block -> (sequence, head tile): the head tiles of one sequence land on blocks
  // 8 apart, which the dispatcher places on the same XCD, so they share its L2.
  const int nt = Hq / 32;
  const int L = blockIdx.x;
  const int xcd = L & 7, round = L >> 3;
  const int ht = round % nt;
  const int b = (round / nt) * 8 + xcd;
  if (b >= B) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, col = lane & 31;
  const int head = ht * 32 + col;

  // Q^T (B operand) for this wave's K-steps 9*wave .. 9*wave + 8
  bf16x8 qb[9];
  const uint16_t* qrow = q + ((int64_t)b * Hq + head) * AT_DQK;
#pragma unroll
  for (int kk = 0; kk < 9; ++kk) {
    const int g = 9 * wave + kk;
    qb[kk] = __builtin_bit_cast(bf16x8, *(const uint4*)(qrow + 16 * g + 8 * hf));
  }

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) o[t] = (f32x16){};

  const int32_t* irow = idx + (int64_t)b * k;
  for (int c0 = 0; c0 < k; c0 += AT_CH) {
    // gather 32 rows (72 x 16 B each) into LDS
    for (int ci = tid; ci < AT_CH * 72; ci += 256) {
      const int r = ci / 72, part = ci - r * 72;
      const int id = (c0 + r < k) ? irow[c0 + r] : -1;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (id >= 0 && id < S) v = ((const uint4*)(kv + ((int64_t)b * S + id) * AT_DQK))[part];
      *(uint4*)(skv + r * AT_ROWB + part * 16) = v;
    }
    if (tid < AT_CH) {
      const int id = (c0 + tid < k) ? irow[c0 + tid] : -1;
      svalid[tid] = (id >= 0 && id < S);
    }
    __syncthreads();

    // partial S^T over this wave's K-steps
    f32x16 s = {};
#pragma unroll
    for (int kk = 0; kk < 9; ++kk) {
      const int g = 9 * wave + kk;
      const bf16x8 a = __builtin_bit_cast(bf16x8, *(const uint4*)(skv + col * AT_ROWB + 2 * (16 * g + 8 * hf)));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[kk], s, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) spart[wave][r][lane] = s[r];
    __syncthreads();

    float st[16];
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = (r & 3) + 8 * (r >> 2) + 4 * hf;
      float x = spart[0][r][lane] + spart[1][r][lane] + spart[2][r][lane] + spart[3][r][lane];
      x = svalid[row] ? x * tau : -INFINITY;
      st[r] = x;
      mloc = fmaxf(mloc, x);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    float alpha, lsum = 0.0f;
    bf16x8 pb[2];
    if (m_new == -INFINITY) {
      alpha = 1.0f;
#pragma unroll
      for (int sidx = 0; sidx < 2; ++sidx) pb[sidx] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    } else {
      alpha = expf(m_run - m_new);
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = expf(st[r] - m_new);
        lsum += p[r];
      }
#pragma unroll
      for (int sidx = 0; sidx < 2; ++sidx) {
        uint32_t wds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          wds[e] = (uint32_t)f32_to_bf16(p[8 * sidx + 2 * e]) | ((uint32_t)f32_to_bf16(p[8 * sidx + 2 * e + 1]) << 16);
        pb[sidx] = __builtin_bit_cast(bf16x8, make_uint4(wds[0], wds[1], wds[2], wds[3]));
      }
    }
    lsum += __shfl_xor(lsum, 32, 64);
    l_run = l_run * alpha + lsum;
    m_run = m_new;

#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
      const int dv = (4 * wave + t) * 32 + col;
#pragma unroll
      for (int sidx = 0; sidx < 2; ++sidx) {
        uint32_t wds[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int e0 = 2 * e2, e1 = 2 * e2 + 1;
          const int r0 = (e0 & 3) + 8 * (e0 >> 2) + 4 * hf + 16 * sidx;
          const int r1 = (e1 & 3) + 8 * (e1 >> 2) + 4 * hf + 16 * sidx;
          const uint32_t v0 = *(const uint16_t*)(skv + r0 * AT_ROWB + 2 * dv);
          const uint32_t v1 = *(const uint16_t*)(skv + r1 * AT_ROWB + 2 * dv);
          wds[e2] = v0 | (v1 << 16);
        }
        const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(wds[0], wds[1], wds[2], wds[3]));
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[sidx], o[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  uint16_t* orow = out + ((int64_t)b * Hq + head) * AT_DV;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dv = (4 * wave + t) * 32 + (r & 3) + 8 * (r >> 2) + 4 * hf;
      orow[dv] = f32_to_bf16(o[t][r] * inv);
    }
  }
  if (lse && wave == 0 && hf == 0) lse[(int64_t)b * Hq + head] = l_run > 0.0f ? m_run + logf(l_run) : -INFINITY;
}

size_t attn_ws_bytes(int B, int Hq, int k, int dv) {
  (void)B; (void)Hq; (void)k; (void)dv;
  return 0;
}

hipError_t launch_attn(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int B, int Hq, int S, int k,
                       float sm_scale, uint16_t* out, float* lse, void* ws, hipStream_t st) {
  (void)ws;
  const int nt = Hq / 32;
  const int blocks = ((B + 7) / 8) * 8 * nt;
  sparse_attn_kernel<<<blocks, 256, 0, st>>>(q, kv, idx, B, Hq, S, k, sm_scale, out, lse);
  return hipGetLastError();
}

}  // namespace li
