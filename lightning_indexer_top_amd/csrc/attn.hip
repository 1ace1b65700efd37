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
constexpr int AT_KMAX = 2048;  // selected rows per sequence at most
constexpr int AT_GU = AT_CH * 72 / 256;  // 16-byte pieces per thread per chunk
static_assert(AT_CH * 72 == AT_GU * 256, "whole pieces per thread");

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Transpose read of 4 bf16 (gfx950 ds_read_b64_tr_b16): in each group of 16 lanes,
// lane 4 a + b receives element b of the 4-element rows read by lanes a, a + 4,
// a + 8 and a + 12.
__device__ __forceinline__ bf16x4 ds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(__attribute__((address_space(3))) const uint8_t*)p);
}

// the value of x held by the other lane half (lane l +- 32)
__device__ __forceinline__ float other_half(float x, int hf) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(hf ? r[0] : r[1]);
}

__global__ __launch_bounds__(256) void sparse_attn_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ kv,
                                                          const int32_t* __restrict__ idx, int B, int Hq, int S, int k,
                                                          float tau, uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  // two chunk buffers: the rows of chunk c + 1 are loaded (into VGPRs) while
  // chunk c is computed, and stored into the other buffer after it
  __shared__ __attribute__((aligned(16))) uint8_t skv2[2][AT_CH * AT_ROWB];
  __shared__ float spart[4][16][64];
  __shared__ int sidx[AT_KMAX];

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

  // softmax in base 2: exp(tau x - m) == 2^(tau log2(e) x - m / ln 2)
  const float tau2 = tau * 1.4426950408889634f;
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) o[t] = (f32x16){};

  // the selected rows' indices, -1 for entries that select nothing
  const int32_t* irow = idx + (int64_t)b * k;
  for (int i = tid; i < k; i += 256) {
    const int id = irow[i];
    sidx[i] = (id >= 0 && id < S) ? id : -1;
  }
  __syncthreads();
  const uint16_t* kvb = kv + (int64_t)b * S * AT_DQK;
  // thread tid moves the 16-byte pieces tid + 256 u (u < 9) of a chunk: row
  // piece / 72, part piece % 72; skipped rows load row 0 and store zeros
  // chunk c + 2 is loaded (into VGPRs) while chunk c is computed, chunk c + 1
  // (loaded during chunk c - 1) is stored into the other LDS buffer after it:
  // two register sets, used in turn
  uint4 gA[AT_GU], gB[AT_GU];
  // per-thread piece coordinates (the same for every chunk)
  int prow[AT_GU], ppart[AT_GU];
#pragma unroll
  for (int u = 0; u < AT_GU; ++u) {
    const int pc = tid + 256 * u;
    prow[u] = pc / 72;
    ppart[u] = pc - prow[u] * 72;
  }
  // index reads first (unconditional, clamped), then every row load
#define AT_LOAD(G, c0)                                                                      \
  do {                                                                                      \
    int id_[AT_GU];                                                                         \
    _Pragma("unroll") for (int u = 0; u < AT_GU; ++u) id_[u] = sidx[min((c0) + prow[u], k - 1)]; \
    _Pragma("unroll") for (int u = 0; u < AT_GU; ++u)                                       \
      G[u] = ((const uint4*)(kvb + (int64_t)(id_[u] < 0 ? 0 : id_[u]) * AT_DQK))[ppart[u]];  \
  } while (0)
#define AT_STORE(G, c0, buf)                                                                \
  do {                                                                                      \
    int id_[AT_GU];                                                                         \
    _Pragma("unroll") for (int u = 0; u < AT_GU; ++u) id_[u] = sidx[min((c0) + prow[u], k - 1)]; \
    _Pragma("unroll") for (int u = 0; u < AT_GU; ++u) {                                     \
      const bool live = (c0) + prow[u] < k && id_[u] >= 0;                                 \
      *(uint4*)((buf) + prow[u] * AT_ROWB + ppart[u] * 16) = live ? G[u] : make_uint4(0, 0, 0, 0); \
    }                                                                                       \
  } while (0)
#define AT_BODY(GL, GS)                                                                                               \
    const uint8_t* skv = skv2[it & 1];                                                                                \
    if (c0 + 2 * AT_CH < k) AT_LOAD(GL, c0 + 2 * AT_CH);                                                              \
    /* rows of this chunk that select something (bit r: row c0 + r) */                                                \
    const uint64_t vrow = __ballot(lane < AT_CH && c0 + lane < k && sidx[min(c0 + lane, k - 1)] >= 0);                \
    /* partial S^T over this wave's K-steps: all operand reads first */                                               \
    bf16x8 av[9];                                                                                                     \
    _Pragma("unroll")                                                                                                 \
    for (int kk = 0; kk < 9; ++kk)                                                                                    \
      av[kk] = __builtin_bit_cast(bf16x8, *(const uint4*)(skv + col * AT_ROWB + 2 * (16 * (9 * wave + kk) + 8 * hf))); \
    f32x16 s = {};                                                                                                    \
    _Pragma("unroll")                                                                                                 \
    for (int kk = 0; kk < 9; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kk], qb[kk], s, 0, 0, 0);           \
    _Pragma("unroll")                                                                                                 \
    for (int r = 0; r < 16; ++r) spart[wave][r][lane] = s[r];                                                         \
    lds_barrier();                                                                                                    \
    /* logits in base-2 units (tau log2 e folded in), running max and sum */                                          \
    float st[16];                                                                                                     \
    float mloc = -INFINITY;                                                                                           \
    _Pragma("unroll")                                                                                                 \
    for (int r = 0; r < 16; ++r) {                                                                                    \
      const int row = (r & 3) + 8 * (r >> 2) + 4 * hf;                                                                \
      const float x = spart[0][r][lane] + spart[1][r][lane] + spart[2][r][lane] + spart[3][r][lane];                  \
      st[r] = ((vrow >> row) & 1ull) ? x * tau2 : -INFINITY;                                                          \
      mloc = fmaxf(mloc, st[r]);                                                                                      \
    }                                                                                                                 \
    mloc = fmaxf(mloc, other_half(mloc, hf));                                                                         \
    const float m_new = fmaxf(m_run, mloc);                                                                           \
    float alpha = 1.0f, lsum = 0.0f;                                                                                  \
    bf16x8 pb[2];                                                                                                     \
    if (m_new == -INFINITY) {                                                                                         \
      pb[0] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));                                                     \
      pb[1] = pb[0];                                                                                                  \
    } else {                                                                                                          \
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);                                                                  \
      float p[16];                                                                                                    \
      _Pragma("unroll")                                                                                               \
      for (int r = 0; r < 16; ++r) {                                                                                  \
        p[r] = __builtin_amdgcn_exp2f(st[r] - m_new);                                                                 \
        lsum += p[r];                                                                                                 \
      }                                                                                                               \
      _Pragma("unroll")                                                                                               \
      for (int s2 = 0; s2 < 2; ++s2) {                                                                                \
        bf16x8 v;                                                                                                     \
        _Pragma("unroll")                                                                                             \
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)p[8 * s2 + e];                                                     \
        pb[s2] = v;                                                                                                   \
      }                                                                                                               \
    }                                                                                                                 \
    lsum += other_half(lsum, hf);                                                                                     \
    l_run = l_run * alpha + lsum;                                                                                     \
    m_run = m_new;                                                                                                    \
    /* rescale the outputs only when some head's maximum moved */                                                     \
    const bool rescale = __ballot(alpha != 1.0f) != 0ull;                                                             \
    _Pragma("unroll")                                                                                                 \
    for (int t = 0; t < 4; ++t) {                                                                                     \
      /* V^T operands of this dv tile, lane (dv, hf): rows 4 hf + 0..3 and 8 + 4 hf + 0..3 of */                      \
      /* column dv (then the same 16 rows on), by transpose reads: lane 4 a + b of a group of */                      \
      /* 16 receives element b of the 4-element reads of lanes a, a + 4, a + 8, a + 12, so */                         \
      /* lane i reads columns 4 (i % 4) .. + 3 of row i / 4 */                                                        \
      const int dv0 = (4 * wave + t) * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);                                   \
      bf16x4 vq[4];                                                                                                   \
      _Pragma("unroll")                                                                                               \
      for (int e = 0; e < 4; ++e) {                                                                                   \
        const int row = 4 * hf + 8 * (e & 1) + 16 * (e >> 1) + ((lane >> 2) & 3);                                       \
        vq[e] = ds_read_tr16(skv + row * AT_ROWB + 2 * dv0);                                                          \
      }                                                                                                               \
      if (rescale) {                                                                                                  \
        _Pragma("unroll")                                                                                             \
        for (int r = 0; r < 16; ++r) o[t][r] *= alpha;                                                                \
      }                                                                                                               \
      _Pragma("unroll")                                                                                               \
      for (int sidx2 = 0; sidx2 < 2; ++sidx2) {                                                                       \
        const bf16x8 va = __builtin_shufflevector(vq[2 * sidx2], vq[2 * sidx2 + 1], 0, 1, 2, 3, 4, 5, 6, 7);          \
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[sidx2], o[t], 0, 0, 0);                                 \
      }                                                                                                               \
    }                                                                                                                 \
    if (c0 + AT_CH < k) AT_STORE(GS, c0 + AT_CH, skv2[(it + 1) & 1]);                                                 \
    lds_barrier();
  AT_LOAD(gA, 0);
  AT_STORE(gA, 0, skv2[0]);
  if (AT_CH < k) AT_LOAD(gA, AT_CH);
  lds_barrier();    
  for (int c0 = 0, it = 0; c0 < k;) {
    { AT_BODY(gB, gA); }
    c0 += AT_CH;
    ++it;
    if (c0 >= k) break;
    { AT_BODY(gA, gB); }
    c0 += AT_CH;
    ++it;
  }
#undef AT_BODY
#undef AT_LOAD
#undef AT_STORE

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
  if (lse && wave == 0 && hf == 0)
    lse[(int64_t)b * Hq + head] = l_run > 0.0f ? (m_run + log2f(l_run)) * 0.6931471805599453f : -INFINITY;
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
