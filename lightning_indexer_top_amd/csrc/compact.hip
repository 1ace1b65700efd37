// Two-stage decode search over compact keys for gfx950.
//
// LeanSparse podcast transcript, cues 07:12-08:00: a cheap, lossy pass over compact
// indexer keys keeps a shortlist of 2,048 candidates, only their original keys are
// fetched, and an exact rerank picks the final 512.  The compact keys here are a
// fixed Gaussian 128 -> 32 projection stored as int8 with a per-key fp32 scale.
//
// Every step is defined to be bit-reproducible on any IEEE machine:
//   query   y_h = P q_h (fp64 fma chain over the 128 dims, ascending),
//           qs_h = max|y_h| / 127 (1 if zero), q8_h = rint(y_h / qs_h) clamped to
//           [-127, 127], W_h = w_h * qs_h (fp64);
//   stage 1 D_h = q8_h . c_s (exact int32), s1 = cs_s * chain_h(W_h, max(D_h, 0))
//           (fp64 fma chain over h ascending), shortlist = top-m of s1;
//   stage 2 s2 = chain_h(w_h, max(chain_j(q_hj, k_sj), 0)) over the shortlisted
//           original bf16 keys (fp64 fma chains, ascending), result = top-k of s2.
// A selection keeps the best entries by (score desc, key index asc) and lists them
// in ascending key index.
#include "common.h"
#include "launch.h"

namespace li {

constexpr int DC = 32;

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// One wave per (b, h).
__global__ __launch_bounds__(64) void compact_query_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                                                           const float* __restrict__ P, int H,
                                                           int8_t* __restrict__ q8, double* __restrict__ W) {
  const int bh = blockIdx.x;
  const int i = threadIdx.x;
  const uint16_t* qr = q + (int64_t)bh * 128;
  double y = 0.0;
  if (i < DC) {
    // the chain runs in ascending j; its operands arrive 64 at a time
#pragma unroll
    for (int j0 = 0; j0 < 128; j0 += 64) {
      float pv[64];
      uint16_t qv[64];
#pragma unroll
      for (int j = 0; j < 64; ++j) {
        pv[j] = P[i * 128 + j0 + j];
        qv[j] = qr[j0 + j];
      }
#pragma unroll
      for (int j = 0; j < 64; ++j) y = fma((double)pv[j], (double)bf16_to_f32(qv[j]), y);
    }
  }
  const double amax = wave_max_d(i < DC ? fabs(y) : 0.0);
  const double s = amax > 0.0 ? amax / 127.0 : 1.0;
  if (i < DC) {
    double t = rint(y / s);
    t = fmin(fmax(t, -127.0), 127.0);
    q8[(int64_t)bh * DC + i] = (int8_t)(int)t;
  }
  if (i == 0) W[bh] = (double)w[bh] * s;
}

// Stage 1.  A wave scores 64 keys at a time: the exact int32 dots D[h][s] of the
// int8 query block (A operand, in VGPRs) against two tiles of 32 compact keys (B
// operand) come from v_mfma_i32_32x32x32_i8, 32 heads per instruction (a query
// row and a compact key are one K = 32 step).  In the accumulator lane (s, half)
// holds half of the heads of key s; one v_permlane32_swap per register pair
// trades the second tile's low half for the first tile's high half, after which
// lane l holds every head dot of key l of the 64, and runs that key's fp64 head
// chain in ascending head order from registers.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

template <int HT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void compact_stage1_kernel(
    const int8_t* __restrict__ q8, const double* __restrict__ W, const int8_t* __restrict__ ck,
    const float* __restrict__ cks, int S, int H, int kpb, double* __restrict__ s1) {
  constexpr bool WREG = HT <= 2;  // head weights in VGPRs (up to 64 heads), else LDS broadcasts
  __shared__ __attribute__((aligned(16))) double sW[WREG ? 2 : 32 * HT];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, col = lane & 31;
  // A operand: head ht*32 + col, query bytes [16 hf, 16 hf + 16)
  i32x4 a[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int h = ht * 32 + col;
    a[ht] = h < H ? *(const i32x4*)(q8 + ((int64_t)b * H + h) * DC + 16 * hf) : i32x4{0, 0, 0, 0};
  }
  double wr[WREG ? 32 * HT : 1];
  if constexpr (WREG) {
    // a lane-dependent zero keeps the (uniform) weights in VGPRs rather than SGPRs
    const int z = __builtin_amdgcn_mbcnt_lo(0u, 0u);
#pragma unroll
    for (int h = 0; h < 32 * HT; ++h) wr[h] = h < H ? W[(int64_t)b * H + h + z] : 0.0;
  } else {
    for (int h = tid; h < 32 * HT; h += 256) sW[h] = h < H ? W[(int64_t)b * H + h] : 0.0;
    __syncthreads();
  }
  const int key0 = blockIdx.x * kpb, kend = min(key0 + kpb, S);
  const int8_t* cbase = ck + (int64_t)b * S * DC;
  const float* sbase = cks + (int64_t)b * S;
  // the next 64-key tile is loaded while this one is scored (compact keys and
  // scales in VGPRs); loads past the range read the last key and are not used
#define LI_S1_LOAD(X, kb)                                                                      \
  do {                                                                                         \
    X##0 = *(const i32x4*)(cbase + (int64_t)min((kb) + col, S - 1) * DC + 16 * hf);            \
    X##1 = *(const i32x4*)(cbase + (int64_t)min((kb) + 32 + col, S - 1) * DC + 16 * hf);       \
    X##s = sbase[min((kb) + lane, S - 1)];                                                     \
  } while (0)
#define LI_S1_TILE(X, kb)                                                                                      \
  do {                                                                                                         \
    double acc = 0.0;                                                                                          \
    _Pragma("unroll") for (int ht = 0; ht < HT; ++ht) {                                                        \
      i32x16 d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ht], X##0, i32x16{}, 0, 0, 0);                       \
      i32x16 d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ht], X##1, i32x16{}, 0, 0, 0);                       \
      /* register r of a tile holds head 8 (r >> 2) + 4 hf + (r & 3); after the swap */                        \
      /* d0 holds heads 8 (r >> 2) + (r & 3) and d1 heads 8 (r >> 2) + 4 + (r & 3)  */                         \
      /* of key lane (tile 0 in lanes 0..31, tile 1 in lanes 32..63) */                                         \
      _Pragma("unroll") for (int r = 0; r < 16; ++r) {                                                          \
        const auto sw2 = __builtin_amdgcn_permlane32_swap((unsigned)d0[r], (unsigned)d1[r], false, false);    \
        d0[r] = (int)sw2[0];                                                                                    \
        d1[r] = (int)sw2[1];                                                                                    \
      }                                                                                                        \
      _Pragma("unroll") for (int g4 = 0; g4 < 4; ++g4) {                                                        \
        /* the group's dots count as depending on the running sum, so they are */                               \
        /* widened when the chain reaches them (not all at once, ahead of it) */                                \
        asm volatile("" : "+v"(d0[4 * g4]), "+v"(d0[4 * g4 + 1]), "+v"(d0[4 * g4 + 2]), "+v"(d0[4 * g4 + 3]),   \
                     "+v"(d1[4 * g4]), "+v"(d1[4 * g4 + 1]), "+v"(d1[4 * g4 + 2]), "+v"(d1[4 * g4 + 3])         \
                     : "v"(acc));                                                                              \
        _Pragma("unroll") for (int e = 0; e < 8; ++e) {                                                         \
          const int h = 32 * ht + 8 * g4 + e;                                                                  \
          const int dv = e < 4 ? d0[4 * g4 + e] : d1[4 * g4 + e - 4];                                           \
          double wh;                                                                                           \
          if constexpr (WREG) wh = wr[h]; else wh = sW[h];                                                      \
          acc = fma(wh, (double)(dv > 0 ? dv : 0), acc); /* heads past H: fma(0, 0, acc) == acc */             \
        }                                                                                                      \
      }                                                                                                        \
      /* the next head group's MFMAs stay after this group's chain */                                          \
      asm volatile("" : "+v"(X##0), "+v"(X##1));                                                               \
    }                                                                                                          \
    if ((kb) + lane < kend) s1[(int64_t)b * S + (kb) + lane] = (double)X##s * acc;                             \
  } while (0)
  i32x4 A0, A1, B0, B1;
  float As, Bs;
  int kb = key0 + 64 * wave;
  LI_S1_LOAD(A, kb);
  for (; kb < kend; kb += 512) {
    LI_S1_LOAD(B, kb + 256);
    LI_S1_TILE(A, kb);
    if (kb + 256 >= kend) break;
    LI_S1_LOAD(A, kb + 512);
    LI_S1_TILE(B, kb + 256);
  }
#undef LI_S1_LOAD
#undef LI_S1_TILE
}

// Stage 2.  A quad of lanes serves two shortlisted candidates: lane g computes,
// for both, the dots of heads g, g + 4, g + 8, ..., eight heads at a time, each
// an fp64 fma chain over the 128 dimensions in ascending order, against the
// query block held as fp64 in LDS (rows padded to 129 doubles, so the quad's four
// heads sit in different banks); every query operand read serves both candidates.
// The keys stay in VGPRs as bf16 and each element is widened once per eight
// FMAs.  After each group of eight heads per lane (32 consecutive heads) the head
// chain advances over those heads in ascending order in all four lanes, each step
// taking its dot from the owning lane with a quad broadcast (DPP).
constexpr int S2_THREADS = 256;
constexpr int S2_QROW = 129;  // LDS row stride of the query block, doubles
constexpr int S2_CPB = S2_THREADS / 2;  // candidates per workgroup

template <int G>
__device__ __forceinline__ double quad_bcast(double v) {
  const int64_t x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)x, G * 0x55, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(x >> 32), G * 0x55, 0xF, 0xF, false);
  return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}

#define LI_TOUCH4(v, i)                                                                                     \
  asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w), "+v"(v[i + 1].x), "+v"(v[i + 1].y), \
               "+v"(v[i + 1].z), "+v"(v[i + 1].w), "+v"(v[i + 2].x), "+v"(v[i + 2].y), "+v"(v[i + 2].z),       \
               "+v"(v[i + 2].w), "+v"(v[i + 3].x), "+v"(v[i + 3].y), "+v"(v[i + 3].z), "+v"(v[i + 3].w))

template <int U>
__global__ __launch_bounds__(S2_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void compact_stage2_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ kf,
    const int32_t* __restrict__ sl, const int32_t* __restrict__ nv, int S, int H, int m, double* __restrict__ s2,
    int32_t* __restrict__ cnt) {
  static_assert(U % 8 == 0, "eight heads per lane at a time");
  extern __shared__ double sqd[];  // [4 U][S2_QROW] query as fp64 (zero past H), then [4 U] weights
  constexpr int HP = 4 * U;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  for (int i = tid; i < HP * 128; i += S2_THREADS) {
    const int h = i >> 7, j = i & 127;
    sqd[h * S2_QROW + j] = h < H ? (double)bf16_to_f32(q[((int64_t)b * H + h) * 128 + j]) : 0.0;
  }
  double* sw = sqd + HP * S2_QROW;
  for (int i = tid; i < HP; i += S2_THREADS) sw[i] = i < H ? (double)w[(int64_t)b * H + i] : 0.0;
  __syncthreads();
  const int c0 = blockIdx.x * S2_CPB + 2 * (tid >> 2), g = tid & 3;
  if (c0 == 0 && g == 0) {
    int n = S;
    if (nv) n = min(max(nv[b], 0), S);
    cnt[b] = min(n, m);
  }
  // lanes past the shortlist recompute its last entry and store nothing
  const int id0 = sl[(int64_t)b * m + min(c0, m - 1)], id1 = sl[(int64_t)b * m + min(c0 + 1, m - 1)];
  const bool v0 = id0 >= 0 && id0 < S, v1 = id1 >= 0 && id1 < S;
  const uint4* kp0 = (const uint4*)(kf + ((int64_t)b * S + (v0 ? id0 : 0)) * 128);
  const uint4* kp1 = (const uint4*)(kf + ((int64_t)b * S + (v1 ? id1 : 0)) * 128);
  uint4 k0[16], k1[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    k0[i] = kp0[i];
    k1[i] = kp1[i];
  }
  double acc0 = 0.0, acc1 = 0.0;
#pragma unroll
  for (int ug = 0; ug < U; ug += 8) {
    // groups of eight heads one after the other: the keys count as rewritten
    // here, so no work of this group moves into the previous one
    LI_TOUCH4(k0, 0); LI_TOUCH4(k0, 4); LI_TOUCH4(k0, 8); LI_TOUCH4(k0, 12);
    LI_TOUCH4(k1, 0); LI_TOUCH4(k1, 4); LI_TOUCH4(k1, 8); LI_TOUCH4(k1, 12);
    const double* qrow = sqd + (4 * ug + g) * S2_QROW;  // head 4 (ug + t) + g is row 4 t ahead
    double d0[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    double d1[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t w0[4] = {k0[i].x, k0[i].y, k0[i].z, k0[i].w};
      const uint32_t w1[4] = {k1[i].x, k1[i].y, k1[i].z, k1[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 8 * i + e;
        const uint32_t b0 = (e & 1) ? (w0[e >> 1] & 0xFFFF0000u) : (w0[e >> 1] << 16);
        const uint32_t b1 = (e & 1) ? (w1[e >> 1] & 0xFFFF0000u) : (w1[e >> 1] << 16);
        const double kv0 = (double)__uint_as_float(b0), kv1 = (double)__uint_as_float(b1);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const double qv = qrow[4 * t * S2_QROW + j];
          d0[t] = fma(qv, kv0, d0[t]);
          d1[t] = fma(qv, kv1, d1[t]);
        }
        // advance all chains together, two elements at a time (run one after
        // the other they would keep every widened key value and query operand live)
        if (e & 1)
          asm volatile("" : "+v"(d0[0]), "+v"(d0[1]), "+v"(d0[2]), "+v"(d0[3]), "+v"(d0[4]), "+v"(d0[5]),
                       "+v"(d0[6]), "+v"(d0[7]), "+v"(d1[0]), "+v"(d1[1]), "+v"(d1[2]), "+v"(d1[3]), "+v"(d1[4]),
                       "+v"(d1[5]), "+v"(d1[6]), "+v"(d1[7]));
      }
    }
    // head chain over heads 4 ug .. 4 ug + 31, ascending
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int h = 4 * (ug + t);
#define LI_STEP(G_)                                                             \
  if (h + G_ < H) {                                                             \
    const double x0 = quad_bcast<G_>(d0[t]), x1 = quad_bcast<G_>(d1[t]);       \
    acc0 = fma(sw[h + G_], x0 > 0.0 ? x0 : 0.0, acc0);                          \
    acc1 = fma(sw[h + G_], x1 > 0.0 ? x1 : 0.0, acc1);                          \
  }
      LI_STEP(0) LI_STEP(1) LI_STEP(2) LI_STEP(3)
#undef LI_STEP
    }
  }
  if (g == 0 && c0 < m) s2[(int64_t)b * m + c0] = v0 ? acc0 : -INFINITY;
  if (g == 0 && c0 + 1 < m) s2[(int64_t)b * m + c0 + 1] = v1 ? acc1 : -INFINITY;
}
#undef LI_TOUCH4

size_t compact_ws_bytes(int B, int S, int H, int m, int k) {
  (void)k;
  size_t n = 0;
  n += align256((size_t)B * H * DC);          // q8
  n += align256((size_t)B * H * 8);           // W
  n += align256((size_t)B * S * 8);           // s1
  n += align256((size_t)B * m * 4);           // shortlist
  n += align256((size_t)B * m * 8);           // s2
  n += align256((size_t)B * 4);               // cnt
  n += align256(topk_f64_rows_ws_bytes(B, S));  // shortlist selection
  return n;
}

static int stage1_keys_per_block(int B, int S) {
  int per_row = (1024 + B - 1) / B;  // about four workgroups per CU in all
  if (per_row < 1) per_row = 1;
  int kpb = (S + per_row - 1) / per_row;
  kpb = ((kpb + 255) / 256) * 256;
  return kpb < 256 ? 256 : kpb;
}

hipError_t launch_compact(const uint16_t* q, const float* w, const float* P, const int8_t* ck, const float* cks,
                          const uint16_t* kf, const int32_t* nv, int B, int S, int H, int m, int k,
                          int32_t* shortlist, int32_t* idx, double* val, void* ws, hipStream_t st) {
  uint8_t* p = (uint8_t*)ws;
  int8_t* q8 = (int8_t*)p;
  p += align256((size_t)B * H * DC);
  double* W = (double*)p;
  p += align256((size_t)B * H * 8);
  double* s1 = (double*)p;
  p += align256((size_t)B * S * 8);
  int32_t* sl_ws = (int32_t*)p;
  p += align256((size_t)B * m * 4);
  double* s2 = (double*)p;
  p += align256((size_t)B * m * 8);
  int32_t* cnt = (int32_t*)p;
  p += align256((size_t)B * 4);
  void* tk_ws = p;
  int32_t* sl = shortlist ? shortlist : sl_ws;

  compact_query_kernel<<<B * H, 64, 0, st>>>(q, w, P, H, q8, W);
  const int kpb = stage1_keys_per_block(B, S);
  const dim3 g1((S + kpb - 1) / kpb, B);
  if (H <= 32)
    compact_stage1_kernel<1><<<g1, 256, 0, st>>>(q8, W, ck, cks, S, H, kpb, s1);
  else if (H <= 64)
    compact_stage1_kernel<2><<<g1, 256, 0, st>>>(q8, W, ck, cks, S, H, kpb, s1);
  else
    compact_stage1_kernel<4><<<g1, 256, 0, st>>>(q8, W, ck, cks, S, H, kpb, s1);
  hipError_t e = launch_topk_f64_rows(s1, nv, B, S, m, sl, nullptr, tk_ws, st);
  if (e != hipSuccess) return e;
  static const bool attr_set = [] {
    // 128 heads need 130 KB of dynamic LDS (the query block in fp64)
    (void)hipFuncSetAttribute((const void*)compact_stage2_kernel<8>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipFuncSetAttribute((const void*)compact_stage2_kernel<16>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipFuncSetAttribute((const void*)compact_stage2_kernel<32>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    return true;
  }();
  (void)attr_set;
  const dim3 g2((m + S2_CPB - 1) / S2_CPB, B);
#define LI_STAGE2(U_)                                                                                    \
  compact_stage2_kernel<U_><<<g2, S2_THREADS, sizeof(double) * (size_t)(4 * U_) * (S2_QROW + 1), st>>>( \
      q, w, kf, sl, nv, S, H, m, s2, cnt)
  if (H <= 32)
    LI_STAGE2(8);
  else if (H <= 64)
    LI_STAGE2(16);
  else
    LI_STAGE2(32);
#undef LI_STAGE2
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_f64(s2, m, cnt, sl, B, m, k, idx, val, st);
}

}  // namespace li
