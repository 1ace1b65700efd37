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
#include "select.h"

namespace li {

constexpr int DC = 32;

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// One workgroup per sequence and 8 heads: thread t computes output t & 31 of head
// 8 blockIdx.x + (t >> 5), so each wave serves two heads, one per 32-lane half.
__global__ __launch_bounds__(256) void compact_query_kernel(const uint16_t* __restrict__ q,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ P, int H,
                                                            int8_t* __restrict__ q8, double* __restrict__ W) {
  const int b = blockIdx.y, h = 8 * blockIdx.x + (threadIdx.x >> 5), i = threadIdx.x & 31;
  const bool hv = h < H;
  const int64_t bh = (int64_t)b * H + min(h, H - 1);
  const uint16_t* qr = q + bh * 128;
  double y = 0.0;
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
  // max |y| over the head's 32 outputs (one half of the wave)
  double amax = fabs(y);
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) amax = fmax(amax, __shfl_xor(amax, o, WAVE));
  const double s = amax > 0.0 ? amax / 127.0 : 1.0;
  if (hv) {
    double t = rint(y / s);
    t = fmin(fmax(t, -127.0), 127.0);
    q8[bh * DC + i] = (int8_t)(int)t;
    if (i == 0) W[bh] = (double)w[bh] * s;
  }
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

//
// LIST (a workgroup's keys are exactly one region of the shortlist selection's
// per-region lists, LT_E * 256 keys): the scores also go to LDS, and once the
// workgroup's tiles are done it lists its region's entries above a threshold of its
// own (list_above_local_threshold), so the selection only runs its exact pass over
// the lists; s1 is still written for the rows whose lists cannot be used.
struct S1List {
  const int32_t* nv;
  int m;
  double* cval;
  int32_t* cid;
  uint32_t* bcnt;
  uint32_t* tau_used;
};

template <int HT, bool LIST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void compact_stage1_kernel(
    const int8_t* __restrict__ q8, const double* __restrict__ W, const int8_t* __restrict__ ck,
    const float* __restrict__ cks, int S, int H, int kpb, double* __restrict__ s1, S1List ls) {
  // head weights in VGPRs up to 32 heads, else LDS broadcasts (64 heads' fp64 weights
  // would take 128 VGPRs and halve the waves per SIMD)
  constexpr bool WREG = HT <= 1;
  __shared__ __attribute__((aligned(16))) double sW[WREG ? 2 : 32 * HT];
  __shared__ __attribute__((aligned(16))) double sv[LIST ? LT_E * 256 : 1];
  __shared__ __attribute__((aligned(16))) uint32_t lscr[LIST ? 24 : 1];
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
  // the next tiles are loaded while this one is scored (compact keys and scales in
  // VGPRs); loads past the range read the last key and are not used
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
    const double sc_ = (double)X##s * acc;                                                                     \
    if ((kb) + lane < kend) s1[(int64_t)b * S + (kb) + lane] = sc_;                                            \
    if constexpr (LIST) sv[(kb) - key0 + lane] = sc_;                                                          \
  } while (0)
  // three tiles rotate: two are in flight while one is scored (one HBM round trip
  // is several tiles' worth of scoring)
  i32x4 A0, A1, B0, B1, C0, C1;
  float As, Bs, Cs;
  int kb = key0 + 64 * wave;
  LI_S1_LOAD(A, kb);
  LI_S1_LOAD(B, kb + 256);
  for (; kb < kend; kb += 768) {
    LI_S1_LOAD(C, kb + 512);
    LI_S1_TILE(A, kb);
    if (kb + 256 >= kend) break;
    LI_S1_LOAD(A, kb + 768);
    LI_S1_TILE(B, kb + 256);
    if (kb + 512 >= kend) break;
    LI_S1_LOAD(B, kb + 1024);
    LI_S1_TILE(C, kb + 512);
  }
#undef LI_S1_LOAD
#undef LI_S1_TILE
  if constexpr (LIST) {
    __syncthreads();
    double v[LT_E];
#pragma unroll
    for (int e = 0; e < LT_E; ++e) v[e] = sv[e * 256 + tid];
    int n_row = S;
    if (ls.nv) n_row = min(max(ls.nv[b], 0), S);
    const int n = max(min(n_row - key0, kpb), 0);
    const int P = gridDim.x;
    list_above_local_threshold<double>(v, n, ls.m, P, (int)blockIdx.x, ls.cval + (int64_t)b * S + key0,
                                       ls.cid + (int64_t)b * S + key0, key0, ls.bcnt + (int64_t)b * P + blockIdx.x,
                                       ls.tau_used + (int64_t)b * 256, lscr);
  }
}

// Stage 2.  A quad of lanes serves two shortlisted candidates: lane g computes,
// for both, the dots of heads 8 g .. 8 g + 7 of each group of 32 heads, each an fp64
// fma chain over the 128 dimensions in ascending order, against the query block
// held as fp64 in LDS dimension-major ([j][head]), so a lane's eight query
// operands of one dimension are four 16-byte reads from one address (the quad's
// four lanes read 256 contiguous bytes, every quad of the wave the same ones), and
// they are read one dimension ahead of the FMAs that use them.  Every query
// operand read serves both candidates.  The keys stay in VGPRs as bf16 and each
// element is widened once per group.  After each group the head chain advances
// over its 32 heads in ascending order in all four lanes, each step taking its dot
// from the owning lane with a quad broadcast (DPP).
constexpr int S2_THREADS = 256;
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

// eight fp64 query operands (16-byte LDS reads at a, a + 16, a + 32, a + 48)
__device__ __forceinline__ void s2_read_q(double (&v)[8], const double* a) {
  const double2* p = (const double2*)a;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double2 x = p[i];
    v[2 * i] = x.x;
    v[2 * i + 1] = x.y;
  }
}

template <int U>
__global__ __launch_bounds__(S2_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void compact_stage2_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ kf,
    const int32_t* __restrict__ sl, const int32_t* __restrict__ nv, int S, int H, int m, double* __restrict__ s2,
    int32_t* __restrict__ cnt) {
  static_assert(U % 8 == 0, "eight heads per lane at a time");
  constexpr int HP = 4 * U;  // heads, padded to whole groups of 32
  extern __shared__ __attribute__((aligned(16))) double sqd[];  // [128][HP] query as fp64 (zero past H), [HP] w
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  // a thread widens eight dimensions of one head; neighbouring threads take
  // neighbouring heads, so each 8-byte store lands next to the last one's
  for (int i = tid; i < HP * 16; i += S2_THREADS) {
    const int h = i % HP, jb = i / HP;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (h < H) x = *(const uint4*)(q + ((int64_t)b * H + h) * 128 + 8 * jb);
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sqd[(8 * jb + 2 * e) * HP + h] = (double)__uint_as_float(xw[e] << 16);
      sqd[(8 * jb + 2 * e + 1) * HP + h] = (double)__uint_as_float(xw[e] & 0xFFFF0000u);
    }
  }
  double* sw = sqd + 128 * HP;
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
#pragma unroll 1
  for (int hb = 0; hb < HP; hb += 32) {
    // the keys count as rewritten here, so their widened values are not hoisted
    // out of the loop (kept for every group they would need 512 registers)
    LI_TOUCH4(k0, 0); LI_TOUCH4(k0, 4); LI_TOUCH4(k0, 8); LI_TOUCH4(k0, 12);
    LI_TOUCH4(k1, 0); LI_TOUCH4(k1, 4); LI_TOUCH4(k1, 8); LI_TOUCH4(k1, 12);
    // this lane's heads hb + 8 g .. hb + 8 g + 7; dimension j's operands at qrow + j HP
    const double* qrow = sqd + hb + 8 * g;
    double d0[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    double d1[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    double qa[8], qb[8];
    s2_read_q(qa, qrow);
    // dimensions in pairs: the odd one's operands are read before the even one's FMAs,
    // the next even one's before the odd one's
#define LI_S2_FMA(QV, KV0, KV1)                                                     \
  _Pragma("unroll") for (int t = 0; t < 8; ++t) {                                   \
    d0[t] = fma(QV[t], KV0, d0[t]);                                                 \
    d1[t] = fma(QV[t], KV1, d1[t]);                                                 \
  }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t w0[4] = {k0[i].x, k0[i].y, k0[i].z, k0[i].w};
      const uint32_t w1[4] = {k1[i].x, k1[i].y, k1[i].z, k1[i].w};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int j = 8 * i + 2 * e2;
        s2_read_q(qb, qrow + (j + 1) * HP);
        {
          const double kv0 = (double)__uint_as_float(w0[e2] << 16), kv1 = (double)__uint_as_float(w1[e2] << 16);
          LI_S2_FMA(qa, kv0, kv1)
        }
        if (j + 2 < 128) s2_read_q(qa, qrow + (j + 2) * HP);
        {
          const double kv0 = (double)__uint_as_float(w0[e2] & 0xFFFF0000u);
          const double kv1 = (double)__uint_as_float(w1[e2] & 0xFFFF0000u);
          LI_S2_FMA(qb, kv0, kv1)
        }
        // all sixteen chains advance together, a pair of dimensions at a time (run one
        // after the other they would keep every query operand live)
        asm volatile("" : "+v"(d0[0]), "+v"(d0[1]), "+v"(d0[2]), "+v"(d0[3]), "+v"(d0[4]), "+v"(d0[5]),
                     "+v"(d0[6]), "+v"(d0[7]), "+v"(d1[0]), "+v"(d1[1]), "+v"(d1[2]), "+v"(d1[3]), "+v"(d1[4]),
                     "+v"(d1[5]), "+v"(d1[6]), "+v"(d1[7]));
      }
    }
#undef LI_S2_FMA
    // head chain over heads hb .. hb + 31, ascending: head hb + 8 G + t is lane G's d[t]
#define LI_STEP(G_)                                                               \
  _Pragma("unroll") for (int t = 0; t < 8; ++t) {                                 \
    const int h = hb + 8 * (G_) + t;                                              \
    const double x0 = quad_bcast<G_>(d0[t]), x1 = quad_bcast<G_>(d1[t]);          \
    if (h < H) {                                                                  \
      acc0 = fma(sw[h], x0 > 0.0 ? x0 : 0.0, acc0);                               \
      acc1 = fma(sw[h], x1 > 0.0 ? x1 : 0.0, acc1);                               \
    }                                                                             \
  }
    LI_STEP(0) LI_STEP(1) LI_STEP(2) LI_STEP(3)
#undef LI_STEP
  }
  if (g == 0 && c0 < m) s2[(int64_t)b * m + c0] = v0 ? acc0 : -INFINITY;
  if (g == 0 && c0 + 1 < m) s2[(int64_t)b * m + c0 + 1] = v1 ? acc1 : -INFINITY;
}
#undef LI_TOUCH4

// 128 heads need 130 KB of dynamic LDS in stage 2 (the query block in fp64)
static void stage2_attrs() {
  static const bool set = [] {
    (void)hipFuncSetAttribute((const void*)compact_stage2_kernel<8>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipFuncSetAttribute((const void*)compact_stage2_kernel<16>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipFuncSetAttribute((const void*)compact_stage2_kernel<32>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    return true;
  }();
  (void)set;
}

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

  compact_query_kernel<<<dim3((H + 7) / 8, B), 256, 0, st>>>(q, w, P, H, q8, W);
  const int kpb = stage1_keys_per_block(B, S);
  const dim3 g1((S + kpb - 1) / kpb, B);
  // the shortlist's per-region lists straight from stage 1 when its workgroups are
  // the selection's regions
  int region = 0;
  const bool listed = topk_f64_rows_listed(B, S, &region) && kpb == region;
  S1List ls{nv, m, nullptr, nullptr, nullptr, nullptr};
  if (listed) topk_mb_layout_f64(tk_ws, B, S, &ls.tau_used, &ls.bcnt, &ls.cval, &ls.cid);
#define LI_STAGE1(HT_)                                                                     \
  do {                                                                                     \
    if (listed)                                                                            \
      compact_stage1_kernel<HT_, true><<<g1, 256, 0, st>>>(q8, W, ck, cks, S, H, kpb, s1, ls);  \
    else                                                                                   \
      compact_stage1_kernel<HT_, false><<<g1, 256, 0, st>>>(q8, W, ck, cks, S, H, kpb, s1, ls); \
  } while (0)
  if (H <= 32)
    LI_STAGE1(1);
  else if (H <= 64)
    LI_STAGE1(2);
  else
    LI_STAGE1(4);
#undef LI_STAGE1
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = listed ? launch_topk_finalize_f64(s1, nv, B, S, m, ls.bcnt, ls.cval, ls.cid, sl, nullptr, ls.tau_used, st)
             : launch_topk_f64_rows(s1, nv, B, S, m, sl, nullptr, tk_ws, st);
  if (e != hipSuccess) return e;
  stage2_attrs();
  const dim3 g2((m + S2_CPB - 1) / S2_CPB, B);
#define LI_STAGE2(U_)                                                                                    \
  compact_stage2_kernel<U_><<<g2, S2_THREADS, sizeof(double) * (size_t)(4 * U_) * (128 + 1), st>>>( \
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

// ---- product-quantised compact keys ----------------------------------------
// LeanSparse podcast transcript, cues 07:12-07:34: each 128-d key is split into 32
// four-dimension pieces, each stored as a one-byte index into that piece's
// 256-entry codebook.  The coarse score is the asymmetric distance (the query is
// not quantised by the codebook): per head the dot of the query with the decoded
// key, computed exactly from int8 parts:
//   query   qs_h = max|q_h| / 127 (1 if zero), q8_h = rint(q_h / qs_h) clamped to
//           [-127, 127], W_h = (w_h * qs_h) * sigma (fp64);
//   stage 1 D_h = sum over pieces j of q8_h[4j..4j+3] . cb[j][code_j] (exact
//           int32), s1 = chain_h(W_h, max(D_h, 0)) (fp64 fma chain, h ascending);
// then the same shortlist, exact rerank and final selection as above.
//
// The per-head lookup tables of a classic scan would hold 64 x 32 x 256 sums per
// query (1 MiB at 64 heads), far past LDS; the codebook itself is 32 KiB (one
// 32-bit word per entry), so the stage-1 kernel keeps the codebook in LDS, decodes
// each key's 32 codes into its 128 int8 values with 32 LDS reads, and lets the int8
// matrix core form every head's dot (the same sums the tables would give).
constexpr int PQ_PIECES = 32;

// One wave per (b, h); lane l owns dimensions 2 l and 2 l + 1.
__global__ __launch_bounds__(64) void pq_query_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                                                      double sigma, int8_t* __restrict__ q8,
                                                      double* __restrict__ W) {
  const int bh = blockIdx.x, l = threadIdx.x;
  const uint32_t two = ((const uint32_t*)(q + (int64_t)bh * 128))[l];
  const double v0 = (double)__uint_as_float(two << 16), v1 = (double)__uint_as_float(two & 0xFFFF0000u);
  const double amax = wave_max_d(fmax(fabs(v0), fabs(v1)));
  const double qs = amax > 0.0 ? amax / 127.0 : 1.0;
  const double t0 = fmin(fmax(rint(v0 / qs), -127.0), 127.0), t1 = fmin(fmax(rint(v1 / qs), -127.0), 127.0);
  ((uint16_t*)(q8 + (int64_t)bh * 128))[l] = (uint16_t)(((int)t0 & 0xFF) | (((int)t1 & 0xFF) << 8));
  if (l == 0) W[bh] = ((double)w[bh] * qs) * sigma;
}

// Stage 1.  A wave scores 64 keys per step, as compact_stage1_kernel, with K = 128:
// in K step ks lane half hf carries dimensions 64 hf + 16 ks .. + 15 (pieces
// 16 hf + 4 ks .. + 3) of both the query (A operand) and the key (B operand), so a
// lane's 16 code bytes (one 16-byte load per key) give its four B operands through
// 16 codebook reads.  Four v_mfma_i32_32x32x32_i8 per 32 heads and 32 keys.
template <int HT, bool LIST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void pq_stage1_kernel(
    const int8_t* __restrict__ q8, const double* __restrict__ W, const uint32_t* __restrict__ cb,
    const uint8_t* __restrict__ codes, int S, int H, int kpb, double* __restrict__ s1, S1List ls) {
  constexpr bool WREG = HT <= 1;  // head weights in VGPRs up to 32 heads (64 would spill), else LDS broadcasts
  __shared__ __attribute__((aligned(16))) uint32_t scb[PQ_PIECES * 256];
  __shared__ __attribute__((aligned(16))) double sW[WREG ? 2 : 32 * HT];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, col = lane & 31;
  for (int i = tid; i < PQ_PIECES * 256 / 4; i += 256) ((uint4*)scb)[i] = ((const uint4*)cb)[i];
  i32x4 a[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int h = ht * 32 + col;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      a[ht][ks] = h < H ? *(const i32x4*)(q8 + ((int64_t)b * H + h) * 128 + 64 * hf + 16 * ks) : i32x4{0, 0, 0, 0};
  }
  double wr[WREG ? 32 * HT : 1];
  if constexpr (WREG) {
    const int z = __builtin_amdgcn_mbcnt_lo(0u, 0u);
#pragma unroll
    for (int h = 0; h < 32 * HT; ++h) wr[h] = h < H ? W[(int64_t)b * H + h + z] : 0.0;
  } else {
    for (int h = tid; h < 32 * HT; h += 256) sW[h] = h < H ? W[(int64_t)b * H + h] : 0.0;
  }
  __syncthreads();
  const int key0 = blockIdx.x * kpb, kend = min(key0 + kpb, S);
  const uint8_t* cbase = codes + (int64_t)b * S * PQ_PIECES;
  const uint32_t cbl = lds_addr(scb) + (uint32_t)(16 * hf * 256 * 4);  // this lane half's first piece
  // B operands of K step ks from the 16 code bytes X (pieces 16 hf + 4 ks + e)
  auto decode = [&](const i32x4 X, i32x4 (&bo)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t code = ((uint32_t)X[ks] >> (8 * e)) & 0xFFu;
        const uint32_t addr = cbl + (uint32_t)(((4 * ks + e) * 256) * 4) + 4u * code;
        bo[ks][e] = *(const __attribute__((address_space(3))) int*)(uintptr_t)addr;
      }
  };
#define LI_PQ_LOAD(X, kb)                                                                           \
  do {                                                                                              \
    X##0 = *(const i32x4*)(cbase + (int64_t)min((kb) + col, S - 1) * PQ_PIECES + 16 * hf);         \
    X##1 = *(const i32x4*)(cbase + (int64_t)min((kb) + 32 + col, S - 1) * PQ_PIECES + 16 * hf);    \
  } while (0)
#define LI_PQ_TILE(X, kb)                                                                                      \
  do {                                                                                                         \
    i32x4 b0[4], b1[4];                                                                                        \
    decode(X##0, b0);                                                                                          \
    decode(X##1, b1);                                                                                          \
    double acc = 0.0;                                                                                          \
    _Pragma("unroll") for (int ht = 0; ht < HT; ++ht) {                                                        \
      i32x16 d0 = {}, d1 = {};                                                                                 \
      _Pragma("unroll") for (int ks = 0; ks < 4; ++ks) {                                                       \
        d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ht][ks], b0[ks], d0, 0, 0, 0);                            \
        d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ht][ks], b1[ks], d1, 0, 0, 0);                            \
      }                                                                                                        \
      _Pragma("unroll") for (int r = 0; r < 16; ++r) {                                                          \
        const auto sw2 = __builtin_amdgcn_permlane32_swap((unsigned)d0[r], (unsigned)d1[r], false, false);    \
        d0[r] = (int)sw2[0];                                                                                    \
        d1[r] = (int)sw2[1];                                                                                    \
      }                                                                                                        \
      _Pragma("unroll") for (int g4 = 0; g4 < 4; ++g4) {                                                        \
        asm volatile("" : "+v"(d0[4 * g4]), "+v"(d0[4 * g4 + 1]), "+v"(d0[4 * g4 + 2]), "+v"(d0[4 * g4 + 3]),   \
                     "+v"(d1[4 * g4]), "+v"(d1[4 * g4 + 1]), "+v"(d1[4 * g4 + 2]), "+v"(d1[4 * g4 + 3])         \
                     : "v"(acc));                                                                              \
        _Pragma("unroll") for (int e = 0; e < 8; ++e) {                                                         \
          const int h = 32 * ht + 8 * g4 + e;                                                                  \
          const int dv = e < 4 ? d0[4 * g4 + e] : d1[4 * g4 + e - 4];                                           \
          double wh;                                                                                           \
          if constexpr (WREG) wh = wr[h]; else wh = sW[h];                                                      \
          acc = fma(wh, (double)(dv > 0 ? dv : 0), acc);                                                       \
        }                                                                                                      \
      }                                                                                                        \
    }                                                                                                          \
    if ((kb) + lane < kend) s1[(int64_t)b * S + (kb) + lane] = acc;                                            \
  } while (0)
  i32x4 A0, A1, B0, B1;
  int kb = key0 + 64 * wave;
  LI_PQ_LOAD(A, kb);
  for (; kb < kend; kb += 512) {
    LI_PQ_LOAD(B, kb + 256);
    LI_PQ_TILE(A, kb);
    if (kb + 256 >= kend) break;
    LI_PQ_LOAD(A, kb + 512);
    LI_PQ_TILE(B, kb + 256);
  }
#undef LI_PQ_LOAD
#undef LI_PQ_TILE
  if constexpr (LIST) {
    // this workgroup's region of scores, read back (its own writes: the barrier
    // orders them), then listed above the region's own threshold
    __shared__ __attribute__((aligned(16))) uint32_t lscr[24];
    __syncthreads();
    int n_row = S;
    if (ls.nv) n_row = min(max(ls.nv[b], 0), S);
    const int n = max(min(n_row - key0, kpb), 0);
    double v[LT_E];
#pragma unroll
    for (int e = 0; e < LT_E; ++e) v[e] = e * 256 + tid < n ? s1[(int64_t)b * S + key0 + e * 256 + tid] : 0.0;
    const int P = gridDim.x;
    list_above_local_threshold<double>(v, n, ls.m, P, (int)blockIdx.x, ls.cval + (int64_t)b * S + key0,
                                       ls.cid + (int64_t)b * S + key0, key0, ls.bcnt + (int64_t)b * P + blockIdx.x,
                                       ls.tau_used + (int64_t)b * 256, lscr);
  }
}

size_t pq_ws_bytes(int B, int S, int H, int m, int k) {
  (void)k;
  size_t n = 0;
  n += align256((size_t)B * H * 128);         // q8
  n += align256((size_t)B * H * 8);           // W
  n += align256((size_t)B * S * 8);           // s1
  n += align256((size_t)B * m * 4);           // shortlist
  n += align256((size_t)B * m * 8);           // s2
  n += align256((size_t)B * 4);               // cnt
  n += align256(topk_f64_rows_ws_bytes(B, S));  // shortlist selection
  return n;
}

hipError_t launch_pq(const uint16_t* q, const float* w, const int8_t* cb, float sigma, const uint8_t* codes,
                     const uint16_t* kf, const int32_t* nv, int B, int S, int H, int m, int k, int32_t* shortlist,
                     int32_t* idx, double* val, void* ws, hipStream_t st) {
  uint8_t* p = (uint8_t*)ws;
  int8_t* q8 = (int8_t*)p;
  p += align256((size_t)B * H * 128);
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

  pq_query_kernel<<<B * H, 64, 0, st>>>(q, w, (double)sigma, q8, W);
  const int kpb = stage1_keys_per_block(B, S);
  const dim3 g1((S + kpb - 1) / kpb, B);
  const uint32_t* cbw = (const uint32_t*)cb;
  int region = 0;
  const bool listed = topk_f64_rows_listed(B, S, &region) && kpb == region;
  S1List ls{nv, m, nullptr, nullptr, nullptr, nullptr};
  if (listed) topk_mb_layout_f64(tk_ws, B, S, &ls.tau_used, &ls.bcnt, &ls.cval, &ls.cid);
#define LI_PQ1(HT_)                                                                          \
  do {                                                                                       \
    if (listed)                                                                              \
      pq_stage1_kernel<HT_, true><<<g1, 256, 0, st>>>(q8, W, cbw, codes, S, H, kpb, s1, ls);  \
    else                                                                                     \
      pq_stage1_kernel<HT_, false><<<g1, 256, 0, st>>>(q8, W, cbw, codes, S, H, kpb, s1, ls); \
  } while (0)
  if (H <= 32)
    LI_PQ1(1);
  else if (H <= 64)
    LI_PQ1(2);
  else
    LI_PQ1(4);
#undef LI_PQ1
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = listed ? launch_topk_finalize_f64(s1, nv, B, S, m, ls.bcnt, ls.cval, ls.cid, sl, nullptr, ls.tau_used, st)
             : launch_topk_f64_rows(s1, nv, B, S, m, sl, nullptr, tk_ws, st);
  if (e != hipSuccess) return e;
  stage2_attrs();
  const dim3 g2((m + S2_CPB - 1) / S2_CPB, B);
#define LI_STAGE2(U_)                                                                                    \
  compact_stage2_kernel<U_><<<g2, S2_THREADS, sizeof(double) * (size_t)(4 * U_) * (128 + 1), st>>>( \
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
