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

// Widen 16 fp8 E4M3 codes (one uint4) to two 8-element bf16 MFMA operands.
__device__ __forceinline__ void fp8x16_to_bf16(const uint4 raw, bf16x8& lo8, bf16x8& hi8) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, 1.0f, false);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, 1.0f, true);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, 1.0f, false);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, 1.0f, true);
  bf16x2 p4 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.z, 1.0f, false);
  bf16x2 p5 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.z, 1.0f, true);
  bf16x2 p6 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.w, 1.0f, false);
  bf16x2 p7 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.w, 1.0f, true);
  lo8 = (bf16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  hi8 = (bf16x8){p4[0], p4[1], p5[0], p5[1], p6[0], p6[1], p7[0], p7[1]};
}

// Occupancy target (waves per SIMD) and ring depth (tiles in flight per wave) of
// the streaming kernel, per head-tile count and key format: the VGPR budget of the
// resident query block decides the first, LDS (waves x depth x tile) the second.
#ifndef LI_FP8_WPE
#define LI_FP8_WPE 3
#endif
#ifndef LI_FP8_NST
#define LI_FP8_NST 3
#endif
#ifndef LI_BPC_MUL
#define LI_BPC_MUL 1
#endif
template <int HT, bool FP8>
struct StreamCfg {
  static constexpr int WPE = HT == 1 ? 4 : (HT == 2 ? (FP8 ? LI_FP8_WPE : 2) : 1);
  static constexpr int NST = FP8 ? LI_FP8_NST : 2;  // at most 3: the in-loop wait count stays <= 23
  static constexpr int BPC = WPE * LI_BPC_MUL;      // workgroups of 4 waves per CU
};

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

typedef __attribute__((address_space(3))) void lds_void;

// One 32-key tile of one wave: K rows of ROW bytes, stored in LDS as 16-byte
// chunks with the chunk index XOR-swizzled by the key so that the MFMA operand
// reads (16 lanes of one lane half read the same chunk of 16 different keys) hit
// 16 different bank groups.  The global side of each load instruction is 1 KB of
// consecutive key bytes (a permutation inside each row), so the stream is fully
// coalesced.
template <bool FP8>
struct TileGeom {
  static constexpr int ROW = FP8 ? 128 : 256;       // bytes per key
  static constexpr int CPR = ROW / 16;              // 16-byte chunks per key
  static constexpr int LOADS = 32 * CPR / 64;       // load instructions per tile
  static constexpr int KBYTES = 32 * ROW;           // key bytes per tile
  static constexpr int BYTES = KBYTES + (FP8 ? 128 : 0);  // + 32 fp32 scales
  __device__ static int sw(int n) { return FP8 ? ((n >> 1) & 7) : (n & 15); }
  // LDS chunk slot of (key n, chunk c)
  __device__ static int slot(int n, int c) { return n * CPR + (c ^ sw(n)); }
};

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_u8*)p; }

// Issue the loads of one full tile into its LDS stage.  goff[j] is this lane's
// byte offset inside the tile for load instruction j (precomputed); a tile of fp8
// keys also brings its 32 scales (16 bytes from each of lanes 0-7).
template <bool FP8>
__device__ __forceinline__ void issue_tile_full(const uint8_t* tile_base, const float* scale_base, uint32_t lds_tile,
                                                const uint32_t* goff, int lane) {
  typedef TileGeom<FP8> G;
#pragma unroll
  for (int j = 0; j < G::LOADS; ++j)
    __builtin_amdgcn_global_load_lds((const void*)(tile_base + goff[j]), (lds_void*)(uintptr_t)(lds_tile + j * 1024),
                                     16, 0, 0);
  if constexpr (FP8) {
    if (lane < 8)
      __builtin_amdgcn_global_load_lds((const void*)(scale_base + 4 * lane), (lds_void*)(uintptr_t)(lds_tile + G::KBYTES),
                                       16, 0, 0);
  }
}

// The partial last tile of a range: rows past the end repeat the last valid key,
// and the scales come 4 bytes per key, so no load runs past either array.
template <bool FP8>
__device__ __attribute__((noinline)) void issue_tile_tail(const uint8_t* tile_base, const float* scale_base,
                                                          uint32_t lds_tile, int lane, int nkeys) {
  typedef TileGeom<FP8> G;
#pragma unroll
  for (int j = 0; j < G::LOADS; ++j) {
    const int s = j * 64 + lane;
    const int n = s / G::CPR;
    const int c = (s % G::CPR) ^ G::sw(n);
    const int nl = n < nkeys ? n : nkeys - 1;
    __builtin_amdgcn_global_load_lds((const void*)(tile_base + (int64_t)nl * G::ROW + c * 16),
                                     (lds_void*)(uintptr_t)(lds_tile + j * 1024), 16, 0, 0);
  }
  if constexpr (FP8) {
    if (lane < nkeys)
      __builtin_amdgcn_global_load_lds((const void*)(scale_base + lane), (lds_void*)(uintptr_t)(lds_tile + G::KBYTES), 4,
                                       0, 0);
  }
}

template <bool FP8>
__device__ __forceinline__ void issue_tile(const uint8_t* tile_base, const float* scale_base, uint32_t lds_tile,
                                           const uint32_t* goff, int lane, int nkeys) {
  if (nkeys == 32)
    issue_tile_full<FP8>(tile_base, scale_base, lds_tile, goff, lane);
  else
    issue_tile_tail<FP8>(tile_base, scale_base, lds_tile, lane, nkeys);
}

// max(x, 0) on the bit pattern: non-negative floats order like non-negative
// integers and every negative float is a negative integer (exact, -0 -> +0).
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Four 16-byte LDS reads that complete inside the same asm block (the compiler
// cannot see that they only touch a stage whose loads have already landed).
__device__ __forceinline__ void lds_read4(i32x4& r0, i32x4& r1, i32x4& r2, i32x4& r3, uint32_t a0, uint32_t a1,
                                          uint32_t a2, uint32_t a3) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

__device__ __forceinline__ void lds_read4_f32(i32x4& r0, i32x4& r1, i32x4& r2, i32x4& r3, float& f, uint32_t a0,
                                              uint32_t a1, uint32_t a2, uint32_t a3, uint32_t af) {
  asm volatile(
      "ds_read_b128 %0, %5\n\t"
      "ds_read_b128 %1, %6\n\t"
      "ds_read_b128 %2, %7\n\t"
      "ds_read_b128 %3, %8\n\t"
      "ds_read_b32 %4, %9\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(f)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(af)
      : "memory");
}

__device__ __forceinline__ float lds_read_f32(uint32_t a) {
  float r;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r) : "v"(a) : "memory");
  return r;
}

template <int HT, bool FP8, int NST, int WPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE)))
void score_stream_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w, const uint8_t* __restrict__ k,
                         const float* __restrict__ ks, const int32_t* __restrict__ nv, int T, int S, int H,
                         int keys_per_block, float* __restrict__ scores) {
  typedef TileGeom<FP8> G;
  static_assert(NST >= 1 && NST <= 3, "ring depth");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int r = blockIdx.y;
  const int b = r / T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hf = lane >> 5, col = lane & 31;
  int nvis = S;
  if (nv) nvis = min(max(nv[r], 0), S);

  const int key0 = blockIdx.x * keys_per_block;
  const int key_end = min(key0 + keys_per_block, S);
  float* out_row = scores + (int64_t)r * S;

  const uint8_t* kbase = k + (int64_t)b * S * G::ROW;
  const int vis_end = min(key_end, nvis);
  for (int key = max(key0, vis_end) + (int)threadIdx.x; key < key_end; key += 256) out_row[key] = -INFINITY;

  // LDS: the head weights (2 x HT x 16 floats), then each wave's ring of NST tiles
  uint8_t* ring = lds + 2 * HT * 16 * sizeof(float);
  ring = (uint8_t*)(((uintptr_t)ring + 127) & ~(uintptr_t)127);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t my_ring = lds_addr(ring) + (uint32_t)(wave_u * NST * G::BYTES);
  const float* sbase = ks + (int64_t)b * S;
  float* sw = (float*)lds;  // [2][HT][16]
  const int first = key0 + wave_u * 32;
  const int step = 4 * 32;
  constexpr int OPS = G::LOADS + (FP8 ? 1 : 0);  // memory instructions per tile
  // per-lane constants: source offsets of the load instructions, LDS offsets of
  // this lane's operand chunks
  uint32_t goff[G::LOADS];
#pragma unroll
  for (int j = 0; j < G::LOADS; ++j) {
    const int s = j * 64 + lane;
    const int n = s / G::CPR;
    const int c = (s % G::CPR) ^ G::sw(n);
    goff[j] = (uint32_t)(n * G::ROW + c * 16);
  }
  constexpr int NCH = FP8 ? 4 : 8;  // 16-byte operand chunks per lane
  uint32_t roff[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) roff[j] = (uint32_t)(G::slot(col, NCH * hf + j) * 16);
  const uint32_t soff = (uint32_t)(G::KBYTES + 4 * col);

  // head weights in accumulator row order per lane half (read as LDS broadcasts);
  // written before any LDS DMA is in flight
  if (threadIdx.x < 2 * HT * 16) {
    const int g = threadIdx.x >> 4, i = threadIdx.x & 15;
    const int hf2 = g / HT, t = g % HT;
    const int hh = t * 32 + (i & 3) + 8 * (i >> 2) + 4 * hf2;
    sw[(hf2 * HT + t) * 16 + i] = hh < H ? w[(int64_t)r * H + hh] : 0.0f;
  }
  __syncthreads();

  // prologue: NST tiles in flight, issued before the query block is loaded so
  // the two overlap
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    const int t0 = first + st * step;
    if (t0 < vis_end)
      issue_tile<FP8>(kbase + (int64_t)t0 * G::ROW, sbase + t0, my_ring + st * G::BYTES, goff, lane, min(32, S - t0));
  }

  // A operand: query heads t*32 + col, dims [64 hf, 64 hf + 64).
  bf16x8 a[HT][8];
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const int h = t * 32 + col;
    const uint4* qp = (const uint4*)(q + ((int64_t)r * H + (h < H ? h : 0)) * 128 + 64 * hf);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      uint4 v = h < H ? qp[kk] : make_uint4(0, 0, 0, 0);
      a[t][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  int stage = 0, iter = 0;
  for (int tile = first; tile < vis_end; tile += step) {
    // vmcnt counts loads and stores in issue order.  Issued after this tile's
    // loads: the loads of the n_after younger tiles (OPS instructions each) and
    // the score stores of the last min(iter, NST) iterations (one each), so this
    // tile has landed once no more than that many are outstanding.
    const int n_after = min(NST - 1, (vis_end - 1 - tile) / step);
    wait_vmcnt(n_after * OPS + min(iter, NST));
    ++iter;
    const uint32_t la = my_ring + (uint32_t)(stage * G::BYTES);
    const int key = tile + col;
    bf16x8 bop[8];
    float sc = 1.0f;
    i32x4 raw[NCH];
    if constexpr (FP8) {
      lds_read4_f32(raw[0], raw[1], raw[2], raw[3], sc, la + roff[0], la + roff[1], la + roff[2], la + roff[3],
                    la + soff);
    } else {
      lds_read4(raw[0], raw[1], raw[2], raw[3], la + roff[0], la + roff[1], la + roff[2], la + roff[3]);
      lds_read4(raw[4], raw[5], raw[6], raw[7], la + roff[4], la + roff[5], la + roff[6], la + roff[7]);
    }
    // the stage is free again: refill it with the tile NST steps ahead
    const int tn = tile + NST * step;
    if (tn < vis_end) issue_tile<FP8>(kbase + (int64_t)tn * G::ROW, sbase + tn, la, goff, lane, min(32, S - tn));
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 u = make_uint4((uint32_t)raw[j][0], (uint32_t)raw[j][1], (uint32_t)raw[j][2], (uint32_t)raw[j][3]);
        fp8x16_to_bf16(u, bop[2 * j], bop[2 * j + 1]);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) bop[kk] = __builtin_bit_cast(bf16x8, raw[kk]);
    }
    stage = stage + 1 == NST ? 0 : stage + 1;
    float part = 0.0f;
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t][kk], bop[kk], acc, 0, 0, 0);
      // weights via the asm read as well: a compiler-visible LDS read here would
      // be made to wait for every outstanding key load
      const uint32_t wa = lds_addr(&sw[(hf * HT + t) * 16]);
      i32x4 wr[4];
      lds_read4(wr[0], wr[1], wr[2], wr[3], wa, wa + 16, wa + 32, wa + 48);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) part = fmaf(__int_as_float(wr[i4][e]), relu_bits(acc[4 * i4 + e]), part);
      }
    }
    // lanes 0..31 add the partial sum of lanes 32..63 (same key, other heads)
    part += __uint_as_float(__builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false,
                                                             false)[1]);
    if (hf == 0 && key < key_end) out_row[key] = key < nvis ? part * sc : -INFINITY;
  }
}

template <int HT, bool FP8>
static size_t stream_lds_bytes() {
  return 128 + 2 * HT * 16 * sizeof(float) + 4 * (size_t)StreamCfg<HT, FP8>::NST * TileGeom<FP8>::BYTES;
}

static int num_cus() {
  static const int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 256;
    return v;
  }();
  return n;
}

// Keys per workgroup: a multiple of 128 (4 waves x 32 keys) chosen so the grid is
// about `waves_per_cu` resident waves on every CU, one wave of work each.
static int stream_keys_per_block(int R, int S, int blocks_per_cu) {
  const int64_t target = (int64_t)num_cus() * blocks_per_cu;
  int64_t per_row = (target + R - 1) / R;
  if (per_row < 1) per_row = 1;
  int64_t kpb = ((int64_t)S + per_row - 1) / per_row;
  kpb = ((kpb + 127) / 128) * 128;
  if (kpb < 128) kpb = 128;
  return (int)kpb;
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
  if (prefill_scores_apply(q_type, k_type, T, H))
    return launch_prefill_scores((const uint16_t*)q, w, (const uint16_t*)k, nv, B, T, S, H, scores, st);
  if (q_type == DT_BF16 && (k_type == DT_FP8 || k_type == DT_BF16)) {
    const bool f8 = k_type == DT_FP8;
    const uint16_t* qq = (const uint16_t*)q;
    const uint8_t* kk = (const uint8_t*)k;
#define LI_LAUNCH_STREAM(HT_, F8_)                                                                                  \
  do {                                                                                                              \
    typedef StreamCfg<HT_, F8_> C;                                                                                  \
    auto kern = score_stream_kernel<HT_, F8_, C::NST, C::WPE>;                                                      \
    const size_t lds = stream_lds_bytes<HT_, F8_>();                                                                \
    const int kpb = stream_keys_per_block(R, S, C::BPC);                                                            \
    dim3 grid((S + kpb - 1) / kpb, R);                                                                              \
    static const bool attr = [&] {                                                                                  \
      (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);        \
      return true;                                                                                                  \
    }();                                                                                                            \
    (void)attr;                                                                                                     \
    kern<<<grid, 256, lds, st>>>(qq, w, kk, ks, nv, T, S, H, kpb, scores);                                         \
  } while (0)
    if (H <= 32) {
      if (f8) LI_LAUNCH_STREAM(1, true); else LI_LAUNCH_STREAM(1, false);
    } else if (H <= 64) {
      if (f8) LI_LAUNCH_STREAM(2, true); else LI_LAUNCH_STREAM(2, false);
    } else {
      if (f8) LI_LAUNCH_STREAM(4, true); else LI_LAUNCH_STREAM(4, false);
    }
#undef LI_LAUNCH_STREAM
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
