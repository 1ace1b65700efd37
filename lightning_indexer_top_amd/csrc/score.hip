// Lightning-indexer scoring kernels for gfx950.
//
// score(r, s) = sum_h w[r, h] * max(q[r, h] . k[b, s], 0)  for s < nv[r]
// ("Long context", llm-serving.xyz lecture 03, section "The Architectural Answer:
// Read Less of the Past", paragraph "Stage 1, the lightning indexer"; the 128 B FP8
// key + 4 B scale layout and the 64 x 128 x 2 FLOP per key of Derivation 4).
//
// score_stream_kernel: bf16 queries against fp8 (or bf16) keys.  Decode is a pure
// stream over the key cache, so each wave owns one query row's 64 x 128 query
// block in VGPRs (the MFMA A operand, loaded once) and streams 32-key tiles through
// LDS as the B operand.  bf16 keys: v_mfma_f32_32x32x16_bf16.  fp8 keys: the block-
// scaled fp8 MFMA with the key bytes as they arrive and the query split exactly into
// two E4M3 halves (see QSplit below), so no key is converted.  The per-key scale is
// positive, so it commutes with the ReLU and is applied once after the head sum.
//
// bf16 MFMA layout (32x32x16, wave64): lane l supplies row/column (l & 31) of the
// A/B operands and 8 consecutive K elements chosen by l >> 5; the accumulator
// element (i, j) lives in lane j + 32 * ((i / 4) & 1), register (i & 3) + 4 * (i / 8).
// The dot product does not depend on which K positions a lane carries as long as A
// and B agree, so lane half hf carries key dimensions [64 hf, 64 hf + 64), eight
// per K step: each lane then reads 64 (fp8) or 128 (bf16) contiguous bytes of its
// key row.
#include <atomic>

#include "common.h"
#include "launch.h"
#include "select.h"

namespace li {

// Occupancy target (waves per SIMD) and ring depth (tiles in flight per wave) of
// the streaming kernel, per head-tile count and key format: the VGPR budget of the
// resident query block decides the first, LDS (waves x depth x tile) the second.
template <int HT, bool FP8>
struct StreamCfg {
  static constexpr int WPE = HT == 1 ? 4 : (HT == 2 ? (FP8 ? 3 : 2) : 1);
  static constexpr int NST = FP8 ? 3 : 2;  // at most 3: the in-loop wait count stays <= 23
  static constexpr int BPC = WPE;          // workgroups of 4 waves per CU
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

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

// Issue the loads of one full tile into its LDS stage.  goff[j] is this lane's
// byte offset inside the tile for load instruction j (precomputed); a tile of fp8
// keys also brings its 32 scales (16 bytes from each of lanes 0-7).  Keys are read
// once per launch, so the loads carry the streaming cache policy.
template <bool FP8>
__device__ __forceinline__ void issue_tile_full(const uint8_t* tile_base, const float* scale_base, uint32_t lds_tile,
                                                const uint32_t* goff, int lane) {
  typedef TileGeom<FP8> G;
#pragma unroll
  for (int j = 0; j < G::LOADS; ++j)
    __builtin_amdgcn_global_load_lds((const void*)(tile_base + goff[j]), (lds_void*)(uintptr_t)(lds_tile + j * 1024),
                                     16, 0, CPOL_STREAM);
  if constexpr (FP8) {
    if (lane < 8)
      __builtin_amdgcn_global_load_lds((const void*)(scale_base + 4 * lane), (lds_void*)(uintptr_t)(lds_tile + G::KBYTES),
                                       16, 0, CPOL_STREAM);
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
                                     (lds_void*)(uintptr_t)(lds_tile + j * 1024), 16, 0, CPOL_STREAM);
  }
  if constexpr (FP8) {
    if (lane < nkeys)
      __builtin_amdgcn_global_load_lds((const void*)(scale_base + lane), (lds_void*)(uintptr_t)(lds_tile + G::KBYTES), 4,
                                       0, CPOL_STREAM);
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

// fp8 keys: the bf16 query split exactly into two E4M3 halves with power-of-two
// scales, for the block-scaled fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4).  For each
// run of 32 query values whose largest magnitude lies in [2^E, 2^(E+1)):
//   hi = RNE_e4m3(q 2^-(E-7)),  lo = (q 2^-(E-7) - hi) 2^4,  q = hi 2^(E-7) + lo 2^(E-11).
// hi keeps the top 4 significant bits (|q 2^-(E-7)| < 2^8, inside E4M3's range); the
// remainder is a multiple of q's bf16 ulp at most 2^3 of it, so lo holds it exactly
// for every value down to 2^-13 of the run's maximum (below that lo rounds, an error
// of at most 2^-21 of the maximum).  Code x code products are exact and each run of
// 32 codes carries one E8M0 exponent, so hi.k + lo.k is the bf16-query, fp8-key
// product sum, rounded only by the MFMA's fp32 accumulation (measured: within 3e-6
// of sum |q_i k_i| on Gaussian queries, 3e-5 when a run's values span 24 binades),
// and the key bytes are the MFMA operand as they sit in LDS: no per-key conversion.
//
// Operand layout of the 32x32x64 fp8 MFMA (measured on the device): lane l supplies 32
// codes of row/column (l & 31); A lane l pairs code by code with B lanes of the same
// half (l >> 5).  The scale blocks of 32 codes along K are: block kb = bytes
// [16 kb, 16 kb + 16) of both lane halves, and the scale of (row i, block kb) is the
// byte OPSEL selects of lane i + 32 kb's scale operand.  The accumulator layout is
// that of the other 32x32 MFMAs.  Lane half hf carries key dimensions [64 hf,
// 64 hf + 64), 32 per MFMA (kk), the 64 bytes of its key row the LDS operand reads
// return; so scale block (kk, kb) of a head covers dimensions 32 kk + 16 kb + [0, 16)
// and 64 + 32 kk + 16 kb + [0, 16), and that is the run the query split works on.
//
// Query code layout in LDS: slot ((t * 2 + kk) * 2 + hf) * 32 + col holds the 32 codes
// lane (hf, col) feeds MFMA kk of head tile t: hi codes, then lo codes; then per lane
// (hf, col) a record of 2 HT scale bytes, byte t * 2 + kk = the scale of block kb = hf.
template <int HT>
struct QSplit {
  static constexpr int HI = 0;
  static constexpr int LO = HT * 4 * 32 * 32;
  static constexpr int SC = 2 * LO;
  static constexpr int BYTES = SC + 64 * 2 * HT;
};

// hi and lo codes of one run of 32 bf16 values (four uint4), and its scale exponent
__device__ __forceinline__ int split_run(const uint4 (&v)[4], uint32_t (&hi)[8], uint32_t (&lo)[8]) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      m = fmaxf(m, fmaxf(fabsf(__uint_as_float(u[e] << 16)), fabsf(__uint_as_float(u[e] & 0xffff0000u))));
  }
  const int ex = m > 0.0f ? __builtin_amdgcn_frexp_expf(m) - 1 : 0;
  const int sh = min(max(ex - 7, -122), 120);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      const float a0 = __builtin_ldexpf(__uint_as_float(u[2 * e2] << 16), -sh);
      const float a1 = __builtin_ldexpf(__uint_as_float(u[2 * e2] & 0xffff0000u), -sh);
      const float a2 = __builtin_ldexpf(__uint_as_float(u[2 * e2 + 1] << 16), -sh);
      const float a3 = __builtin_ldexpf(__uint_as_float(u[2 * e2 + 1] & 0xffff0000u), -sh);
      int hc = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
      hc = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, hc, true);
      const float r0 = (a0 - __builtin_amdgcn_cvt_f32_fp8(hc, 0)) * 16.0f;
      const float r1 = (a1 - __builtin_amdgcn_cvt_f32_fp8(hc, 1)) * 16.0f;
      const float r2 = (a2 - __builtin_amdgcn_cvt_f32_fp8(hc, 2)) * 16.0f;
      const float r3 = (a3 - __builtin_amdgcn_cvt_f32_fp8(hc, 3)) * 16.0f;
      int lc = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
      lc = __builtin_amdgcn_cvt_pk_fp8_f32(r2, r3, lc, true);
      hi[2 * j + e2] = (uint32_t)hc;
      lo[2 * j + e2] = (uint32_t)lc;
    }
  }
  return sh;
}

__device__ __forceinline__ i32x8 cat8(const i32x4 a, const i32x4 b) {
  return (i32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// q.k over 128 dimensions for one 32-head tile on the fp8 MFMA: hi and lo codes of
// the tile's two 32-dimension runs per lane; scale byte SEL and SEL + 1 of sh / sl
template <int SEL>
__device__ __forceinline__ f32x16 f8_dot(const i32x8 h0, const i32x8 h1, const i32x8 l0, const i32x8 l1,
                                         const i32x8 b0, const i32x8 b1, int sh, int sl) {
  f32x16 c = {};
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(h0, b0, c, 0, 0, SEL, sh, 0, 127);
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(h1, b1, c, 0, 0, SEL + 1, sh, 0, 127);
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(l0, b0, c, 0, 0, SEL, sl, 0, 127);
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(l1, b1, c, 0, 0, SEL + 1, sl, 0, 127);
  return c;
}

// Selection epilogue of the held-scores form (few long rows): the workgroup's
// scores (keys key0 .. key0 + n - 1, 16 per thread, entry e * 256 + tid) come from
// LDS into registers, go out to the score row, and are listed above a threshold of
// the workgroup's own (list_above_local_threshold) into its region of the candidate
// list (cval / cid at r S + key0), with its count, threshold and largest key.
constexpr int HELD_E = LT_E;  // held scores per thread: at most 4,096 per workgroup
typedef __attribute__((address_space(3))) float lds_f32;

__device__ __forceinline__ void held_select_epilogue(const float* held_g, int n, int r, int key0, int k,
                                                     float* __restrict__ out_row, uint32_t* __restrict__ bcnt,
                                                     float* __restrict__ cval, int32_t* __restrict__ cid,
                                                     uint32_t* __restrict__ tau_used, int S, uint8_t* scratch) {
  const lds_f32* held = (const lds_f32*)(uintptr_t)lds_addr(held_g);
  const int P = gridDim.x, tid = threadIdx.x;
  float v[HELD_E];
#pragma unroll
  for (int e = 0; e < HELD_E; ++e) v[e] = held[e * 256 + tid];
  // scores go out as streaming stores: nothing of them is left dirty in L2 for the
  // write-back at the end of the kernel
#pragma unroll
  for (int e = 0; e < HELD_E; ++e) {
    const int i = e * 256 + tid;
    if (i < n) __builtin_nontemporal_store(v[e], &out_row[key0 + i]);
  }
  list_above_local_threshold(v, n, k, P, (int)blockIdx.x, cval + (int64_t)r * S + key0, cid + (int64_t)r * S + key0,
                             key0, bcnt + (int64_t)r * P + blockIdx.x, tau_used + (int64_t)r * 256, scratch);
}

// PAGED: the keys (and scales) of every sequence live in pages of PAGE keys of a
// shared pool; page_table[b * max_pages + p] is the pool page holding keys
// PAGE p .. PAGE p + PAGE - 1 of sequence b ("Long context", section "Sparsity Is
// a Systems Feature: The Blast Radius", paragraph "KV-cache management": the
// indexer kernel reads its cache in pages of 64 keys).  A workgroup covers at most
// 64 pages: lane l holds the pool page of the workgroup's l-th page and each tile
// (32 keys, inside one page) takes its page by a lane read.  Page ids outside
// [0, num_pages) read page num_pages - 1 or 0 (clamped; no access leaves the pool).
constexpr int PAGE = 64;
constexpr int PAGED_MAX_KPB = 64 * PAGE;

template <int HT, bool FP8, int NST, int WPE, bool STG = false, bool PAGED = false, bool LSEL = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE)))
void score_stream_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w, const uint8_t* __restrict__ k,
                         const float* __restrict__ ks, const int32_t* __restrict__ nv, int T, int S, int H,
                         int keys_per_block, float* __restrict__ scores, int topk, uint32_t* __restrict__ bcnt,
                         float* __restrict__ cval, int32_t* __restrict__ cid, uint32_t* __restrict__ tau_used,
                         const int32_t* __restrict__ page_table, int max_pages, int num_pages) {
  static_assert(!PAGED || FP8, "paged keys are fp8");
  static_assert(!LSEL || STG, "the local selection runs on the held scores");
  typedef TileGeom<FP8> G;
  static_assert(NST >= 1 && NST <= 3, "ring depth");
  // STG: the workgroup's scores are held in LDS behind the ring and written in one
  // pass at the end (keys_per_block floats of dynamic LDS)
  constexpr bool STAGE = STG;
  // fp8: the query codes occupy the last SPL ring stages until every wave has
  // read its operands; those stages are filled after that
  constexpr int SPL = FP8 ? (QSplit<HT>::BYTES + 4 * G::BYTES - 1) / (4 * G::BYTES) : 0;
  static_assert(!FP8 || SPL <= NST, "query codes fit in the ring");
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

  const uint8_t* kbase = k + (PAGED ? 0 : (int64_t)b * S * G::ROW);
  const int vis_end = min(key_end, nvis);
  for (int key = max(key0, vis_end) + (int)threadIdx.x; key < key_end; key += 256) out_row[key] = -INFINITY;

  // LDS: the head weights (2 x HT x 16 floats), then the ring, stage-major: stage st
  // of wave w at ring0 + (st * 4 + w) * BYTES
  // (dynamic LDS starts at offset 0: the kernel has no static LDS; aligning the
  // offset, not the pointer, keeps every access to it an LDS instruction)
  uint8_t* ring = lds + ((2 * HT * 16 * sizeof(float) + 127) & ~(size_t)127);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t ring0 = lds_addr(ring);
  const uint32_t my_ring = ring0 + (uint32_t)(wave_u * G::BYTES);
  constexpr uint32_t SSTRIDE = 4 * G::BYTES;  // bytes between a wave's stages
  const uint32_t stage0 = ring0 + NST * SSTRIDE;  // held scores (STAGE)
  const float* sbase = ks + (PAGED ? 0 : (int64_t)b * S);
  // pool page of the workgroup's page `lane` (paged keys)
  int my_page = 0;
  if constexpr (PAGED) {
    const int pi = (key0 / PAGE) + lane;
    const int npg = min(max_pages, (S + PAGE - 1) / PAGE);
    const int v = pi < npg ? page_table[(int64_t)b * max_pages + pi] : 0;
    my_page = min(max(v, 0), num_pages - 1);
  }
  // key row and scale of the tile starting at key t
  auto tile_k = [&](int t) -> const uint8_t* {
    if constexpr (PAGED) {
      const int pg = __builtin_amdgcn_readlane(my_page, (t - key0) / PAGE);
      return kbase + ((int64_t)pg * PAGE + (t % PAGE)) * G::ROW;
    } else {
      return kbase + (int64_t)t * G::ROW;
    }
  };
  auto tile_s = [&](int t) -> const float* {
    if constexpr (PAGED) {
      const int pg = __builtin_amdgcn_readlane(my_page, (t - key0) / PAGE);
      return sbase + (int64_t)pg * PAGE + (t % PAGE);
    } else {
      return sbase + t;
    }
  };
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

  // head weights in accumulator row order per lane half (read as LDS broadcasts)
  if (threadIdx.x < 2 * HT * 16) {
    const int g = threadIdx.x >> 4, i = threadIdx.x & 15;
    const int hf2 = g / HT, t = g % HT;
    const int hh = t * 32 + (i & 3) + 8 * (i >> 2) + 4 * hf2;
    sw[(hf2 * HT + t) * 16 + i] = hh < H ? w[(int64_t)r * H + hh] : 0.0f;
  }

  // key of the tile of this wave's ring stage st in the prologue, or -1 for none
  auto pro_tile = [&](int st) -> int {
    const int t0 = first + st * step;
    return t0 < vis_end ? t0 : -1;
  };

  // A operand.  bf16: query heads t*32 + col, dims [64 hf, 64 hf + 64), from global.
  // fp8: hi / lo codes and scale bytes, through the block's split in LDS.
  bf16x8 a[FP8 ? 1 : HT][FP8 ? 1 : 8];
  i32x8 ahi[FP8 ? HT : 1][2], alo[FP8 ? HT : 1][2];
  int sch[(HT + 1) / 2], scl[(HT + 1) / 2];
  if constexpr (!FP8) {
    // weights written before any LDS DMA is in flight
    __syncthreads();
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int t0 = pro_tile(st);
      if (t0 >= 0)
        issue_tile<FP8>(tile_k(t0), tile_s(t0), my_ring + st * SSTRIDE, goff, lane, min(32, S - t0));
    }
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
  } else {
    // query runs (thread = head x run of 32 dimensions) loaded before the first
    // tiles' DMA so their wait does not cover it
    // run (kk, kb) of head h: dimensions 32 kk + 16 kb + [0, 16) and 64 + that
    constexpr int RUNS = (HT * 128 + 255) / 256;
    uint4 qv[RUNS][4];
#pragma unroll
    for (int u = 0; u < RUNS; ++u) {
      const int id = (int)threadIdx.x + 256 * u;
      const int h = id >> 2, run = id & 3;
      const bool ok = id < HT * 128 && h < H;
      const uint4* qp = (const uint4*)(q + ((int64_t)r * H + (ok ? h : 0)) * 128 + 16 * run);
      qv[u][0] = ok ? qp[0] : make_uint4(0, 0, 0, 0);
      qv[u][1] = ok ? qp[1] : make_uint4(0, 0, 0, 0);
      qv[u][2] = ok ? qp[8] : make_uint4(0, 0, 0, 0);
      qv[u][3] = ok ? qp[9] : make_uint4(0, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NST - SPL; ++st) {
      const int t0 = pro_tile(st);
      if (t0 >= 0)
        issue_tile<FP8>(tile_k(t0), tile_s(t0), my_ring + st * SSTRIDE, goff, lane, min(32, S - t0));
    }
    uint8_t* split = ring + (NST - SPL) * SSTRIDE;
#pragma unroll
    for (int u = 0; u < RUNS; ++u) {
      const int id = (int)threadIdx.x + 256 * u;
      if (id < HT * 128) {
        const int h = id >> 2, run = id & 3;
        const int t = h >> 5, c = h & 31, kk = run >> 1, kb = run & 1;
        uint32_t hi[8], lo[8];
        const int sh = split_run(qv[u], hi, lo);
        // first 16 codes: lane (0, c); last 16: lane (1, c); bytes [16 kb, 16 kb + 16)
        const int slot0 = ((t * 2 + kk) * 2 + 0) * 32 + c, slot1 = slot0 + 32;
        *(uint4*)(split + QSplit<HT>::HI + slot0 * 32 + 16 * kb) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *(uint4*)(split + QSplit<HT>::HI + slot1 * 32 + 16 * kb) = make_uint4(hi[4], hi[5], hi[6], hi[7]);
        *(uint4*)(split + QSplit<HT>::LO + slot0 * 32 + 16 * kb) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        *(uint4*)(split + QSplit<HT>::LO + slot1 * 32 + 16 * kb) = make_uint4(lo[4], lo[5], lo[6], lo[7]);
        // the scale of block kb comes from lane half kb
        split[QSplit<HT>::SC + (kb * 32 + c) * (2 * HT) + t * 2 + kk] = (uint8_t)(127 + sh);
      }
    }
    lds_barrier();
#pragma unroll
    for (int t = 0; t < HT; ++t)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int slot = ((t * 2 + kk) * 2 + hf) * 32 + col;
        const i32x4* ph = (const i32x4*)(split + QSplit<HT>::HI + slot * 32);
        const i32x4* pl = (const i32x4*)(split + QSplit<HT>::LO + slot * 32);
        ahi[t][kk] = cat8(ph[0], ph[1]);
        alo[t][kk] = cat8(pl[0], pl[1]);
      }
    const uint8_t* psc = split + QSplit<HT>::SC + (hf * 32 + col) * (2 * HT);
#pragma unroll
    for (int p2 = 0; p2 < (HT + 1) / 2; ++p2) {
      // bytes (2 p2 + t') * 2 + kk of the lane's scale record, one word per head pair;
      // the lo scale is the hi scale / 2^4 in every byte (no byte is below 5)
      sch[p2] = HT == 1 ? (int)*(const uint16_t*)psc : ((const int*)psc)[p2];
      scl[p2] = sch[p2] - (HT == 1 ? 0x0404 : 0x04040404);
    }
    lds_barrier();
#pragma unroll
    for (int st = NST - SPL; st < NST; ++st) {
      const int t0 = pro_tile(st);
      if (t0 >= 0)
        issue_tile<FP8>(tile_k(t0), tile_s(t0), my_ring + st * SSTRIDE, goff, lane, min(32, S - t0));
    }
  }

  // ReLU x weight head sum of the tile in raw[] (lanes 0..31 end with the key's total)
#define LI_TILE_PART() \
  do { \
    f32x16 acc[HT]; \
    if constexpr (FP8) { \
      const i32x8 b0 = cat8(raw[0], raw[1]), b1 = cat8(raw[2], raw[3]); \
      acc[0] = f8_dot<0>(ahi[0][0], ahi[0][1], alo[0][0], alo[0][1], b0, b1, sch[0], scl[0]); \
      if constexpr (HT >= 2) acc[1] = f8_dot<2>(ahi[1][0], ahi[1][1], alo[1][0], alo[1][1], b0, b1, sch[0], scl[0]); \
      if constexpr (HT >= 4) { \
        acc[HT - 2] = f8_dot<0>(ahi[HT - 2][0], ahi[HT - 2][1], alo[HT - 2][0], alo[HT - 2][1], b0, b1, \
                                sch[(HT - 1) / 2], scl[(HT - 1) / 2]); \
        acc[HT - 1] = f8_dot<2>(ahi[HT - 1][0], ahi[HT - 1][1], alo[HT - 1][0], alo[HT - 1][1], b0, b1, \
                                sch[(HT - 1) / 2], scl[(HT - 1) / 2]); \
      } \
    } else { \
_Pragma("unroll") \
      for (int t = 0; t < HT; ++t) { \
        f32x16 c = {}; \
_Pragma("unroll") \
        for (int kk = 0; kk < 8; ++kk) \
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t][kk], __builtin_bit_cast(bf16x8, raw[kk]), c, 0, 0, 0); \
        acc[t] = c; \
      } \
    } \
    part = 0.0f; \
_Pragma("unroll") \
    for (int t = 0; t < HT; ++t) { \
      /* weights via the asm read as well: a compiler-visible LDS read here would */ \
      /* be made to wait for every outstanding key load */ \
      const uint32_t wa = lds_addr(&sw[(hf * HT + t) * 16]); \
      i32x4 wr[4]; \
      lds_read4(wr[0], wr[1], wr[2], wr[3], wa, wa + 16, wa + 32, wa + 48); \
_Pragma("unroll") \
      for (int i4 = 0; i4 < 4; ++i4) { \
_Pragma("unroll") \
        for (int e = 0; e < 4; ++e) part = fmaf(__int_as_float(wr[i4][e]), relu_bits(acc[t][4 * i4 + e]), part); \
      } \
    } \
    /* lanes 0..31 add the partial sum of lanes 32..63 (same key, other heads) */ \
    part += __uint_as_float(__builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, \
                                                             false)[1]); \
  } while (0)
  int stage = 0, iter = 0;
  for (int tile = first; tile < vis_end; tile += step) {
    // vmcnt counts loads and stores in issue order.  Issued after this tile's
    // loads: the loads of the n_after younger tiles (OPS instructions each) and
    // the score stores of the last min(iter, NST) iterations (one each; none when
    // the scores are held in LDS), so this tile has landed once no more than that
    // many are outstanding.
    const int n_after = min(NST - 1, (vis_end - 1 - tile) / step);
    wait_vmcnt(n_after * OPS + (STAGE ? 0 : min(iter, NST)));
    ++iter;
    const uint32_t la = my_ring + (uint32_t)(stage * SSTRIDE);
    const int key = tile + col;
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
    if (tn < vis_end) issue_tile<FP8>(tile_k(tn), tile_s(tn), la, goff, lane, min(32, S - tn));
    stage = stage + 1 == NST ? 0 : stage + 1;
    float part;
    LI_TILE_PART();
    if (hf == 0 && key < key_end) {
      const float v = key < nvis ? part * sc : -INFINITY;
      if (STAGE)  // written out to LDS (no compiler-visible LDS access beside the ring's loads)
        asm volatile("ds_write_b32 %0, %1" : : "v"(stage0 + 4u * (uint32_t)(key - key0)), "v"(v) : "memory");
      else
        __builtin_nontemporal_store(v, &out_row[key]);
    }
  }
  if constexpr (STAGE) {
    // every load has landed; the held scores of keys key0 .. vis_end - 1 go out in
    // one coalesced pass (the keys past vis_end were written -inf at the start).
    // The held scores were written by inline ds_write, which the compiler's wait
    // tracking does not see: wait for them here, before the barrier.
    LI_WAIT_VMCNT(0);
    LI_WAIT_LGKM0();
    __syncthreads();
    const float* held = (const float*)(ring + NST * SSTRIDE);
    const int n = vis_end - key0;
    if constexpr (LSEL) {
      // the ring is free: its LDS holds the selection's thresholds and counts
      held_select_epilogue(held, max(n, 0), r, key0, topk, out_row, bcnt, cval, cid, tau_used, S, ring);
    } else {
      for (int i = (int)threadIdx.x; i < n; i += 256) __builtin_nontemporal_store(held[i], &out_row[key0 + i]);
    }
  }
#undef LI_TILE_PART
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

// Keys per workgroup of the staged form (its scores are held in LDS): 16 KB.
constexpr int STAGE_KEYS = 4096;
static_assert(STAGE_KEYS == HELD_E * 256, "the held-scores selection covers the whole staged block");

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

// Generic fp32 path (fp32 queries or keys): a quad of lanes per key, fp32 FMAs,
// the query row staged in LDS.  Lane g accumulates dimensions 32 g .. 32 g + 31 of
// four heads at a time in ascending order; the quad's partial dots are summed as
// (p0 + p1) + (p2 + p3), the head sum runs over h in ascending order, then the key
// scale.  The order is fixed, so results are deterministic.
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
  // a quad of lanes per key: lane g holds dimensions 32 g .. 32 g + 31
  const int g = threadIdx.x & 3;
  const int s = blockIdx.x * 64 + (threadIdx.x >> 2);
  int nvis = S;
  if (nv) nvis = min(max(nv[r], 0), S);
  const int64_t row = (int64_t)b * S + min(s, S - 1);
  float kv[32];
  if constexpr (KT == 0) {
    const float4* kp = (const float4*)((const float*)k + row * 128 + 32 * g);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 v = kp[j];
      kv[4 * j] = v.x; kv[4 * j + 1] = v.y; kv[4 * j + 2] = v.z; kv[4 * j + 3] = v.w;
    }
  } else if constexpr (KT == 1) {
    const uint4* kp = (const uint4*)((const uint16_t*)k + row * 128 + 32 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = kp[j];
      const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv[8 * j + 2 * e] = __uint_as_float(x[e] << 16);
        kv[8 * j + 2 * e + 1] = __uint_as_float(x[e] & 0xFFFF0000u);
      }
    }
  } else {
    const uint4* kp = (const uint4*)((const uint8_t*)k + row * 128 + 32 * g);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint4 v = kp[j];
      const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8(x[e], false);
        const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8(x[e], true);
        kv[16 * j + 4 * e] = p0[0]; kv[16 * j + 4 * e + 1] = p0[1];
        kv[16 * j + 4 * e + 2] = p1[0]; kv[16 * j + 4 * e + 3] = p1[1];
      }
    }
  }
  // the quad's four partial dots of a head, summed as (p0 + p1) + (p2 + p3) in every lane
  auto quad_sum = [](float x) {
    x += __shfl_xor(x, 1, WAVE);
    return x + __shfl_xor(x, 2, WAVE);
  };
  const float* qs = sq + 32 * g;
  float acc = 0.0f;
  int h = 0;
  for (; h + 4 <= H; h += 4) {  // four heads' chains at a time
    float d0 = 0.0f, d1 = 0.0f, d2 = 0.0f, d3 = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      d0 = fmaf(qs[h * 128 + j], kv[j], d0);
      d1 = fmaf(qs[(h + 1) * 128 + j], kv[j], d1);
      d2 = fmaf(qs[(h + 2) * 128 + j], kv[j], d2);
      d3 = fmaf(qs[(h + 3) * 128 + j], kv[j], d3);
    }
    d0 = quad_sum(d0); d1 = quad_sum(d1); d2 = quad_sum(d2); d3 = quad_sum(d3);
    acc = fmaf(sq[H * 128 + h], fmaxf(d0, 0.0f), acc);
    acc = fmaf(sq[H * 128 + h + 1], fmaxf(d1, 0.0f), acc);
    acc = fmaf(sq[H * 128 + h + 2], fmaxf(d2, 0.0f), acc);
    acc = fmaf(sq[H * 128 + h + 3], fmaxf(d3, 0.0f), acc);
  }
  for (; h < H; ++h) {
    float d0 = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) d0 = fmaf(qs[h * 128 + j], kv[j], d0);
    d0 = quad_sum(d0);
    acc = fmaf(sq[H * 128 + h], fmaxf(d0, 0.0f), acc);
  }
  if (ks) acc *= ks[row];
  if (g == 0 && s < S) scores[(int64_t)r * S + s] = s < nvis ? acc : -INFINITY;
}

// One launch of the streaming kernel.  STG: scores held in LDS (two workgroups per
// CU, at most STAGE_KEYS keys each); PAGED: keys in pool pages (at most
// PAGED_MAX_KPB keys per workgroup).
template <int HT, bool F8, bool STG, bool PAGED>
static hipError_t launch_stream(const uint16_t* qq, const float* w, const uint8_t* kk, const float* ks,
                                const int32_t* nv, int R, int T, int S, int H, float* scores,
                                const int32_t* page_table, int max_pages, int num_pages, hipStream_t st) {
  typedef StreamCfg<HT, F8> C;
  auto kern = score_stream_kernel<HT, F8, C::NST, STG ? 2 : C::WPE, STG, PAGED>;
  int kpb = stream_keys_per_block(R, S, STG ? 2 : C::BPC);
  if (STG) kpb = std::min(kpb, STAGE_KEYS);
  if (PAGED) kpb = std::min(kpb, PAGED_MAX_KPB);
  const size_t lds = stream_lds_bytes<HT, F8>() + (STG ? (size_t)kpb * sizeof(float) : 0);
  static const bool attr = [&] {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(stream_lds_bytes<HT, F8>() + (STG ? STAGE_KEYS * sizeof(float) : 0)));
    return true;
  }();
  (void)attr;
  dim3 grid((S + kpb - 1) / kpb, R);
  kern<<<grid, 256, lds, st>>>(qq, w, kk, ks, nv, T, S, H, kpb, scores, 0, nullptr, nullptr, nullptr, nullptr,
                               page_table, max_pages, num_pages);
  return hipGetLastError();
}

// fp8 keys at up to 64 heads hold their scores in LDS and write them once per
// workgroup: writes interleaved with the key stream cost several times their bytes
template <bool PAGED>
static hipError_t launch_stream_fp8(const uint16_t* qq, const float* w, const uint8_t* kk, const float* ks,
                                    const int32_t* nv, int R, int T, int S, int H, float* scores,
                                    const int32_t* page_table, int max_pages, int num_pages, hipStream_t st) {
  // up to 64 heads one kernel: with 32 heads or fewer the second head tile has zero
  // weights (its MFMAs are hidden under the key stream, and the held-scores form
  // streams faster than the 32-head one)
  if (H <= 64)
    return launch_stream<2, true, true, PAGED>(qq, w, kk, ks, nv, R, T, S, H, scores, page_table, max_pages,
                                               num_pages, st);
  return launch_stream<4, true, false, PAGED>(qq, w, kk, ks, nv, R, T, S, H, scores, page_table, max_pages,
                                              num_pages, st);
}

hipError_t launch_score_paged(const uint16_t* q, const float* w, const uint8_t* k_pool, const float* ks_pool,
                              const int32_t* page_table, int max_pages, int num_pages, const int32_t* nv, int B,
                              int T, int S, int H, float* scores, hipStream_t st) {
  return launch_stream_fp8<true>(q, w, k_pool, ks_pool, nv, B * T, T, S, H, scores, page_table, max_pages,
                                 num_pages, st);
}

hipError_t launch_score(const void* q, int q_type, const float* w, const void* k, int k_type, const float* ks,
                        const int32_t* nv, int B, int T, int S, int H, float* scores, hipStream_t st) {
  const int R = B * T;
  if (prefill_scores_apply(q_type, k_type, T, H))
    return launch_prefill_scores((const uint16_t*)q, w, k, k_type, ks, nv, B, T, S, H, scores, st);
  if (q_type == DT_BF16 && (k_type == DT_FP8 || k_type == DT_BF16)) {
    const uint16_t* qq = (const uint16_t*)q;
    const uint8_t* kk = (const uint8_t*)k;
    if (k_type == DT_FP8) return launch_stream_fp8<false>(qq, w, kk, ks, nv, R, T, S, H, scores, nullptr, 0, 0, st);
    if (H <= 32) return launch_stream<1, false, false, false>(qq, w, kk, ks, nv, R, T, S, H, scores, nullptr, 0, 0, st);
    if (H <= 64) return launch_stream<2, false, false, false>(qq, w, kk, ks, nv, R, T, S, H, scores, nullptr, 0, 0, st);
    return launch_stream<4, false, false, false>(qq, w, kk, ks, nv, R, T, S, H, scores, nullptr, 0, 0, st);
  }
  dim3 grid((S + 63) / 64, R);  // 64 keys a workgroup, a quad of lanes each
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

// Few long rows with fp8 keys and at most 64 heads: the held-scores kernel with the
// workgroup-local selection epilogue, then the finalize.
bool held_select_apply(int q_type, int k_type, int R, int S, int H, int topk) {
  if (q_type != DT_BF16 || k_type != DT_FP8 || H < 1 || H > 64) return false;
  if (!topk_use_mb(R, S) || topk > 2048) return false;
  const int kpb = std::min(stream_keys_per_block(R, S, 2), STAGE_KEYS);
  const int P = (S + kpb - 1) / kpb;
  return P <= 256 && kpb >= 1024 && kpb <= HELD_E * 256;
}

template <bool PAGED>
static hipError_t launch_held_select(const uint16_t* qq, const float* w, const uint8_t* kk, const float* ks,
                                     const int32_t* nv, int R, int T, int S, int H, int topk, float* scores,
                                     uint32_t* bcnt, float* cval, int32_t* cid, uint32_t* tau_used, int* P_out,
                                     int* chunk_out, const int32_t* page_table, int max_pages, int num_pages,
                                     hipStream_t st) {
  typedef StreamCfg<2, true> C;
  auto kern = score_stream_kernel<2, true, C::NST, 2, true, PAGED, true>;
  const int kpb = std::min(stream_keys_per_block(R, S, 2), STAGE_KEYS);
  // the epilogue reads all HELD_E * 256 held slots (those past the block's keys
  // are masked), so the held area is always allocated whole
  const size_t lds = stream_lds_bytes<2, true>() + (size_t)HELD_E * 256 * sizeof(float);
  static const bool attr = [&] {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    return true;
  }();
  (void)attr;
  const int P = (S + kpb - 1) / kpb;
  *P_out = P;
  *chunk_out = kpb;
  kern<<<dim3(P, R), 256, lds, st>>>(qq, w, kk, ks, nv, T, S, H, kpb, scores, topk, bcnt, cval, cid, tau_used,
                                     page_table, max_pages, num_pages);
  return hipGetLastError();
}

hipError_t launch_score_held_select(const void* q, const float* w, const void* k, const float* ks, const int32_t* nv,
                                    int B, int T, int S, int H, int topk, float* scores, uint32_t* bcnt, float* cval,
                                    int32_t* cid, uint32_t* tau_used, int* P_out, int* chunk_out, hipStream_t st,
                                    const int32_t* page_table, int max_pages, int num_pages) {
  if (page_table)
    return launch_held_select<true>((const uint16_t*)q, w, (const uint8_t*)k, ks, nv, B * T, T, S, H, topk, scores,
                                    bcnt, cval, cid, tau_used, P_out, chunk_out, page_table, max_pages, num_pages,
                                    st);
  return launch_held_select<false>((const uint16_t*)q, w, (const uint8_t*)k, ks, nv, B * T, T, S, H, topk, scores,
                                   bcnt, cval, cid, tau_used, P_out, chunk_out, nullptr, 0, 0, st);
}


}  // namespace li
