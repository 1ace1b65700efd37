// Scoring followed by per-row selection.
//
// For a prefill chunk (many query rows against the same keys) the selection runs
// inside the scoring kernel, so the [rows, S] score matrix is never written:
// "Latent Sparse Attention" article, section "What the kernels do about the
// top-p" (the score matrix of a prefill chunk is never written to memory; each
// score is compared with a threshold as it comes off the matrix cores and only
// the entries above it are listed).  Score: "Long context", llm-serving.xyz
// lecture 03, section "The Architectural Answer", paragraph "Stage 1, the
// lightning indexer".
//
// prefill_select_kernel: a workgroup owns 8 query rows of one sequence, one per
// wave; each wave keeps its query block (H x 128 bf16) in VGPRs as the MFMA A
// operand.  The workgroup streams every visible key of the sequence through LDS
// in 128-key bf16 tiles (double buffered, loaded cooperatively, XOR-swizzled so
// the operand reads are conflict free); each wave scores each 32-key sub-tile
// with 16 v_mfma_f32_32x32x16_bf16 (64 heads) and reduces ReLU x weight over the
// heads in registers.  fp8 keys (E4M3 codes + one fp32 scale per key, the
// indexer's FP8 key cache of "Long context", "The Architectural Answer",
// Derivation 4) are read as stored, widened to bf16 on their way into LDS (exact:
// every E4M3 value is a bf16 value), and the key's scale multiplies the head sum
// (it is positive, so it commutes with the ReLU).  Selection per row: a running threshold theta (the current
// k-th best) and a candidate list of CAP entries in LDS kept in key-index order.
// A score is listed when it beats theta; when the list is full the wave compacts
// it to the exact current top-k (bisection on the orderable score bits for the
// k-th value, ties to the smaller index, order-preserving) and raises theta.
// Keys arrive in increasing index order, so an entry equal to theta loses its
// tie and a strict comparison is exact.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace li {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int PS_WAVES = 8;    // query rows per workgroup
constexpr int PS_NK = 128;     // keys per LDS tile
constexpr int PS_CPT = PS_NK * 16 / (PS_WAVES * 64);  // 16-byte chunks per thread per tile
constexpr int PS_CAP = 1024;   // candidate list entries per row
constexpr int PS_KMAX = 512;   // largest k the fused kernel takes (CAP - NK - k >= 384)

// max(x, 0) on the bit pattern (exact, -0 -> +0).
__device__ __forceinline__ float relu_bits_f(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// part + w * x, where w is the value that lane i of this lane's row of 16 holds in
// wb (DPP row_newbcast on the fma's first source): one VGPR carries 16 weights per
// lane row.  Every lane of the wave must be active (a disabled source lane would
// leave part unchanged); i is a constant once the callers' loops are unrolled.
__device__ __forceinline__ float fmac_bcast(float part, float wb, float x, int i) {
#define LI_FMAC_B(n)                                                                              \
  case n:                                                                                         \
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:" #n " row_mask:0xf bank_mask:0xf"               \
        : "+v"(part) : "v"(wb), "v"(x));                                                          \
    break;
  switch (i) {
    LI_FMAC_B(0) LI_FMAC_B(1) LI_FMAC_B(2) LI_FMAC_B(3) LI_FMAC_B(4) LI_FMAC_B(5) LI_FMAC_B(6) LI_FMAC_B(7)
    LI_FMAC_B(8) LI_FMAC_B(9) LI_FMAC_B(10) LI_FMAC_B(11) LI_FMAC_B(12) LI_FMAC_B(13) LI_FMAC_B(14) LI_FMAC_B(15)
  }
#undef LI_FMAC_B
  return part;
}

// hist[d] += 1 for every lane with valid set (one wave, LDS atomics); when all
// such lanes share one digit a single atomic adds them.
__device__ __forceinline__ void wave_hist_add(uint32_t* hist, uint32_t d, bool valid) {
  const uint64_t act = __ballot(valid);
  if (!act) return;
  const int first = __ffsll((unsigned long long)act) - 1;
  const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)d, first);  // first is wave-uniform
  if (__ballot(valid && d == d0) == act) {
    if ((int)(threadIdx.x & 63) == first) atomicAdd(&hist[d0], (uint32_t)__popcll(act));
  } else if (valid) {
    atomicAdd(&hist[d], 1u);
  }
}

// Wave-level exact compaction of a candidate list (entries [0, cnt) in index
// order, orderable keys in sk, ids in si) to its best `keep` entries, preserving
// order.  Returns the orderable key T of the worst kept entry.  T comes from a
// radix select (four 8-bit digits, the wave's own 256-bin histogram hw in LDS).
// Lane l handles entries l + 64 e, so the rank of an entry among the kept ones
// is a ballot prefix: rows e' < e, then lanes below l.
__device__ uint32_t ps_compact(uint32_t* sk, int32_t* si, uint32_t* hw, int cnt, int keep) {
  constexpr int E = PS_CAP / 64;
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1;
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = lane + 64 * e < cnt ? sk[lane + 64 * e] : 0u;
  // T: the keep-th largest listed key, digit by digit from the top
  uint32_t prefix = 0u, mask = 0u;
  uint32_t need = (uint32_t)keep;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int shift = 24 - 8 * p;
    *(uint4*)&hw[4 * lane] = make_uint4(0u, 0u, 0u, 0u);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int e = 0; e < E; ++e)
      wave_hist_add(hw, (key[e] >> shift) & 255u, lane + 64 * e < cnt && (key[e] & mask) == prefix);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // lane l holds digits 255 - 4 l .. 252 - 4 l, counted from the top
    const uint4 c4 = *(const uint4*)&hw[252 - 4 * lane];  // digits 252-4l .. 255-4l
    const uint32_t cs = c4.x + c4.y + c4.z + c4.w;
    const uint32_t incl = wave_incl_scan(cs), excl = incl - cs;
    const uint64_t hit = __ballot(excl < need && need <= incl);
    const int hl = __ffsll((unsigned long long)hit) - 1;
    // inside the hit lane: digits 255-4l (c4.w) down to 252-4l (c4.x)
    uint32_t d = 0u, above = excl;
    if (need <= excl + c4.w) {
      d = 255u - 4u * (uint32_t)lane;
    } else if (need <= excl + c4.w + c4.z) {
      d = 254u - 4u * (uint32_t)lane; above = excl + c4.w;
    } else if (need <= excl + c4.w + c4.z + c4.y) {
      d = 253u - 4u * (uint32_t)lane; above = excl + c4.w + c4.z;
    } else {
      d = 252u - 4u * (uint32_t)lane; above = excl + c4.w + c4.z + c4.y;
    }
    const uint32_t dd = (uint32_t)__builtin_amdgcn_readlane((int)d, hl);
    const uint32_t ab = (uint32_t)__builtin_amdgcn_readlane((int)above, hl);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    prefix |= dd << shift;
    mask |= 255u << shift;
    need -= ab;
  }
  const uint32_t T = prefix;
  int gt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) gt += __popcll(__ballot(lane + 64 * e < cnt && key[e] > T));
  const int need_ties = keep - gt;  // entries equal to T to keep, smallest index first
  // a kept entry moves to its rank, never above its own position: the writes of
  // row e land in rows <= e, and row e is read before it is written
  int base = 0, tbase = 0;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane + 64 * e;
    const bool valid = j < cnt;
    const bool tie = valid && key[e] == T;
    const uint64_t mt = __ballot(tie);
    const bool sel = (valid && key[e] > T) || (tie && tbase + __popcll(mt & below) < need_ties);
    tbase += __popcll(mt);
    const uint64_t ms = __ballot(sel);
    const int32_t id = valid ? si[j] : 0;
    if (sel) {
      const int pos = base + __popcll(ms & below);
      sk[pos] = key[e];
      si[pos] = id;
    }
    base += __popcll(ms);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  return T;
}

// Eight key elements into the bf16 LDS tile: bf16 chunks as they are; eight E4M3
// codes widened exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1), element e of
// the chunk from byte e.
__device__ __forceinline__ uint4 widen(const uint4 v) { return v; }
__device__ __forceinline__ uint4 widen(const uint2 v) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                    __builtin_bit_cast(uint32_t, d));
}

// SCORES: write every score to scores [B*T, S] (masked keys -inf) instead of
// selecting (the same contraction for li_indexer_score at prefill shapes).
template <int HT, bool SCORES, bool F8K = false>
__global__ __launch_bounds__(PS_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_select_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                           const void* __restrict__ k, const float* __restrict__ ks, const int32_t* __restrict__ nv,
                           int T, int S, int H, int topk, int32_t* __restrict__ idx_out, float* __restrict__ val_out,
                           float* __restrict__ scores) {
  // LDS: two key tiles (64 keys x 256 B, 16-byte chunks XOR-swizzled by key),
  // then per wave a candidate list (orderable keys, ids)
  __shared__ __attribute__((aligned(16))) uint8_t tiles[2][PS_NK * 256];
  __shared__ uint32_t cand_k[PS_WAVES][PS_CAP];
  __shared__ int32_t cand_i[PS_WAVES][PS_CAP];
  __shared__ __attribute__((aligned(16))) uint32_t whist[PS_WAVES][256];  // compaction histograms

  const int blocks_per_seq = (T + PS_WAVES - 1) / PS_WAVES;
  const int b = blockIdx.x / blocks_per_seq;
  const int t0 = (blockIdx.x % blocks_per_seq) * PS_WAVES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, col = lane & 31;
  const int t = t0 + wave;
  const bool active = t < T;
  const int64_t r = (int64_t)b * T + (active ? t : t0);
  int nvis = S;
  if (nv) nvis = min(max(nv[r], 0), S);
  if (!active) nvis = 0;
  nvis = __builtin_amdgcn_readfirstlane(nvis);  // one row per wave: uniform

  // keys needed by the workgroup: the largest visible count of its rows
  __shared__ int s_kend;
  if (tid == 0) s_kend = 0;
  __syncthreads();
  if (lane == 0) atomicMax(&s_kend, nvis);
  __syncthreads();
  const int kend = s_kend;

  // query block (A operand) and head weights in accumulator row order: register i
  // of a 32 x 32 accumulator holds head 32 ht + (i & 3) + 8 (i >> 2) + 4 hf.  Up to
  // 64 heads every lane keeps its 16 weights per head tile (wv); at 128 heads they
  // would not fit beside the query block, so lane n of each row of 16 keeps the
  // weight of register n for its lane half (wb) and the reduction broadcasts it.
  constexpr bool WB = HT > 2;
  constexpr int NW = WB ? 1 : 16;
  bf16x8 a[HT][8];
  float wv[HT][NW];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int h = ht * 32 + col;
    const uint4* qp = (const uint4*)(q + (r * H + (h < H ? h : 0)) * 128 + 64 * hf);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint4 v = (h < H && active) ? qp[kk] : make_uint4(0, 0, 0, 0);
      a[ht][kk] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int n = WB ? (lane & 15) : i;
      const int hh = ht * 32 + (n & 3) + 8 * (n >> 2) + 4 * hf;
      wv[ht][i] = (hh < H && active) ? w[r * H + hh] : 0.0f;
    }
  }

  // key rows: 256 bytes (bf16) or 128 bytes (fp8 codes) each
  const uint8_t* kbase = (const uint8_t*)k + (int64_t)b * S * (F8K ? 128 : 256);
  const float* sbase = F8K ? ks + (int64_t)b * S : nullptr;
  // cooperative tile load: thread tid moves the 16-byte chunks
  // c = tid + 512 j (key c >> 4, chunk c & 15)
  static_assert(PS_NK * 16 == PS_CPT * PS_WAVES * 64, "whole chunks per thread");
  const int cn0 = tid >> 4, cc = tid & 15;  // key of chunk j: cn0 + 32 j
  constexpr int KSTEP = PS_WAVES * 64 / 16;

  uint32_t* sk = cand_k[wave];
  int32_t* si = cand_i[wave];
  int cnt = 0;                 // listed entries
  float theta_f = -INFINITY;   // score to beat (every finite score beats it at first)

  const int ntiles = (kend + PS_NK - 1) / PS_NK;
  // four named registers, not an array: an array here is kept in scratch memory.
  // A chunk is 8 key elements: 16 bytes of a bf16 row, 8 bytes of an fp8 row.
  static_assert(PS_CPT == 4, "chunk registers below");
  typedef typename std::conditional<F8K, uint2, uint4>::type chunk_t;
  chunk_t reg0, reg1, reg2, reg3;
#define PS_LOAD(j, key0) \
  reg##j = *(const chunk_t*)(kbase + (int64_t)min((key0) + cn0 + KSTEP * j, S - 1) * (F8K ? 128 : 256) + \
                             cc * (F8K ? 8 : 16))
#define PS_STORE(j, buf) \
  *(uint4*)((buf) + (cn0 + KSTEP * j) * 256 + ((cc ^ ((cn0 + KSTEP * j) & 15)) << 4)) = widen(reg##j)
  // scales of this lane's keys of a tile: kt + lane and kt + 64 + lane (the keys
  // whose scores it holds when a pair of sub-tiles leaves)
  float scA = 1.0f, scB = 1.0f, nscA = 1.0f, nscB = 1.0f;
  auto load_scales = [&](int kt, float& a, float& b2) {
    if constexpr (F8K) {
      a = sbase[min(kt + lane, S - 1)];
      b2 = sbase[min(kt + 64 + lane, S - 1)];
    }
  };
  if (ntiles > 0) {
    PS_LOAD(0, 0); PS_LOAD(1, 0); PS_LOAD(2, 0); PS_LOAD(3, 0);
    load_scales(0, scA, scB);
    PS_STORE(0, tiles[0]); PS_STORE(1, tiles[0]); PS_STORE(2, tiles[0]); PS_STORE(3, tiles[0]);
  }
  // every load issued so far (query block, weights, first tile) has landed: the
  // loop then only waits on its own next-tile loads where they are stored
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  __syncthreads();
  constexpr bool PIPE = HT <= 2;
  constexpr int NS = PS_NK / 32;
  bf16x8 bop[8];
#define PS_BOP(sub, buf)                                                                                        \
  do {                                                                                                          \
    const int n_ = 32 * (sub) + col;                                                                            \
    _Pragma("unroll") for (int kk = 0; kk < 8; ++kk) bop[kk] =                                                  \
        __builtin_bit_cast(bf16x8, *(const uint4*)((buf) + n_ * 256 + (((8 * hf + kk) ^ (n_ & 15)) << 4)));     \
  } while (0)
#define PS_MMA(slot, ht, aset)                                                                                  \
  do {                                                                                                          \
    acc[slot][ht] = f32x16{};                                                                                   \
    _Pragma("unroll") for (int kk = 0; kk < 8; ++kk) acc[slot][ht] =                                            \
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[aset][kk], bop[kk], acc[slot][ht], 0, 0, 0);                  \
  } while (0)
// ReLU x weight over this lane's heads of one accumulator slot: the partial sum of
// the lane half's heads (the other half's comes in at emission)
#define PS_RED(part, slot)                                                                                      \
  do {                                                                                                          \
    _Pragma("unroll") for (int ht = 0; ht < HT; ++ht)                                                           \
      _Pragma("unroll") for (int i = 0; i < 16; ++i) part = fmaf(wv[ht][i], relu_bits_f(acc[slot][ht][i]), part); \
  } while (0)
// The MFMAs of one sub-tile into slot ns (both head tiles' chains alternating),
// each followed by two ReLU x weight steps of the sub-tile held in slot os, in
// this order: the reduction runs while the matrix cores work.
#define PS_MMA_RED(ns, os, part)                                                                                \
  do {                                                                                                          \
    _Pragma("unroll") for (int ht = 0; ht < HT; ++ht) acc[ns][ht] = f32x16{};                                   \
    _Pragma("unroll") for (int kk = 0; kk < 8; ++kk) {                                                          \
      _Pragma("unroll") for (int ht = 0; ht < HT; ++ht) {                                                       \
        acc[ns][ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ht][kk], bop[kk], acc[ns][ht], 0, 0, 0);        \
        _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                                         \
          const int e_ = 2 * (HT * kk + ht) + j;                                                                \
          part = fmaf(wv[e_ >> 4][e_ & 15], relu_bits_f(acc[os][e_ >> 4][e_ & 15]), part);                      \
        }                                                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                                      \
      }                                                                                                         \
    }                                                                                                           \
  } while (0)
  // Sub-tiles s and s + 1 (s even) leave together: pa / pb hold each lane half's
  // partial sums of their keys, and one lane-half swap gives lane l the score of
  // key kt + 32 s + l (sub-tile s in lanes 0..31, s + 1 in lanes 32..63), which
  // is written out, or listed when it beats theta (compared as floats: -0 and +0
  // are equal as in the orderable image; lanes ascend with the key, so the list
  // stays in index order).
  auto emit2 = [&](int kt, int s, float pa, float pb, float sc) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pa), __float_as_uint(pb), false, false);
    float v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if constexpr (F8K) v *= sc;
    const int key = kt + 32 * s + lane;
    if constexpr (SCORES) {
      if (active && key < kend) scores[r * S + key] = key < nvis ? v : -INFINITY;
    } else {
      const uint64_t mk = __ballot(key < nvis && v > theta_f);
      if (mk) {
        if ((mk >> lane) & 1ull) {
          const int pos = cnt + __popcll(mk & ((1ull << lane) - 1));
          sk[pos] = ord_f32(v);
          si[pos] = key;
        }
        cnt += __popcll(mk);
      }
    }
  };
  // One sub-tile on its own (128 heads, where a second partial sum held across
  // sub-tiles costs spills): lanes 0..31 end with the scores of keys kt + 32 s + l.
  auto emit1 = [&](int kt, int s, float part) {
    part += __uint_as_float(
        __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false)[1]);
    if constexpr (F8K) {
      // the scale of key kt + 32 s + col: held by lane col (s even) or 32 + col (s odd)
      // of scA (s < 2) or scB
      const float sc = s < 2 ? scA : scB;
      const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc), __float_as_uint(sc), false, false);
      part *= (s & 1) ? __uint_as_float(x[1]) : sc;
    }
    const int key = kt + 32 * s + col;
    if constexpr (SCORES) {
      if (active && hf == 0 && key < kend) scores[r * S + key] = key < nvis ? part : -INFINITY;
    } else {
      const uint64_t mk = __ballot(hf == 0 && key < nvis && part > theta_f);
      if (mk) {
        if ((mk >> lane) & 1ull) {
          const int pos = cnt + __popcll(mk & ((1ull << lane) - 1));
          sk[pos] = ord_f32(part);
          si[pos] = key;
        }
        cnt += __popcll(mk);
      }
    }
  };
  // room for the next tile's entries
  auto make_room = [&]() {
    if (!SCORES && cnt > PS_CAP - PS_NK) {
      theta_f = unord_f32(ps_compact(sk, si, whist[wave], cnt, topk));
      cnt = topk;
    }
  };
  if constexpr (PIPE) {
    // Software pipeline over 32-key sub-tiles (up to 64 heads), carried across
    // tiles: the MFMAs of sub-tile s + 1 issue before the ReLU x weight reduction
    // of sub-tile s, so the reduction runs in the shadow of the matrix cores; the
    // last sub-tile of a tile is reduced after the barrier that publishes the
    // next tile, beside that tile's first MFMAs.  Sub-tile s accumulates in slot
    // s & 1.
    f32x16 acc[2][HT];
    if (ntiles > 0 && nvis > 0) {
      PS_BOP(0, tiles[0]);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) PS_MMA(0, ht, ht);
    }
    for (int it = 0; it < ntiles; ++it) {
      const int kt = it * PS_NK;
      const bool more = it + 1 < ntiles;
      if (more) {
        PS_LOAD(0, kt + PS_NK); PS_LOAD(1, kt + PS_NK); PS_LOAD(2, kt + PS_NK); PS_LOAD(3, kt + PS_NK);
        load_scales(kt + PS_NK, nscA, nscB);
      }
      const uint8_t* buf = tiles[it & 1];
      const bool cur = kt < nvis;  // uniform per wave
      // partial sums of sub-tiles 0 and 1, then 2 (3 is reduced after the barrier)
      float p0 = 0.0f, p1 = 0.0f, p2 = 0.0f;
      static_assert(NS == 4, "sub-tiles leave in pairs");
      if (cur) {
        PS_BOP(1, buf);
        PS_MMA_RED(1, 0, p0);
        PS_BOP(2, buf);
        PS_MMA_RED(0, 1, p1);
        emit2(kt, 0, p0, p1, scA);
        PS_BOP(3, buf);
        PS_MMA_RED(1, 0, p2);
      }
      // keep the store of the next tile after the sub-tiles above: hoisted above
      // them, the store would wait for the tile's global loads before any MFMA
      asm volatile("" ::: "memory");
      if (more) {
        uint8_t* nb = tiles[(it + 1) & 1];
        PS_STORE(0, nb); PS_STORE(1, nb); PS_STORE(2, nb); PS_STORE(3, nb);
      }
      __syncthreads();
      const bool nxt = more && kt + PS_NK < nvis;
      float part = 0.0f;
      if (nxt && cur) {
        PS_BOP(0, tiles[(it + 1) & 1]);
        PS_MMA_RED(0, (NS - 1) & 1, part);
      } else if (nxt) {
        PS_BOP(0, tiles[(it + 1) & 1]);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) PS_MMA(0, ht, ht);
      } else if (cur) {
        PS_RED(part, (NS - 1) & 1);
      }
      if (cur) {
        emit2(kt, 2, p2, part, scB);
        make_room();
      }
      scA = nscA;
      scB = nscB;
    }
  } else {
    // 128 heads: a second accumulator set of all four head tiles does not fit the
    // register file, so each sub-tile is scored one group of 32 heads at a time, the
    // MFMAs of group g + 1 (slot (g + 1) & 1) interleaved with the reduction of group
    // g (slot g & 1), weights broadcast from wb; the chain order of the reduction
    // (group by group, register by register) is unchanged.
    static_assert(HT == 4, "the 128-head path");
    f32x16 acc[2][1];
    for (int it = 0; it < ntiles; ++it) {
      const int kt = it * PS_NK;
      const bool more = it + 1 < ntiles;
      if (more) {
        PS_LOAD(0, kt + PS_NK); PS_LOAD(1, kt + PS_NK); PS_LOAD(2, kt + PS_NK); PS_LOAD(3, kt + PS_NK);
        load_scales(kt + PS_NK, nscA, nscB);
      }
      const uint8_t* buf = tiles[it & 1];
      if (kt < nvis) {  // uniform per wave: every lane runs the reductions
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          float part = 0.0f;
          PS_BOP(s, buf);
          PS_MMA(0, 0, 0);
#pragma unroll
          for (int g = 1; g < HT; ++g) {
            const int ns = g & 1, os = ns ^ 1;
            acc[ns][0] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
              acc[ns][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[g][kk], bop[kk], acc[ns][0], 0, 0, 0);
#pragma unroll
              for (int j = 0; j < 2; ++j) part = fmac_bcast(part, wv[g - 1][0], relu_bits_f(acc[os][0][2 * kk + j]), 2 * kk + j);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) part = fmac_bcast(part, wv[HT - 1][0], relu_bits_f(acc[(HT - 1) & 1][0][i]), i);
          emit1(kt, s, part);
        }
        make_room();
      }
      asm volatile("" ::: "memory");
      if (more) {
        uint8_t* nb = tiles[(it + 1) & 1];
        PS_STORE(0, nb); PS_STORE(1, nb); PS_STORE(2, nb); PS_STORE(3, nb);
      }
      __syncthreads();
      scA = nscA;
      scB = nscB;
    }
  }
#undef PS_MMA_RED
#undef PS_RED
#undef PS_MMA
#undef PS_BOP
#undef PS_LOAD
#undef PS_STORE
  if (!active) return;
  if constexpr (SCORES) {
    // keys this row's tiles did not cover: the tiles from the first at or past
    // nvis were skipped, keys past kend were not scored
    const int from = min((nvis + PS_NK - 1) / PS_NK * PS_NK, kend);
    for (int key = from + lane; key < S; key += 64) scores[r * S + key] = -INFINITY;
    return;
  }
  if (cnt > topk) {
    ps_compact(sk, si, whist[wave], cnt, topk);
    cnt = topk;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  int32_t* io = idx_out + r * topk;
  float* vo = val_out ? val_out + r * topk : nullptr;
  for (int j = lane; j < topk; j += 64) {
    const bool v = j < cnt;
    io[j] = v ? si[j] : -1;
    if (vo) vo[j] = v ? unord_f32(sk[j]) : -INFINITY;
  }
}

bool prefill_scores_apply(int q_type, int k_type, int T, int H) {
  return q_type == DT_BF16 && (k_type == DT_BF16 || k_type == DT_FP8) && T >= 2 * PS_WAVES && H <= 128;
}

// One launch of the tiled kernel: scores (SC) or the fused selection, bf16 or fp8
// keys, 32 / 64 / 128 heads.
template <bool SC>
static hipError_t launch_prefill(const uint16_t* q, const float* w, const void* k, int k_type, const float* ks,
                                 const int32_t* nv, int B, int T, int S, int H, int topk, int32_t* idx, float* val,
                                 float* scores, hipStream_t st) {
  const int blocks = B * ((T + PS_WAVES - 1) / PS_WAVES);
  const dim3 g(blocks), t(PS_WAVES * 64);
  const bool f8 = k_type == DT_FP8;
  if (H <= 32) {
    if (f8) prefill_select_kernel<1, SC, true><<<g, t, 0, st>>>(q, w, k, ks, nv, T, S, H, topk, idx, val, scores);
    else prefill_select_kernel<1, SC, false><<<g, t, 0, st>>>(q, w, k, ks, nv, T, S, H, topk, idx, val, scores);
  } else if (H <= 64) {
    if (f8) prefill_select_kernel<2, SC, true><<<g, t, 0, st>>>(q, w, k, ks, nv, T, S, H, topk, idx, val, scores);
    else prefill_select_kernel<2, SC, false><<<g, t, 0, st>>>(q, w, k, ks, nv, T, S, H, topk, idx, val, scores);
  } else {
    if (f8) prefill_select_kernel<4, SC, true><<<g, t, 0, st>>>(q, w, k, ks, nv, T, S, H, topk, idx, val, scores);
    else prefill_select_kernel<4, SC, false><<<g, t, 0, st>>>(q, w, k, ks, nv, T, S, H, topk, idx, val, scores);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_scores(const uint16_t* q, const float* w, const void* k, int k_type, const float* ks,
                                 const int32_t* nv, int B, int T, int S, int H, float* scores, hipStream_t st) {
  return launch_prefill<true>(q, w, k, k_type, ks, nv, B, T, S, H, 0, nullptr, nullptr, scores, st);
}

static bool use_fused(int q_type, int k_type, int T, int H, int topk) {
  return prefill_scores_apply(q_type, k_type, T, H) && topk <= PS_KMAX;
}

bool prefill_fused_apply(int q_type, int k_type, int T, int H, int topk) {
  return use_fused(q_type, k_type, T, H, topk);
}

size_t indexer_topk_ws_bytes(int q_type, int k_type, int B, int T, int S, int H, int topk) {
  // the same predicate as launch_indexer_topk: the fused prefill kernel needs
  // nothing; every other path the scores and the top-k's own workspace (the held
  // decode path lists its candidates into the top-k's regions)
  (void)H;
  if (use_fused(q_type, k_type, T, H, topk)) return 0;
  return align256((size_t)B * T * S * sizeof(float)) + topk_ws_bytes(B * T, S, topk);
}

hipError_t launch_indexer_topk(const void* q, int q_type, const float* w, const void* k, int k_type, const float* ks,
                               const int32_t* nv, int B, int T, int S, int H, int topk, int32_t* idx, float* val,
                               void* ws, hipStream_t st) {
  if (use_fused(q_type, k_type, T, H, topk))
    return launch_prefill<false>((const uint16_t*)q, w, k, k_type, ks, nv, B, T, S, H, topk, idx, val, nullptr, st);
  float* scores = (float*)ws;
  void* tws = (uint8_t*)ws + align256((size_t)B * T * S * sizeof(float));
  if (held_select_apply(q_type, k_type, B * T, S, H, topk)) {
    // few long rows, fp8 keys, at most 64 heads: each scoring workgroup lists its own
    // entries above a threshold of its own (into the top-k's threshold area and
    // regions), one finalize selects
    uint32_t *tau_used, *bcnt;
    float* cval;
    int32_t* cid;
    topk_mb_layout(tws, B * T, S, &tau_used, &bcnt, &cval, &cid);
    int P = 0, chunk = 0;
    hipError_t e = launch_score_held_select(q, w, k, ks, nv, B, T, S, H, topk, scores, bcnt, cval, cid, tau_used, &P,
                                            &chunk, st);
    if (e != hipSuccess) return e;
    return launch_topk_finalize_f32(scores, nv, B * T, S, topk, P, chunk, bcnt, cval, cid, idx, val, tau_used, st);
  }
  // otherwise score, then select (few long rows: every region of a row lists its
  // entries above a threshold of its own, as above)
  hipError_t e = launch_score(q, q_type, w, k, k_type, ks, nv, B, T, S, H, scores, st);
  if (e != hipSuccess) return e;
  return launch_topk_f32(scores, nv, B * T, S, topk, idx, val, tws, st);
}

size_t indexer_topk_paged_ws_bytes(int B, int T, int S, int H, int topk) {
  (void)H;
  // the scores and the top-k's workspace (either path fits)
  return align256((size_t)B * T * S * sizeof(float)) + topk_ws_bytes(B * T, S, topk);
}

hipError_t launch_indexer_topk_paged(const uint16_t* q, const float* w, const uint8_t* k_pool, const float* ks_pool,
                                     const int32_t* page_table, int max_pages, int num_pages, const int32_t* nv,
                                     int B, int T, int S, int H, int topk, int32_t* idx, float* val, void* ws,
                                     hipStream_t st) {
  const int R = B * T;
  float* scores = (float*)ws;
  void* tws = (uint8_t*)ws + align256((size_t)R * S * sizeof(float));
  if (held_select_apply(DT_BF16, DT_FP8, R, S, H, topk)) {
    uint32_t *tau_used, *bcnt;
    float* cval;
    int32_t* cid;
    topk_mb_layout(tws, R, S, &tau_used, &bcnt, &cval, &cid);
    int P = 0, chunk = 0;
    hipError_t e = launch_score_held_select(q, w, k_pool, ks_pool, nv, B, T, S, H, topk, scores, bcnt, cval, cid,
                                            tau_used, &P, &chunk, st, page_table, max_pages, num_pages);
    if (e != hipSuccess) return e;
    return launch_topk_finalize_f32(scores, nv, R, S, topk, P, chunk, bcnt, cval, cid, idx, val, tau_used, st);
  }
  hipError_t e = launch_score_paged(q, w, k_pool, ks_pool, page_table, max_pages, num_pages, nv, B, T, S, H, scores,
                                    st);
  if (e != hipSuccess) return e;
  return launch_topk_f32(scores, nv, R, S, topk, idx, val, tws, st);
}

}  // namespace li
