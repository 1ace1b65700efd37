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
// heads in registers.  Selection per row: a running threshold theta (the current
// k-th best) and a candidate list of CAP entries in LDS kept in key-index order.
// A score is listed when it beats theta; when the list is full the wave compacts
// it to the exact current top-k (bisection on the orderable score bits for the
// k-th value, ties to the smaller index, order-preserving) and raises theta.
// Keys arrive in increasing index order, so an entry equal to theta loses its
// tie and a strict comparison is exact.
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

// SCORES: write every score to scores [B*T, S] (masked keys -inf) instead of
// selecting (the same contraction for li_indexer_score at prefill shapes).
template <int HT, bool SCORES>
__global__ __launch_bounds__(PS_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_select_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                           const uint16_t* __restrict__ k, const int32_t* __restrict__ nv, int T, int S, int H,
                           int topk, int32_t* __restrict__ idx_out, float* __restrict__ val_out,
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

  // keys needed by the workgroup: the largest visible count of its rows
  __shared__ int s_kend;
  if (tid == 0) s_kend = 0;
  __syncthreads();
  if (lane == 0) atomicMax(&s_kend, nvis);
  __syncthreads();
  const int kend = s_kend;

  // query block (A operand) and head weights in accumulator row order
  bf16x8 a[HT][8];
  float wv[HT][16];
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
    for (int i = 0; i < 16; ++i) {
      const int hh = ht * 32 + (i & 3) + 8 * (i >> 2) + 4 * hf;
      wv[ht][i] = (hh < H && active) ? w[r * H + hh] : 0.0f;
    }
  }

  const uint16_t* kbase = k + (int64_t)b * S * 128;
  // cooperative tile load: thread tid moves the 16-byte chunks
  // c = tid + 512 j (key c >> 4, chunk c & 15)
  static_assert(PS_NK * 16 == PS_CPT * PS_WAVES * 64, "whole chunks per thread");
  const int cn0 = tid >> 4, cc = tid & 15;  // key of chunk j: cn0 + 32 j
  constexpr int KSTEP = PS_WAVES * 64 / 16;

  uint32_t* sk = cand_k[wave];
  int32_t* si = cand_i[wave];
  int cnt = 0;          // listed entries
  uint32_t theta = 0u;  // orderable key to beat

  const int ntiles = (kend + PS_NK - 1) / PS_NK;
  // four named registers, not an array: an array here is kept in scratch memory
  static_assert(PS_CPT == 4, "chunk registers below");
  uint4 reg0, reg1, reg2, reg3;
#define PS_LOAD(j, key0) \
  reg##j = *(const uint4*)(kbase + (int64_t)min((key0) + cn0 + KSTEP * j, S - 1) * 128 + cc * 8)
#define PS_STORE(j, buf) \
  *(uint4*)((buf) + (cn0 + KSTEP * j) * 256 + ((cc ^ ((cn0 + KSTEP * j) & 15)) << 4)) = reg##j
  if (ntiles > 0) {
    PS_LOAD(0, 0); PS_LOAD(1, 0); PS_LOAD(2, 0); PS_LOAD(3, 0);
    PS_STORE(0, tiles[0]); PS_STORE(1, tiles[0]); PS_STORE(2, tiles[0]); PS_STORE(3, tiles[0]);
  }
  // every load issued so far (query block, weights, first tile) has landed: the
  // loop then only waits on its own next-tile loads where they are stored
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int kt = it * PS_NK;
    const bool more = it + 1 < ntiles;
    if (more) {
      PS_LOAD(0, kt + PS_NK); PS_LOAD(1, kt + PS_NK); PS_LOAD(2, kt + PS_NK); PS_LOAD(3, kt + PS_NK);
    }
    const uint8_t* buf = tiles[it & 1];
    if (kt < nvis) {  // uniform per wave
      // software pipeline over the tile's 32-key sub-tiles (up to 64 heads):
      // the MFMAs of sub-tile s + 1 issue before the ReLU x weight reduction of
      // sub-tile s, so that reduction runs in the shadow of the matrix cores.
      // With 128 heads a second accumulator set does not fit the register file:
      // each group of 32 heads is scored, then reduced.
      constexpr bool PIPE = HT <= 2;
      constexpr int NS = PS_NK / 32;
      f32x16 acc[PIPE ? 2 : 1][PIPE ? HT : 1];
      bf16x8 bop[8];
#define PS_BOP(sub)                                                                                             \
  do {                                                                                                          \
    const int n_ = 32 * (sub) + col;                                                                            \
    _Pragma("unroll") for (int kk = 0; kk < 8; ++kk) bop[kk] =                                                  \
        __builtin_bit_cast(bf16x8, *(const uint4*)(buf + n_ * 256 + (((8 * hf + kk) ^ (n_ & 15)) << 4)));       \
  } while (0)
#define PS_MMA(slot, ht, aset)                                                                                  \
  do {                                                                                                          \
    acc[slot][ht] = f32x16{};                                                                                   \
    _Pragma("unroll") for (int kk = 0; kk < 8; ++kk) acc[slot][ht] =                                            \
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[aset][kk], bop[kk], acc[slot][ht], 0, 0, 0);                  \
  } while (0)
      if constexpr (PIPE) {
        PS_BOP(0);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) PS_MMA(0, ht, ht);
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float part = 0.0f;
        if constexpr (!PIPE) {
          PS_BOP(s);
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) {
            PS_MMA(0, 0, ht);
#pragma unroll
            for (int i = 0; i < 16; ++i) part = fmaf(wv[ht][i], relu_bits_f(acc[0][0][i]), part);
          }
        } else {
          if (s + 1 < NS) {
            PS_BOP(s + 1);
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) PS_MMA((s + 1) & 1, ht, ht);
          }
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
            for (int i = 0; i < 16; ++i) part = fmaf(wv[ht][i], relu_bits_f(acc[s & 1][ht][i]), part);
          }
        }
        // lanes 0..31 add the partial sum of lanes 32..63 (same key, other heads)
        part += __uint_as_float(__builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part),
                                                                 false, false)[1]);
        if (PIPE && s + 1 < NS) {
          // interleave: one MFMA, then four VALU operations of the reduction
#pragma unroll
          for (int g = 0; g < 8 * HT; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          }
        }
        const int key = kt + 32 * s + col;
        if constexpr (SCORES) {
          if (active && hf == 0 && key < kend) scores[r * S + key] = key < nvis ? part : -INFINITY;
          continue;
        }
        const uint32_t ok = ord_f32(part);
        const uint64_t mk = __ballot(hf == 0 && key < nvis && ok > theta);
        if (mk) {
          if ((mk >> lane) & 1ull) {
            const int pos = cnt + __popcll(mk & ((1ull << lane) - 1));
            sk[pos] = ok;
            si[pos] = key;
          }
          cnt += __popcll(mk);
        }
      }
      // room for the next tile's entries
      if (!SCORES && cnt > PS_CAP - PS_NK) {
        theta = ps_compact(sk, si, whist[wave], cnt, topk);
        cnt = topk;
      }
    }
    // keep the store of the next tile after this tile's compute: hoisted above
    // it, the store would wait for the tile's global loads before any MFMA issues
    asm volatile("" ::: "memory");
    if (more) {
      uint8_t* nb = tiles[(it + 1) & 1];
      PS_STORE(0, nb); PS_STORE(1, nb); PS_STORE(2, nb); PS_STORE(3, nb);
    }
    __syncthreads();
  }
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
  return q_type == DT_BF16 && k_type == DT_BF16 && T >= 2 * PS_WAVES && H <= 128;
}

hipError_t launch_prefill_scores(const uint16_t* q, const float* w, const uint16_t* k, const int32_t* nv, int B,
                                 int T, int S, int H, float* scores, hipStream_t st) {
  const int blocks = B * ((T + PS_WAVES - 1) / PS_WAVES);
  if (H <= 32)
    prefill_select_kernel<1, true><<<blocks, PS_WAVES * 64, 0, st>>>(q, w, k, nv, T, S, H, 0, nullptr, nullptr,
                                                                    scores);
  else if (H <= 64)
    prefill_select_kernel<2, true><<<blocks, PS_WAVES * 64, 0, st>>>(q, w, k, nv, T, S, H, 0, nullptr, nullptr,
                                                                    scores);
  else
    prefill_select_kernel<4, true><<<blocks, PS_WAVES * 64, 0, st>>>(q, w, k, nv, T, S, H, 0, nullptr, nullptr,
                                                                    scores);
  return hipGetLastError();
}

static bool use_fused(int q_type, int k_type, int T, int H, int topk) {
  return q_type == DT_BF16 && k_type == DT_BF16 && T >= 2 * PS_WAVES && topk <= PS_KMAX && H <= 128;
}

size_t indexer_topk_ws_bytes(int B, int T, int S, int H, int topk) {
  (void)H;
  // the fused path needs no workspace; sized for the score-then-select path,
  // which any shape may take
  return align256((size_t)B * T * S * sizeof(float)) + topk_ws_bytes(B * T, S, topk) +
         align256((size_t)B * T * 1024 * sizeof(uint32_t)) + align256((size_t)B * T * 256 * sizeof(uint32_t)) +
         align256((size_t)B * T * 128);
}

hipError_t launch_indexer_topk(const void* q, int q_type, const float* w, const void* k, int k_type, const float* ks,
                               const int32_t* nv, int B, int T, int S, int H, int topk, int32_t* idx, float* val,
                               void* ws, hipStream_t st) {
  if (use_fused(q_type, k_type, T, H, topk)) {
    const int blocks = B * ((T + PS_WAVES - 1) / PS_WAVES);
    const uint16_t* qq = (const uint16_t*)q;
    const uint16_t* kk = (const uint16_t*)k;
    if (H <= 32)
      prefill_select_kernel<1, false><<<blocks, PS_WAVES * 64, 0, st>>>(qq, w, kk, nv, T, S, H, topk, idx, val,
                                                                       nullptr);
    else if (H <= 64)
      prefill_select_kernel<2, false><<<blocks, PS_WAVES * 64, 0, st>>>(qq, w, kk, nv, T, S, H, topk, idx, val,
                                                                       nullptr);
    else
      prefill_select_kernel<4, false><<<blocks, PS_WAVES * 64, 0, st>>>(qq, w, kk, nv, T, S, H, topk, idx, val,
                                                                       nullptr);
    return hipGetLastError();
  }
  float* scores = (float*)ws;
  void* tws = (uint8_t*)ws + align256((size_t)B * T * S * sizeof(float));
  if (select_score_apply(q_type, k_type, B * T, S, H, topk)) {
    // few long rows: the scoring kernel lists the candidates, one finalize selects
    uint32_t *unused, *bcnt;
    float* cval;
    int32_t* cid;
    topk_mb_layout(tws, B * T, S, &unused, &bcnt, &cval, &cid);
    // after the top-k's area: the sample flags (1024 words per row), the threshold
    // each region used (256 words per row), the published thresholds (one 128-byte
    // line per row)
    uint32_t* counters = (uint32_t*)((uint8_t*)tws + topk_ws_bytes(B * T, S, topk));
    uint32_t* tau_used = counters + align256((size_t)B * T * 1024 * sizeof(uint32_t)) / sizeof(uint32_t);
    uint64_t* taupub = (uint64_t*)(tau_used + align256((size_t)B * T * 256 * sizeof(uint32_t)) / sizeof(uint32_t));
    int P = 0, chunk = 0;
    hipError_t e = launch_score_select(q, k_type, w, k, ks, nv, B, T, S, H, topk, scores, counters, bcnt, cval, cid,
                                       taupub, tau_used, &P, &chunk, st);
    if (e != hipSuccess) return e;
    return launch_topk_finalize_f32(scores, nv, B * T, S, topk, P, chunk, bcnt, cval, cid, idx, val, counters,
                                    tau_used, st);
  }
  hipError_t e = launch_score(q, q_type, w, k, k_type, ks, nv, B, T, S, H, scores, st);
  if (e != hipSuccess) return e;
  return launch_topk_f32(scores, nv, B * T, S, topk, idx, val, tws, st);
}

}  // namespace li
