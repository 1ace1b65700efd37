// Selection building blocks shared by the top-k kernels and the scoring kernel's
// selection epilogue (gfx950, wave64): orderable score keys, wave-aggregated LDS
// histograms, a workgroup radix select over 8-bit digits, and the threshold filter
// that lists a range's entries at or above a threshold in index order.
#pragma once

#include "common.h"

namespace li {

constexpr int MB_THREADS = 256;
constexpr int MB_SAMPLES = 4096;
constexpr int MB_BATCH = 16;  // loads in flight per thread
constexpr int MB_KEEP = 8192;  // kept entries the exact final pass holds

template <typename S>
struct ScoreTraits;
template <>
struct ScoreTraits<float> {
  typedef uint32_t K;
  static constexpr int BITS = 32;
  __device__ static K ord(float x) { return ord_f32(x); }
};
template <>
struct ScoreTraits<double> {
  typedef uint64_t K;
  static constexpr int BITS = 64;
  __device__ static K ord(double x) { return ord_f64(x); }
};

// Lane exchange of a 32- or 64-bit key.
__device__ __forceinline__ uint32_t shfl_xor_k(uint32_t x, int o) { return (uint32_t)__shfl_xor((int)x, o); }
__device__ __forceinline__ uint64_t shfl_xor_k(uint64_t x, int o) {
  const uint32_t l = (uint32_t)__shfl_xor((int)(uint32_t)x, o), h = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), o);
  return ((uint64_t)h << 32) | l;
}

// hist[d] += 1 for every lane with valid set; when all such lanes of the wave
// share one digit (scores concentrated in few bins) a single atomic adds them.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t d, bool valid) {
  const uint64_t act = __ballot(valid);
  if (!act) return;
  const int first = __ffsll((unsigned long long)act) - 1;
  const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)d, first);  // first is wave-uniform
  const uint64_t same = __ballot(valid && d == d0);
  if (same == act) {
    if ((int)(threadIdx.x & 63) == first) atomicAdd(&hist[d0], (uint32_t)__popcll(act));
  } else if (valid) {
    atomicAdd(&hist[d], 1u);
  }
}

// The kth largest (1-based) of the valid keys held E per thread over a workgroup
// of NT >= 256 threads, by PASSES 8-bit digits from the top (LDS histograms of
// 256 bins).  With fewer than 4 passes the unresolved low bits come back zero:
// the result is then the lower edge of the bucket holding the kth largest, so at
// least kth keys are >= it.  With 4 passes *n_above receives how many valid keys
// exceed the result.
template <int NT, int E, int PASSES, typename K>
__device__ __forceinline__ K block_kth8(const K (&key)[E], const bool (&valid)[E], uint32_t kth, uint32_t* hist,
                                        uint32_t* wsum, uint32_t* res, uint32_t* n_above = nullptr) {
  static_assert(NT >= 256 && NT % 64 == 0, "one thread per bin");
  constexpr int NW = NT / 64;
  constexpr int BITS = 8 * (int)sizeof(K);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  K prefix = 0, mask = 0;
  uint32_t need = kth;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int shift = BITS - 8 - 8 * p;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
      hist_add(hist, (uint32_t)(key[e] >> shift) & 255u, valid[e] && (key[e] & mask) == prefix);
    __syncthreads();
    // counts of digits 255, 254, ... accumulated in that order
    const uint32_t c = tid < 256 ? hist[255 - tid] : 0u;
    uint32_t v = c;
    v = wave_incl_scan(v);
    if (lane == 63) wsum[wid] = v;
    __syncthreads();
    uint32_t base = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) base += w < wid ? wsum[w] : 0u;
    const uint32_t incl = base + v, excl = incl - c;
    if (tid < 256 && excl < need && need <= incl) {
      res[0] = 255u - (uint32_t)tid;
      res[1] = excl;
    }
    __syncthreads();
    const uint32_t d = res[0], above = res[1];
    __syncthreads();
    prefix |= (K)d << shift;
    mask |= (K)255 << shift;
    need -= above;
  }
  if (n_above) *n_above = kth - need;
  return prefix;
}

// Digits of the wide select: 12 bits, a 4,096-bin LDS histogram.
constexpr int KW_BITS = 12;
constexpr int KW_BINS = 1 << KW_BITS;

// The kth largest (1-based) of the valid keys held E per thread over a workgroup
// of NT threads, exactly, with *n_above receiving how many valid keys exceed it
// (kth <= the number of valid keys).  The bits above the highest bit in which the
// valid keys differ are common to all of them (block minimum and maximum); the
// rest is resolved KW_BITS bits per pass from the top.  A list of candidates
// above a threshold spans few binades, so 32-bit keys take two or three passes
// and 64-bit keys four or five, against four and eight 8-bit passes; and once the
// digit holding the kth key holds no other key, that key is the answer and the
// remaining passes are skipped (one key per digit is the common case after the
// first pass or two).
// hist: KW_BINS words; wsum: room for 2 NT / 64 keys; res: 3 words.
template <int NT, int E, typename K>
__device__ __forceinline__ K block_kth_wide(const K (&key)[E], const bool (&valid)[E], uint32_t kth, uint32_t* hist,
                                            uint32_t* wsum, uint32_t* res, uint32_t* n_above) {
  static_assert(NT % 64 == 0 && KW_BINS % NT == 0, "whole bins per thread");
  constexpr int NW = NT / 64;
  constexpr int BPT = KW_BINS / NT;  // bins per thread
  constexpr int BITS = 8 * (int)sizeof(K);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // common high bits: minimum and maximum over the valid keys
  K mn = ~(K)0, mx = 0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (valid[e]) {
      mn = key[e] < mn ? key[e] : mn;
      mx = key[e] > mx ? key[e] : mx;
    }
  for (int o = 32; o > 0; o >>= 1) {
    const K a = shfl_xor_k(mn, o), c = shfl_xor_k(mx, o);
    mn = a < mn ? a : mn;
    mx = c > mx ? c : mx;
  }
  K* wk = (K*)wsum;  // NW minima, then NW maxima
  if (lane == 0) {
    wk[wid] = mn;
    wk[NW + wid] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mn = wk[w] < mn ? wk[w] : mn;
    mx = wk[NW + w] > mx ? wk[NW + w] : mx;
  }
  __syncthreads();
  const K diff = mn ^ mx;
  // bits [0, hi] vary; the ones above are mx's
  int hi = diff == 0 ? -1 : BITS - 1 - (sizeof(K) == 8 ? __clzll((unsigned long long)diff) : __clz((uint32_t)diff));
  K prefix = hi + 1 >= BITS ? (K)0 : (mx >> (hi + 1)) << (hi + 1);
  K mask = hi + 1 >= BITS ? (K)0 : ~(K)0 << (hi + 1);
  uint32_t need = kth;
  while (hi >= 0) {  // uniform
    const int lo = hi - KW_BITS + 1 > 0 ? hi - KW_BITS + 1 : 0;
    const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
#pragma unroll
    for (int i = 0; i < BPT; ++i) hist[tid + NT * i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
      hist_add(hist, (uint32_t)(key[e] >> lo) & dmask, valid[e] && (key[e] & mask) == prefix);
    __syncthreads();
    // thread t holds digits KW_BINS - 1 - BPT t - i, i < BPT (largest first)
    uint32_t c[BPT], s = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      c[i] = hist[KW_BINS - 1 - BPT * tid - i];
      s += c[i];
    }
    uint32_t v = wave_incl_scan(s);
    if (lane == 63) wsum[wid] = v;
    __syncthreads();
    uint32_t base = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) base += w < wid ? wsum[w] : 0u;
    uint32_t above = base + v - s;  // keys in larger digits
    if (above < need && need <= above + s) {
#pragma unroll
      for (int i = 0; i < BPT; ++i) {
        if (above < need && need <= above + c[i]) {
          res[0] = (uint32_t)(KW_BINS - 1 - BPT * tid - i);
          res[1] = above;
          res[2] = c[i];
        }
        above += c[i];
      }
    }
    __syncthreads();
    const uint32_t d = res[0], ab = res[1], cd = res[2];
    __syncthreads();
    prefix |= (K)d << lo;
    mask |= (K)dmask << lo;
    need -= ab;
    hi = lo - 1;
    if (cd == 1u && hi >= 0) {  // uniform: the digit's only key is the kth
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (valid[e] && (key[e] & mask) == prefix) wk[0] = key[e];
      __syncthreads();
      const K kv = wk[0];
      __syncthreads();
      *n_above = kth - need;
      return kv;
    }
  }
  *n_above = kth - need;
  return prefix;
}

// Exclusive prefix sum of x over the workgroup (blockDim.x = NW * 64), in thread
// order; scratch holds NW entries.
template <int NW>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* scratch) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t incl = x;
  incl = wave_incl_scan(incl);
  if (lane == 63) scratch[wid] = incl;
  __syncthreads();
  uint32_t base = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) base += w < wid ? scratch[w] : 0u;
  __syncthreads();
  return base + incl - x;
}

// The entries of row[lo, hi) whose orderable key is >= t, listed in index order at
// ov / oi (values, positions); returns how many.  A workgroup of MB_THREADS threads
// (every thread calls it); cnt_uw holds MB_BATCH * MB_THREADS / 64 + 1 words of LDS.
// A batch holds entries base + tid + 256 u (u < MB_BATCH), so ordering by
// (u, wave, lane) is index order; each wave's ballots give the counts, and one
// prefix over the (u, wave) counts gives every lane its position.
template <typename Sc>
__device__ __forceinline__ uint32_t filter_region(const Sc* __restrict__ row, int lo, int hi,
                                                  typename ScoreTraits<Sc>::K t, Sc* __restrict__ ov,
                                                  int32_t* __restrict__ oi, uint32_t* cnt_uw) {
  constexpr int NW = MB_THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t written = 0;
  for (int base = lo; base < hi; base += MB_THREADS * MB_BATCH) {
    Sc x[MB_BATCH];
#pragma unroll
    for (int u = 0; u < MB_BATCH; ++u) {
      const int i = base + tid + MB_THREADS * u;
      x[u] = i < hi ? row[i] : (Sc)-INFINITY;
    }
    uint64_t mk[MB_BATCH];
#pragma unroll
    for (int u = 0; u < MB_BATCH; ++u) {
      const int i = base + tid + MB_THREADS * u;
      mk[u] = __ballot(i < hi && ScoreTraits<Sc>::ord(x[u]) >= t);
      if (lane == 0) cnt_uw[u * NW + wid] = (uint32_t)__popcll(mk[u]);
    }
    __syncthreads();
    // exclusive prefix of the (u, wave) counts: one wave, one entry per lane
    static_assert(MB_BATCH * NW == 64, "one count per lane of a wave");
    if (tid < 64) {
      const uint32_t c = cnt_uw[tid];
      uint32_t incl = c;
      incl = wave_incl_scan(incl);
      cnt_uw[tid] = incl - c;
      if (tid == 63) cnt_uw[64] = incl;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < MB_BATCH; ++u) {
      if ((mk[u] >> lane) & 1ull) {
        const uint32_t pos = written + cnt_uw[u * NW + wid] + (uint32_t)__popcll(mk[u] & ((1ull << lane) - 1));
        ov[pos] = x[u];
        oi[pos] = base + tid + MB_THREADS * u;
      }
    }
    written += cnt_uw[MB_BATCH * NW];
    __syncthreads();
  }
  return written;
}

// How many of m samples of an n-entry row the threshold estimate keeps above it:
// j = max(ceil((2k + 1024) m / n), 16), at most m.  About 2k + 1024 entries of the
// row (at least 16 sample gaps) then clear the j-th largest sample.
__device__ __forceinline__ uint32_t sample_rank(int k, int m, int n) {
  int64_t j = ((int64_t)(2 * k + 1024) * m + n - 1) / n;
  if (j < 16) j = 16;
  if (j > m) j = m;
  return (uint32_t)j;
}

// Region count marking a range that was not filtered (its threshold was not
// available): the final selection then takes the whole row.
constexpr uint32_t REGION_UNFILTERED = 0xFFFFFFFFu;

// ---- lists above a threshold of the region's own ------------------------------
// After [LSA] "What the kernels do about the top-p" (a threshold, then a list of
// the entries above it), with the threshold taken by each of the P regions of a
// row from its own scores, so that no workgroup waits for another.  A workgroup of
// 256 threads holds the n <= 4096 scores of its region, 16 per thread (entry
// e * 256 + tid in v[e]).  Each wave finds the c-th largest of its 64 per-thread
// maxima, c = ceil(j / 4), by a binary search on a 32-bit ordered key (one compare
// and one ballot count per bit), and the region's threshold is the smallest of its
// four waves': every wave holds at least c entries at or above it, so at least j
// are listed (all of a wave's entries when fewer than c of its threads hold any).
// fp32 scores: the key is the whole ordered value and j = max(ceil(3 k / P), 16).
// fp64 scores: the key is the upper 32 bits of the ordered value (an entry is
// listed when its upper half reaches the threshold, so every unlisted entry lies
// below threshold << 32), and j = max(u + 6 sqrt(u) + 8, 16) with u = ceil(k / P),
// the region's expected share of the top k plus six of its standard deviations:
// for k = 2,048 over 32 regions the lists stay near 6,000 entries, within the exact
// pass.  The entries at or above the threshold go to ov / oi (values, ids id0 +
// entry) in index order; the region records its count (*bc), its threshold
// (tu_row[region]) and, with at most 128 regions a row, its largest key
// (tu_row[128 + region]; it is always listed).  A row's top k lies among the
// lists whenever its kth listed value reaches every region's threshold: the
// finalize checks that and otherwise selects over the whole row.  scratch: 96
// bytes of LDS (16-byte aligned); both barriers order LDS only.
constexpr int LT_E = 16;  // entries per thread: regions of at most 4,096 scores
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

__device__ __forceinline__ uint32_t lt_key(float x) { return ord_f32(x); }
__device__ __forceinline__ uint32_t lt_key(double x) { return (uint32_t)(ord_f64(x) >> 32); }

// Listed entries a region aims for (see above).
template <typename Sc>
__device__ __forceinline__ uint32_t lt_listed_target(int k, int P) {
  if constexpr (sizeof(Sc) == 4) {
    return (uint32_t)max((3 * k + P - 1) / P, 16);
  } else {
    const int u = (k + P - 1) / P;
    const int sq = (int)ceilf(sqrtf((float)u));
    return (uint32_t)max(u + 6 * sq + 8, 16);
  }
}

template <typename Sc>
__device__ __forceinline__ void list_above_local_threshold(const Sc (&v)[LT_E], int n, int k, int P, int region,
                                                           Sc* __restrict__ ov, int32_t* __restrict__ oi,
                                                           int id0, uint32_t* __restrict__ bc,
                                                           uint32_t* __restrict__ tu_row, void* scratch) {
  lds_u32* wt = (lds_u32*)(uintptr_t)lds_addr(scratch);  // 4 wave thresholds, 4 wave maxima
  lds_u32* cnt = wt + 8;                                   // 4 waves x 16 byte counts
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t key[LT_E];
  uint32_t m = 0u;  // entries past n hold the smallest key, 0
#pragma unroll
  for (int e = 0; e < LT_E; ++e) {
    key[e] = e * 256 + tid < n ? lt_key(v[e]) : 0u;
    m = max(m, key[e]);
  }
  const uint32_t c = (lt_listed_target<Sc>(k, P) + 3u) / 4u;
  uint32_t t = 0u;  // the largest t with at least c maxima >= t
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    if ((uint32_t)__popcll(__ballot(m >= cand)) >= c) t = cand;
  }
  uint32_t mx = m;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  if (lane == 0) {
    wt[wid] = t;
    wt[4 + wid] = mx;
  }
  lds_barrier();
  const uint32_t tau = min(min(wt[0], wt[1]), min(wt[2], wt[3]));
  // entries e * 256 + tid: ordering by (e, wave, lane) is index order.  The wave's
  // 16 counts (each at most 64) go to LDS as bytes, four to a word, in one write
  uint64_t mk[LT_E];
  uint32_t pk[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < LT_E; ++e) {
    mk[e] = __ballot(e * 256 + tid < n && key[e] >= tau);
    pk[e >> 2] |= (uint32_t)__popcll(mk[e]) << (8 * (e & 3));
  }
  if (lane == 0) *(lds_u32x4*)(cnt + 4 * wid) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
  lds_barrier();
  // lane l takes the count of slot l = 4 e + w (entry slot e of wave w)
  const int le = lane >> 2, lw = lane & 3;
  const uint32_t cl = (cnt[4 * lw + (le >> 2)] >> (8 * (le & 3))) & 0xFFu;
  const uint32_t incl = wave_incl_scan(cl);
  const uint32_t excl = incl - cl;
#pragma unroll
  for (int e = 0; e < LT_E; ++e) {
    const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)excl, e * 4 + wid);
    if ((mk[e] >> lane) & 1ull) {
      const uint32_t pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(mk[e] >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)mk[e], 0u));
      ov[pos] = v[e];
      oi[pos] = id0 + e * 256 + tid;
    }
  }
  if (tid == 0) {
    *bc = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    tu_row[region] = tau;
    if (P <= 128) tu_row[128 + region] = max(max(wt[4], wt[5]), max(wt[6], wt[7]));
  }
}

}  // namespace li
