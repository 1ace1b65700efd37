// Per-row top-k selection (k <= 2048) for gfx950.
//
// The k best entries of a row are the k largest packed keys (orderable score bits
// above the inverted key id), which makes the result unique: among equal scores
// the smaller id wins ("Latent Sparse Attention" article, section "What the
// kernels do about the top-p": a radix select over packed 64-bit keys, score bits
// above and inverted id below).  Here the packed key is never formed in memory:
//   1. an MSD radix select over the orderable score bits (11-bit digits, LDS
//      histograms) finds T, the score of the k-th best entry, and how many entries
//      equal to T are still needed;
//   2. if more entries equal T than are needed, a second radix select over the
//      inverted ids of those entries finds the id cut (smallest ids win);
//   3. one pass gathers the selected entries into LDS, a bitonic sort puts them in
//      ascending id order (the set is unique; attention does not depend on the
//      order, and ascending ids keep the later gather sequential), and they are
//      written out.
// One workgroup of 1024 threads handles one row.
#include <mutex>

#include "common.h"
#include "launch.h"
#include "select.h"

namespace li {

constexpr int TK_THREADS = 1024;
constexpr int TK_BINS = 2048;  // 11-bit digits

// Block-wide search for the digit d such that (count of entries above d) < need
// <= (count above d) + hist[d], scanning digits from the top.  Returns d and sets
// *above to the count strictly above d.  hist has TK_BINS entries in LDS.
__device__ int find_cut(const uint32_t* hist, uint32_t need, uint32_t* above, uint32_t* sh_scan, int* sh_res) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    sh_res[0] = 0;
    sh_res[1] = 0;
  }
  // thread t owns reversed bins 2t, 2t+1 (bin index TK_BINS-1-2t, TK_BINS-2-2t)
  const uint32_t c0 = hist[TK_BINS - 1 - 2 * tid];
  const uint32_t c1 = hist[TK_BINS - 2 - 2 * tid];
  uint32_t v = c0 + c1;
  // inclusive scan across the wave
  const int lane = tid & 63, wid = tid >> 6;
  v = wave_incl_scan(v);
  if (lane == 63) sh_scan[wid] = v;
  __syncthreads();
  if (tid < 64) {
    uint32_t x = tid < TK_THREADS / 64 ? sh_scan[tid] : 0;
    x = wave_incl_scan(x);
    if (tid < TK_THREADS / 64) sh_scan[tid] = x;  // inclusive over waves
  }
  __syncthreads();
  const uint32_t base = (wid ? sh_scan[wid - 1] : 0) + v - (c0 + c1);  // exclusive start of this thread
  if (base < need && need <= base + c0) {
    sh_res[0] = TK_BINS - 1 - 2 * tid;
    sh_res[1] = base;
  } else if (base + c0 < need && need <= base + c0 + c1) {
    sh_res[0] = TK_BINS - 2 - 2 * tid;
    sh_res[1] = base + c0;
  }
  __syncthreads();
  const int d = min(max(sh_res[0], 0), TK_BINS - 1);
  *above = (uint32_t)sh_res[1];
  __syncthreads();
  return d;
}

struct Sel {
  uint64_t key;  // orderable score bits (float: in the low 32 bits)
  uint32_t inv_id;
};

// list order: ascending id (inverted id descending); ids in a list are unique
__device__ __forceinline__ bool sel_greater(const Sel& a, const Sel& b) { return a.inv_id > b.inv_id; }

// Exact selection of the k best of row[0..n) (ids: idrow, or the position) by one
// workgroup of TK_THREADS threads; results in ascending id order into
// idx_out[0..k) and val_out[0..k).
template <typename S>
__device__ void select_block(const S* __restrict__ row, const int32_t* __restrict__ idrow, int n, int k,
                             int32_t* __restrict__ idx_out, S* __restrict__ val_out) {
  typedef typename ScoreTraits<S>::K K;
  constexpr int BITS = ScoreTraits<S>::BITS;
  __shared__ uint32_t hist[TK_BINS];
  __shared__ uint32_t sh_scan[64];
  __shared__ int sh_res[2];
  __shared__ uint32_t sh_count;
  __shared__ Sel list[LI_TOPK_MAX_DEV];

  const int tid = threadIdx.x;
  const int take = min(n, k);

  K prefix = 0, mask = 0;  // score-bit prefix of T
  uint32_t need = (uint32_t)take;
  bool all_of_prefix = false;  // every entry matching the prefix is selected
  uint32_t iprefix = 0, imask = 0;  // ties with (inv_id & imask) >= iprefix are selected
  bool need_tie_cut = false;

  if (n > k) {
    // ---- 1. radix select over the score bits --------------------------------
    int shift = BITS;
    while (shift > 0 && !all_of_prefix) {
      const int width = shift >= 11 ? 11 : shift;
      shift -= width;
      const uint32_t dmask = (1u << width) - 1;
      for (int i = tid; i < TK_BINS; i += TK_THREADS) hist[i] = 0;
      __syncthreads();
      for (int i0 = 0; i0 < n; i0 += TK_THREADS) {
        const int i = i0 + tid;
        K key = 0;
        if (i < n) key = ScoreTraits<S>::ord(row[i]);
        hist_add(hist, (uint32_t)(key >> shift) & dmask, i < n && (key & mask) == prefix);
      }
      __syncthreads();
      uint32_t above;
      const int d = find_cut(hist, need, &above, sh_scan, sh_res);
      const uint32_t in_bin = hist[d];
      __syncthreads();
      prefix |= (K)d << shift;
      mask |= (K)dmask << shift;
      need -= above;
      if (need == in_bin) all_of_prefix = true;  // the whole bin is taken
    }
    // ---- 2. among entries equal to T, pick the smallest ids --------------------
    if (!all_of_prefix) {
      // here mask covers every score bit: entries with key == T number > need
      need_tie_cut = true;
      int ishift = 32;
      bool done = false;
      while (ishift > 0 && !done) {
        const int width = ishift >= 11 ? 11 : ishift;
        ishift -= width;
        const uint32_t dmask = (1u << width) - 1;
        for (int i = tid; i < TK_BINS; i += TK_THREADS) hist[i] = 0;
        __syncthreads();
        for (int i0 = 0; i0 < n; i0 += TK_THREADS) {
          const int i = i0 + tid;
          bool v = false;
          uint32_t inv = 0;
          if (i < n && ScoreTraits<S>::ord(row[i]) == prefix) {
            inv = ~(uint32_t)(idrow ? idrow[i] : i);
            v = (inv & imask) == iprefix;
          }
          hist_add(hist, (inv >> ishift) & dmask, v);
        }
        __syncthreads();
        uint32_t above;
        const int d = find_cut(hist, need, &above, sh_scan, sh_res);
        const uint32_t in_bin = hist[d];
        __syncthreads();
        iprefix |= (uint32_t)d << ishift;
        imask |= dmask << ishift;
        need -= above;
        if (need == in_bin) done = true;
      }
    }
  }

  // ---- 3. gather, sort, write -------------------------------------------------
  if (tid == 0) sh_count = 0;
  __syncthreads();
  for (int i = tid; i < n; i += TK_THREADS) {
    const S x = row[i];
    const K key = ScoreTraits<S>::ord(x);
    const uint32_t id = (uint32_t)(idrow ? idrow[i] : i);
    bool sel;
    if (n <= k) {
      sel = true;
    } else if (!need_tie_cut) {
      sel = (key & mask) >= prefix;  // all entries at or above the resolved prefix
    } else {
      sel = key > prefix || (key == prefix && ((~id) & imask) >= iprefix);
    }
    if (sel) {
      const uint32_t pos = atomicAdd(&sh_count, 1u);
      if (pos < (uint32_t)LI_TOPK_MAX_DEV) list[pos] = Sel{(uint64_t)key, ~id};
    }
  }
  __syncthreads();
  const int cnt = min((int)sh_count, take);
  int P2 = 1;
  while (P2 < cnt) P2 <<= 1;
  for (int i = cnt + tid; i < P2; i += TK_THREADS) list[i] = Sel{0, 0};
  __syncthreads();
  // bitonic sort by id, ascending
  for (int size = 2; size <= P2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P2 / 2; i += TK_THREADS) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = ((lo & size) == 0);
        Sel a = list[lo], b = list[hi];
        const bool swap = desc ? sel_greater(b, a) : sel_greater(a, b);
        if (swap) {
          list[lo] = b;
          list[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int j = tid; j < k; j += TK_THREADS) {
    int32_t oi = -1;
    S ov = -INFINITY;
    if (j < cnt) {
      oi = (int32_t)(~list[j].inv_id);
      if constexpr (BITS == 32)
        ov = unord_f32((uint32_t)list[j].key);
      else
        ov = unord_f64(list[j].key);
    }
    idx_out[j] = oi;
    if (val_out) val_out[j] = ov;
  }
}

// The k best of the valid entries held E per thread in list order (entry E tid + e,
// a list in index order), written in that order at io / vo: T, the k-th best key,
// by the wide radix select, then every entry above T and the first (k - count
// above T) entries equal to T, each at its position from a prefix scan.  Every
// thread of the TK_THREADS workgroup calls it; at least k entries are valid.
// With a floor: when the kth value T lies below it nothing is written and false
// comes back (T is the same in every thread, so all of them return together).
template <typename Sc, int E>
__device__ __forceinline__ bool write_top_listed(const typename ScoreTraits<Sc>::K (&key)[E], const Sc (&val)[E],
                                                 const int32_t (&id)[E], const bool (&valid)[E], uint32_t k,
                                                 int32_t* __restrict__ io, Sc* __restrict__ vo, uint32_t* hist,
                                                 uint64_t* wsum8, uint32_t* res, uint32_t* scan1, uint32_t* scan2,
                                                 typename ScoreTraits<Sc>::K floor = 0) {
  typedef typename ScoreTraits<Sc>::K K;
  constexpr int NW = TK_THREADS / 64;
  uint32_t n_gt_all;
  const K T = block_kth_wide<TK_THREADS, E>(key, valid, k, hist, (uint32_t*)wsum8, res, &n_gt_all);
  if (T < floor) return false;
  uint32_t ties = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) ties += valid[e] && key[e] == T ? 1u : 0u;
  // rank of this thread's first tie in list order
  const uint32_t tie_rank0 = block_exclusive_scan<NW>(ties, scan1);
  const uint32_t need = k - n_gt_all;  // ties taken, first in the list first
  bool sel[E];
  uint32_t tr = tie_rank0, nsel = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool tie = valid[e] && key[e] == T;
    sel[e] = (valid[e] && key[e] > T) || (tie && tr < need);
    tr += tie ? 1u : 0u;
    nsel += sel[e] ? 1u : 0u;
  }
  uint32_t pos = block_exclusive_scan<NW>(nsel, scan2);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (sel[e]) {
      io[pos] = id[e];
      if (vo) vo[pos] = val[e];
      ++pos;
    }
  }
  return true;
}

// LDS scratch of the selections below, declared once by the kernel whatever
// entries-per-thread instance runs.
struct SelScratch {
  uint32_t scan1[TK_THREADS / 64], scan2[TK_THREADS / 64];
  uint32_t hist[KW_BINS];
  uint64_t wsum8[2 * (TK_THREADS / 64)];  // minima and maxima of the keys, per wave
  uint32_t res[3];
};

// A row of at most MB_KEEP entries whose ids ascend along the row (a row of scores
// by position, or a list of candidates kept in index order): every entry is held
// in registers, and the selection above writes the k best in position order, which
// is ascending-id order, so no sort is needed.  Rows whose ids do not ascend take
// select_block.  E entries per thread (n <= E * TK_THREADS): every pass of the
// selection loops over them, so short rows take a small E.
template <typename S, int E>
__device__ void select_small(const S* __restrict__ row, const int32_t* __restrict__ idrow, int n, int k,
                             int32_t* __restrict__ idx_out, S* __restrict__ val_out, SelScratch& sc) {
  typedef typename ScoreTraits<S>::K K;
  const int tid = threadIdx.x;
  K key[E];
  S val[E];
  int32_t id[E];
  bool valid[E];
  bool asc = true;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = E * tid + e;
    valid[e] = j < n;
    const int jc = valid[e] ? j : 0;
    val[e] = row[jc];
    id[e] = idrow ? idrow[jc] : jc;
    // the id of the next entry (this thread's last one looks at the following thread's first)
    if (idrow && j + 1 < n) asc = asc && idrow[j + 1] > id[e];
  }
  if (!__syncthreads_and(asc)) {
    select_block<S>(row, idrow, n, k, idx_out, val_out);
    return;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = valid[e] ? ScoreTraits<S>::ord(val[e]) : (K)0;
  if (n <= k) {  // every entry, then padding
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (valid[e]) {
        idx_out[E * tid + e] = id[e];
        if (val_out) val_out[E * tid + e] = val[e];
      }
    for (int j = n + tid; j < k; j += TK_THREADS) {
      idx_out[j] = -1;
      if (val_out) val_out[j] = (S)-INFINITY;
    }
    return;
  }
  write_top_listed<S, E>(key, val, id, valid, (uint32_t)k, idx_out, val_out, sc.hist, sc.wsum8, sc.res, sc.scan1,
                         sc.scan2);
}

template <typename S>
__global__ __launch_bounds__(TK_THREADS) void topk_row_kernel(const S* __restrict__ scores, int64_t row_stride,
                                                              const int32_t* __restrict__ nv,
                                                              const int32_t* __restrict__ ids, int S_len, int k,
                                                              int32_t* __restrict__ idx_out, S* __restrict__ val_out) {
  const int r = blockIdx.x;
  int n = S_len;
  if (nv) n = min(max(nv[r], 0), S_len);
  const S* row = scores + (int64_t)r * row_stride;
  const int32_t* idrow = ids ? ids + (int64_t)r * row_stride : nullptr;
  int32_t* io = idx_out + (int64_t)r * k;
  S* vo = val_out ? val_out + (int64_t)r * k : nullptr;
  __shared__ SelScratch sc;
  if (n <= 2 * TK_THREADS)
    select_small<S, 2>(row, idrow, n, k, io, vo, sc);
  else if (n <= 4 * TK_THREADS)
    select_small<S, 4>(row, idrow, n, k, io, vo, sc);
  else if (n <= MB_KEEP)
    select_small<S, MB_KEEP / TK_THREADS>(row, idrow, n, k, io, vo, sc);
  else
    select_block<S>(row, idrow, n, k, io, vo);
}

// ---- many workgroups per row (few, long rows) --------------------------------
// After the threshold selection of the "Latent Sparse Attention" article (section
// "What the kernels do about the top-p"): a threshold is estimated from a sample
// of the row, a streaming pass keeps only the entries at or above it, and an
// exact selection runs over the kept entries.  The threshold decides how many
// entries are kept, never which are picked: whenever at least k entries clear it
// (checked), the k best are among them.  A row whose estimate misses, or keeps
// more entries than the final sort holds, falls back to the exact single-workgroup
// selection over the whole row, so the result is always the exact top-k.
//   1. tau is the j-th largest of m = min(n, 4096) samples (64 runs of 64
//      consecutive entries spread evenly over the row: 16 KB read),
//      j = max(ceil((2k + 1024) m / n), 16): about 2k + 1024 entries (at least 16
//      sample gaps) should clear it, with a relative spread of 1/sqrt(j); the
//      estimate needs only the top 16 key bits;
//      one workgroup per row estimates it;
//   2. many workgroups per row append every entry of their chunk with ord >= tau
//      to their own region of the list (no global atomics, nothing to clear);
//   3. one workgroup per row selects exactly among the kept entries, or over the
//      whole row.
// Both k-th searches are radix selects over LDS histograms (11-bit digits).

constexpr int MB_RUNS = 64;  // sample runs of 64 entries

// tau of row `row` (n > k entries): the j-th largest of m = min(n, MB_SAMPLES)
// samples, 64 runs of 64 consecutive entries spread evenly over the row, by a
// workgroup of NT threads (every one of them gets the result).
template <typename Sc, int NT>
__device__ __forceinline__ typename ScoreTraits<Sc>::K sample_tau(const Sc* __restrict__ row, int n, int k,
                                                                   uint32_t* hist, uint32_t* wsum, uint32_t* res) {
  typedef typename ScoreTraits<Sc>::K K;
  constexpr int NW = NT / 64;
  constexpr int E = MB_RUNS * 64 / NT;
  static_assert(MB_RUNS * 64 == MB_SAMPLES && E * NT == MB_SAMPLES, "sample count");
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const bool runs = n >= MB_SAMPLES;
  const int m = runs ? MB_SAMPLES : n;
  const int step = runs ? (n - 64) / (MB_RUNS - 1) : 64;  // run starts: the last at most n - 64
  K key[E];
  bool valid[E];
  // unconditional loads at clamped positions, so all of them are in flight at once
  Sc x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = row[min((NW * e + wid) * step + lane, n - 1)];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    valid[e] = (NW * e + wid) * step + lane < n;
    key[e] = valid[e] ? ScoreTraits<Sc>::ord(x[e]) : (K)0;
  }
  // the top 16 key bits of a float (sign, exponent, 7 mantissa bits), 24 of a double
  return block_kth8<NT, E, sizeof(K) == 4 ? 2 : 3>(key, valid, sample_rank(k, m, n), hist, wsum, res);
}

template <typename Sc>
__global__ __launch_bounds__(TK_THREADS) void topk_thresh_kernel(const Sc* __restrict__ scores,
                                                                const int32_t* __restrict__ nv, int S, int k,
                                                                typename ScoreTraits<Sc>::K* __restrict__ tau) {
  constexpr int NW = TK_THREADS / 64;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[NW];
  __shared__ uint32_t res[2];
  const int r = blockIdx.x;
  int n = S;
  if (nv) n = min(max(nv[r], 0), S);
  if (n <= k) {  // every entry is kept
    if (threadIdx.x == 0) tau[r] = 0;
    return;
  }
  const typename ScoreTraits<Sc>::K t = sample_tau<Sc, TK_THREADS>(scores + (int64_t)r * S, n, k, hist, wsum, res);
  if (threadIdx.x == 0) tau[r] = t;
}

// Kept entries go to this workgroup's region of the list in index order: a batch
// holds entries base + tid + 256 u (u < MB_BATCH), so ordering by (u, wave, lane)
// is index order; each wave's ballots give the counts, one prefix over the
// (u, wave) counts gives every lane its position.
template <typename Sc>
__global__ __launch_bounds__(MB_THREADS) void topk_filter_kernel(const Sc* __restrict__ scores,
                                                                const int32_t* __restrict__ nv, int S, int k,
                                                                int chunk,
                                                                const typename ScoreTraits<Sc>::K* __restrict__ tau,
                                                                Sc* __restrict__ cval, int32_t* __restrict__ cid,
                                                                uint32_t* __restrict__ bcnt) {
  __shared__ uint32_t cnt_uw[MB_BATCH * (MB_THREADS / 64) + 1];
  const int r = blockIdx.y, p = blockIdx.x, P = gridDim.x, tid = threadIdx.x;
  int n = S;
  if (nv) n = min(max(nv[r], 0), S);
  if (n <= k) {  // the final pass takes the whole row
    if (tid == 0) bcnt[(int64_t)r * P + p] = 0u;
    return;
  }
  const int lo = p * chunk, hi = min(lo + chunk, n);
  const uint32_t written = filter_region<Sc>(scores + (int64_t)r * S, lo, hi, tau[r], cval + (int64_t)r * S + lo,
                                             cid + (int64_t)r * S + lo, cnt_uw);
  if (tid == 0) bcnt[(int64_t)r * P + p] = written;
}

// Exact selection over the kept entries (at most MB_KEEP, in index order): the
// k-th best orderable score T by radix select, then every entry above T and the
// first (k - count above T) entries equal to T, written in index order at
// positions from a prefix scan.  Rows whose list cannot be used take the
// whole-row path.

// The selection over a usable list of c entries (region offsets off[0..P]), E
// entries per thread (c <= E * TK_THREADS): every pass of the selection loops over
// them, so short lists take a small E.  sc: the caller's LDS scratch.
template <typename Sc, int E>
__device__ void finalize_listed(int r, const Sc* __restrict__ scores, int S, int n, int k, int P, int chunk,
                                uint32_t c, const uint32_t* off, uint32_t floor32, const Sc* __restrict__ cval,
                                const int32_t* __restrict__ cid, int32_t* __restrict__ io, Sc* __restrict__ vo,
                                SelScratch& sc) {
  typedef typename ScoreTraits<Sc>::K K;
  const int tid = threadIdx.x;
  // entries E*tid .. E*tid+E-1 of the concatenated regions (index order)
  K key[E];
  Sc val[E];
  int32_t id[E];
  bool valid[E];
  // every load is issued (entries past the list read its last entry) before any
  // is used; a thread's entries are consecutive, so after one binary search for
  // the region of its first entry the later ones only step forward
  int rg;
  {
    const uint32_t jf = min((uint32_t)(E * tid), c - 1u);
    int lo2 = 0, hi2 = P - 1;  // region b with off[b] <= jf < off[b+1]
    while (lo2 < hi2) {
      const int mid = (lo2 + hi2 + 1) >> 1;
      if (off[mid] <= jf) lo2 = mid; else hi2 = mid - 1;
    }
    rg = lo2;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t j0 = (uint32_t)(E * tid + e);
    valid[e] = j0 < c;
    const uint32_t j = valid[e] ? j0 : c - 1u;
    while (rg + 1 < P && off[rg + 1] <= j) ++rg;
    const int64_t src = (int64_t)r * S + (int64_t)rg * chunk + (j - off[rg]);
    val[e] = cval[src];
    id[e] = cid[src];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = valid[e] ? ScoreTraits<Sc>::ord(val[e]) : (K)0;
  // every unlisted entry of a region lies below its threshold; when the kth listed
  // value reaches the largest threshold no unlisted entry can enter the top k
  // (fp64 regions record the upper half of their threshold key)
  const K floor = (K)floor32 << (8 * sizeof(K) - 32);
  if (!write_top_listed<Sc, E>(key, val, id, valid, (uint32_t)k, io, vo, sc.hist, sc.wsum8, sc.res, sc.scan1,
                               sc.scan2, floor))
    select_block<Sc>(scores + (int64_t)r * S, nullptr, n, k, io, vo);
}

template <typename Sc>
__device__ void finalize_lists(int r, const Sc* __restrict__ scores, const int32_t* __restrict__ nv, int S, int k,
                               int P, int chunk, const uint32_t* __restrict__ bcnt, const Sc* __restrict__ cval,
                               const int32_t* __restrict__ cid, int32_t* __restrict__ idx_out,
                               Sc* __restrict__ val_out, const uint32_t* __restrict__ tau_used) {
  __shared__ uint32_t off[257];
  __shared__ int s_unfiltered;
  __shared__ uint32_t s_floor;
  __shared__ SelScratch sc;
  const int tid = threadIdx.x;
  int n = S;
  if (nv) n = min(max(nv[r], 0), S);
  if (tid == 0) s_unfiltered = 0;
  __syncthreads();
  // exclusive prefix of the region counts (P <= 256): one wave, four per lane.  A
  // region left unfiltered makes the lists unusable.  Regions that filtered with
  // thresholds of their own (tau_used) leave the largest of them as the floor the
  // selected kth value must reach.
  if (tid < 64) {
    uint32_t c4[4], tot = 0, fl = 0;
    bool unf = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int b = 4 * tid + e;
      c4[e] = b < P ? bcnt[(int64_t)r * P + b] : 0u;
      unf = unf || c4[e] == REGION_UNFILTERED;
      if (tau_used && b < P) fl = max(fl, tau_used[(int64_t)r * 256 + b]);
      tot += c4[e];
    }
    if (__ballot(unf) && tid == 0) s_unfiltered = 1;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) fl = max(fl, (uint32_t)__shfl_xor((int)fl, o));
    if (tid == 0) s_floor = fl;
    uint32_t incl = tot;
    incl = wave_incl_scan(incl);
    uint32_t ex = incl - tot;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int b = 4 * tid + e;
      if (b <= P) off[b] = ex;
      ex += c4[e];
    }
  }
  __syncthreads();
  const uint32_t c = off[P];
  int32_t* io = idx_out + (int64_t)r * k;
  Sc* vo = val_out ? val_out + (int64_t)r * k : nullptr;
  // the list is usable when every region was filtered and at least k entries
  // cleared the threshold
  if (n <= k || s_unfiltered || c < (uint32_t)k || c > (uint32_t)MB_KEEP) {
    select_block<Sc>(scores + (int64_t)r * S, nullptr, n, k, io, vo);
    return;
  }
  if (c <= 2u * TK_THREADS)
    finalize_listed<Sc, 2>(r, scores, S, n, k, P, chunk, c, off, s_floor, cval, cid, io, vo, sc);
  else if (c <= 4u * TK_THREADS)
    finalize_listed<Sc, 4>(r, scores, S, n, k, P, chunk, c, off, s_floor, cval, cid, io, vo, sc);
  else if (c <= 6u * TK_THREADS)
    finalize_listed<Sc, 6>(r, scores, S, n, k, P, chunk, c, off, s_floor, cval, cid, io, vo, sc);
  else
    finalize_listed<Sc, MB_KEEP / TK_THREADS>(r, scores, S, n, k, P, chunk, c, off, s_floor, cval, cid, io, vo,
                                              sc);
}

template <typename Sc>
__global__ __launch_bounds__(TK_THREADS) void topk_finalize_kernel(const Sc* __restrict__ scores,
                                                                  const int32_t* __restrict__ nv, int S, int k,
                                                                  int P, int chunk,
                                                                  const uint32_t* __restrict__ bcnt,
                                                                  const Sc* __restrict__ cval,
                                                                  const int32_t* __restrict__ cid,
                                                                  int32_t* __restrict__ idx_out,
                                                                  Sc* __restrict__ val_out,
                                                                  const uint32_t* __restrict__ tau_used) {
  finalize_lists<Sc>(blockIdx.x, scores, nv, S, k, P, chunk, bcnt, cval, cid, idx_out, val_out, tau_used);
}

// The finalize of lists filtered with thresholds of their own (at most LF_MAXP
// regions): the first M = LF_SLOTS / P entries of every region are loaded in the
// same round trip as the region counts and thresholds, before either is known
// (thread t holds slots 4 t .. 4 t + 3; slot s is entry s % M of region s / M, so
// thread order is index order), and the exact selection runs over them with the
// entries past each count masked off.  A row with a region that listed more than
// M entries takes finalize_lists; one whose kth value falls below the largest
// threshold, or that listed fewer than k, takes the whole row.
constexpr int LF_MAXP = 64;
constexpr int LF_E = 4;
constexpr int LF_SLOTS = LF_E * TK_THREADS;

// The kth largest T (1-based) of the valid keys that are >= lo_key, all of them at
// most hi_key, by 12-bit digits from the highest bit in which lo_key and hi_key
// differ; false when fewer than kth valid keys reach lo_key.  *n_above receives
// how many valid keys exceed T, *ties_all whether every key equal to T is among
// the kth.  The two histograms alternate between passes (the next one is cleared
// while the current one is scanned) and every bin keeps the largest key it
// counted, so a bin holding only the kth key gives it at once: three barriers a
// pass.  histA (with bmaxA) must be zero on entry.
template <int NT, int E>
__device__ __forceinline__ bool block_kth_bounded(const uint32_t (&key)[E], const bool (&valid)[E], uint32_t kth,
                                                  uint32_t lo_key, uint32_t hi_key, uint32_t* histA,
                                                  uint32_t* histB, uint32_t* bmaxA, uint32_t* bmaxB,
                                                  uint32_t* wsum, uint32_t* res, uint32_t* T_out,
                                                  uint32_t* n_above, bool* ties_all) {
  constexpr int NW = NT / 64;
  constexpr int BPT = KW_BINS / NT;
  static_assert(BPT * NT == KW_BINS, "whole bins per thread");
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const uint32_t diff = lo_key ^ hi_key;
  int hi = diff == 0u ? -1 : 31 - __clz(diff);
  uint32_t prefix = hi >= 31 ? 0u : (hi_key >> (hi + 1)) << (hi + 1);
  uint32_t mask = hi >= 31 ? 0u : ~0u << (hi + 1);
  uint32_t need = kth;
  bool first = true;
  for (int pass = 0;; ++pass) {  // uniform
    uint32_t* hist = (pass & 1) ? histB : histA;
    uint32_t* bmax = (pass & 1) ? bmaxB : bmaxA;
    uint32_t* nhist = (pass & 1) ? histA : histB;
    uint32_t* nbmax = (pass & 1) ? bmaxA : bmaxB;
    const int lo = hi - KW_BITS + 1 > 0 ? hi - KW_BITS + 1 : 0;
    const uint32_t dmask = hi >= 0 ? (uint32_t)((1ull << (hi - lo + 1)) - 1ull) : 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (valid[e] && key[e] >= lo_key && (key[e] & mask) == prefix) {
        const uint32_t d = hi >= 0 ? (key[e] >> lo) & dmask : 0u;
        atomicAdd(&hist[d], 1u);
        atomicMax(&bmax[d], key[e]);
      }
    }
    __syncthreads();
    // thread t holds digits KW_BINS - 1 - BPT t - i, i < BPT (largest first), and
    // clears its bins of the other histogram for the next pass
    uint32_t c[BPT], sum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int b = KW_BINS - 1 - BPT * tid - i;
      c[i] = hist[b];
      sum += c[i];
      nhist[b] = 0u;
      nbmax[b] = 0u;
    }
    const uint32_t v = wave_incl_scan(sum);
    if (lane == 63) wsum[wid] = v;
    __syncthreads();
    uint32_t base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t x = wsum[w];
      base += w < wid ? x : 0u;
      total += x;
    }
    if (first && total < kth) return false;  // uniform
    first = false;
    uint32_t above = base + v - sum;  // keys in larger digits
    if (above < need && need <= above + sum) {
#pragma unroll
      for (int i = 0; i < BPT; ++i) {
        if (above < need && need <= above + c[i]) {
          const int b = KW_BINS - 1 - BPT * tid - i;
          res[0] = (uint32_t)b;
          res[1] = above;
          res[2] = c[i];
          res[3] = bmax[b];
        }
        above += c[i];
      }
    }
    __syncthreads();
    const uint32_t d = res[0], ab = res[1], cd = res[2], bm = res[3];
    need -= ab;
    if (hi < 0 || cd == 1u || lo == 0) {
      // resolved: the bin's only key, or every bit fixed (all cd keys equal T)
      const uint32_t T = (cd == 1u) ? bm : (prefix | (hi >= 0 ? d << lo : 0u));
      *T_out = T;
      *n_above = kth - need;
      *ties_all = need == cd;
      return true;
    }
    prefix |= d << lo;
    mask |= dmask << lo;
    hi = lo - 1;
  }
}

__global__ __launch_bounds__(TK_THREADS) void topk_finalize_local_kernel(const float* __restrict__ scores,
                                                                        const int32_t* __restrict__ nv, int S,
                                                                        int k, int P, int chunk,
                                                                        const uint32_t* __restrict__ bcnt,
                                                                        const float* __restrict__ cval,
                                                                        const int32_t* __restrict__ cid,
                                                                        int32_t* __restrict__ idx_out,
                                                                        float* __restrict__ val_out,
                                                                        const uint32_t* __restrict__ tau_used) {
  constexpr int NW = TK_THREADS / 64;
  __shared__ uint32_t cnt[LF_MAXP];
  __shared__ uint32_t s_state[4];  // total, floor, overflow, largest key
  __shared__ uint32_t scan1[NW], scan2[NW];
  __shared__ uint32_t histA[KW_BINS], histB[KW_BINS], bmaxA[KW_BINS], bmaxB[KW_BINS];
  __shared__ uint32_t wsum[NW];
  __shared__ uint32_t res4[4];
  const int r = blockIdx.x, tid = threadIdx.x;
  // the first pass's histogram starts at zero
#pragma unroll
  for (int i = 0; i < KW_BINS / TK_THREADS; ++i) {
    histA[tid + TK_THREADS * i] = 0u;
    bmaxA[tid + TK_THREADS * i] = 0u;
  }
  const int M = LF_SLOTS / P;
  float val[LF_E];
  int32_t id[LF_E];
  int rg[LF_E], pos[LF_E];
  const int64_t rb = (int64_t)r * S;
#pragma unroll
  for (int e = 0; e < LF_E; ++e) {
    const int sl = LF_E * tid + e;
    rg[e] = sl / M;
    pos[e] = sl - rg[e] * M;
    const int64_t at = (int64_t)rg[e] * chunk + pos[e];
    const bool in = rg[e] < P && at < S;
    val[e] = in ? cval[rb + at] : 0.0f;
    id[e] = in ? cid[rb + at] : 0;
  }
  int n = S;
  if (nv) n = min(max(nv[r], 0), S);
  if (tid < 64) {
    const uint32_t c = tid < P ? bcnt[(int64_t)r * P + tid] : 0u;
    uint32_t fl = tid < P ? tau_used[(int64_t)r * 256 + tid] : 0u;
    uint32_t mk = tid < P ? tau_used[(int64_t)r * 256 + 128 + tid] : 0u;
    uint32_t tot = c;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      fl = max(fl, (uint32_t)__shfl_xor((int)fl, o));
      mk = max(mk, (uint32_t)__shfl_xor((int)mk, o));
      tot += (uint32_t)__shfl_xor((int)tot, o);
    }
    const bool over = __ballot(tid < P && c > (uint32_t)M) != 0ull;
    if (tid < P) cnt[tid] = c;
    if (tid == 0) {
      s_state[0] = tot;
      s_state[1] = fl;
      s_state[2] = over ? 1u : 0u;
      s_state[3] = mk;
    }
  }
  __syncthreads();
  const uint32_t total = s_state[0], floor_key = s_state[1], max_key = s_state[3];
  int32_t* io = idx_out + (int64_t)r * k;
  float* vo = val_out ? val_out + (int64_t)r * k : nullptr;
  if (n <= k || total < (uint32_t)k) {
    select_block<float>(scores + rb, nullptr, n, k, io, vo);
    return;
  }
  if (s_state[2]) {
    finalize_lists<float>(r, scores, nv, S, k, P, chunk, bcnt, cval, cid, idx_out, val_out, tau_used);
    return;
  }
  uint32_t key[LF_E];
  bool valid[LF_E];
#pragma unroll
  for (int e = 0; e < LF_E; ++e) {
    valid[e] = rg[e] < P && (uint32_t)pos[e] < cnt[min(rg[e], P - 1)];
    key[e] = valid[e] ? ord_f32(val[e]) : 0u;
  }
  // every unlisted entry of a region lies below its threshold, so the top k lies
  // among the lists exactly when at least k listed keys reach the largest
  // threshold; T is then the kth of those, and at most max_key
  uint32_t T, n_above;
  bool ties_all;
  if (floor_key > max_key ||
      !block_kth_bounded<TK_THREADS, LF_E>(key, valid, (uint32_t)k, floor_key, max_key, histA, histB, bmaxA, bmaxB,
                                           wsum, res4, &T, &n_above, &ties_all)) {
    select_block<float>(scores + rb, nullptr, n, k, io, vo);
    return;
  }
  // every key above T, and the first (k - n_above) equal to T in list order
  bool sel[LF_E];
  uint32_t nsel = 0;
  if (ties_all) {
#pragma unroll
    for (int e = 0; e < LF_E; ++e) {
      sel[e] = valid[e] && key[e] >= T;
      nsel += sel[e] ? 1u : 0u;
    }
  } else {
    uint32_t ties = 0;
#pragma unroll
    for (int e = 0; e < LF_E; ++e) ties += valid[e] && key[e] == T ? 1u : 0u;
    uint32_t tr = block_exclusive_scan<NW>(ties, scan1);
    const uint32_t need = (uint32_t)k - n_above;
#pragma unroll
    for (int e = 0; e < LF_E; ++e) {
      const bool tie = valid[e] && key[e] == T;
      sel[e] = (valid[e] && key[e] > T) || (tie && tr < need);
      tr += tie ? 1u : 0u;
      nsel += sel[e] ? 1u : 0u;
    }
  }
  uint32_t at = block_exclusive_scan<NW>(nsel, scan2);
#pragma unroll
  for (int e = 0; e < LF_E; ++e) {
    if (sel[e]) {
      io[at] = id[e];
      if (vo) vo[at] = val[e];
      ++at;
    }
  }
}

static int mb_chunks(int R, int S) {
  int p = (2048 + R - 1) / R;  // about eight workgroups per CU over the rows
  const int max_p = (S + MB_THREADS * MB_BATCH - 1) / (MB_THREADS * MB_BATCH);
  if (p > max_p) p = max_p;
  if (p > 256) p = 256;
  return p < 1 ? 1 : p;
}

static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// The selection on few long rows: every workgroup takes a region of TK_LOCAL_CHUNK
// scores of its row (16 a thread, entry e * 256 + tid, loads all in flight) and
// lists its entries above a threshold of its own (list_above_local_threshold);
// the finalize then selects among the lists.
constexpr int TK_LOCAL_CHUNK = LT_E * 256;

template <typename Sc>
__global__ __launch_bounds__(256) void topk_local_filter_kernel(const Sc* __restrict__ scores,
                                                                const int32_t* __restrict__ nv, int S, int k,
                                                                Sc* __restrict__ cval, int32_t* __restrict__ cid,
                                                                uint32_t* __restrict__ bcnt,
                                                                uint32_t* __restrict__ tau_used) {
  __shared__ __attribute__((aligned(16))) uint32_t scratch[24];
  const int r = blockIdx.y, p = blockIdx.x, P = gridDim.x, tid = threadIdx.x;
  int n_row = S;
  if (nv) n_row = min(max(nv[r], 0), S);
  const int lo = p * TK_LOCAL_CHUNK;
  const int n = max(min(n_row - lo, TK_LOCAL_CHUNK), 0);
  const Sc* row = scores + (int64_t)r * S + lo;
  Sc v[LT_E];
#pragma unroll
  for (int e = 0; e < LT_E; ++e) {
    const int i = e * 256 + tid;
    v[e] = i < n ? row[i] : (Sc)0;
  }
  list_above_local_threshold(v, n, k, P, p, cval + (int64_t)r * S + lo, cid + (int64_t)r * S + lo, lo,
                             bcnt + (int64_t)r * P + p, tau_used + (int64_t)r * 256, scratch);
}

// Workspace of the multi-workgroup selection: the row thresholds (the sampled one,
// or the regions' own: 256 words a row), the region counts (256 words a row), then
// the candidate values and ids (R x S each).
template <typename Sc>
static size_t topk_mb_ws_bytes(int R, int S) {
  return a256((size_t)R * 256 * 4) + a256((size_t)R * 256 * 4) + a256((size_t)R * S * sizeof(Sc)) +
         a256((size_t)R * S * 4);
}

bool topk_use_mb(int R, int S) { return R < 160 && S >= 16384; }

template <typename Sc>
static hipError_t launch_topk_mb(const Sc* scores, const int32_t* nv, int R, int S, int k, int32_t* idx, Sc* val,
                                 void* ws, hipStream_t st) {
  typedef typename ScoreTraits<Sc>::K K;
  uint8_t* p = (uint8_t*)ws;
  K* tau = (K*)p;
  p += a256((size_t)R * 256 * 4);
  uint32_t* bcnt = (uint32_t*)p;
  p += a256((size_t)R * 256 * 4);
  Sc* cval = (Sc*)p;
  p += a256((size_t)R * S * sizeof(Sc));
  int32_t* cid = (int32_t*)p;
  {
    // regions of LT_E x 256 scores, each listed above a threshold of its own
    const int Pl = (S + TK_LOCAL_CHUNK - 1) / TK_LOCAL_CHUNK;
    if (Pl <= 256) {
      uint32_t* tau_used = (uint32_t*)tau;
      topk_local_filter_kernel<Sc><<<dim3(Pl, R), 256, 0, st>>>(scores, nv, S, k, cval, cid, bcnt, tau_used);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if constexpr (sizeof(Sc) == 4) {
        return launch_topk_finalize_f32((const float*)scores, nv, R, S, k, Pl, TK_LOCAL_CHUNK, bcnt,
                                        (const float*)cval, cid, idx, (float*)val, tau_used, st);
      } else {
        topk_finalize_kernel<Sc><<<R, TK_THREADS, 0, st>>>(scores, nv, S, k, Pl, TK_LOCAL_CHUNK, bcnt, cval, cid,
                                                            idx, val, tau_used);
        return hipGetLastError();
      }
    }
  }
  const int P = mb_chunks(R, S);
  const int chunk = (S + P - 1) / P;
  topk_thresh_kernel<Sc><<<R, TK_THREADS, 0, st>>>(scores, nv, S, k, tau);
  topk_filter_kernel<Sc><<<dim3(P, R), MB_THREADS, 0, st>>>(scores, nv, S, k, chunk, tau, cval, cid, bcnt);
  topk_finalize_kernel<Sc><<<R, TK_THREADS, 0, st>>>(scores, nv, S, k, P, chunk, bcnt, cval, cid, idx, val,
                                                      nullptr);
  return hipGetLastError();
}

void topk_mb_layout(void* ws, int R, int S, uint32_t** thresholds, uint32_t** bcnt, float** cval, int32_t** cid) {
  uint8_t* p = (uint8_t*)ws;
  *thresholds = (uint32_t*)p;  // the threshold area: 256 words per row
  p += a256((size_t)R * 256 * 4);
  *bcnt = (uint32_t*)p;
  p += a256((size_t)R * 256 * 4);
  *cval = (float*)p;
  p += a256((size_t)R * S * sizeof(float));
  *cid = (int32_t*)p;
}

hipError_t launch_topk_finalize_f32(const float* scores, const int32_t* nv, int R, int S, int k, int P, int chunk,
                                    const uint32_t* bcnt, const float* cval, const int32_t* cid, int32_t* idx,
                                    float* val, const uint32_t* tau_used, hipStream_t st) {
  if (tau_used && P >= 1 && P <= LF_MAXP) {
    topk_finalize_local_kernel<<<R, TK_THREADS, 0, st>>>(scores, nv, S, k, P, chunk, bcnt, cval, cid, idx, val,
                                                         tau_used);
    return hipGetLastError();
  }
  topk_finalize_kernel<float><<<R, TK_THREADS, 0, st>>>(scores, nv, S, k, P, chunk, bcnt, cval, cid, idx, val,
                                                        tau_used);
  return hipGetLastError();
}

size_t topk_ws_bytes(int R, int S, int k) {
  (void)k;
  return topk_use_mb(R, S) ? topk_mb_ws_bytes<float>(R, S) : 0;
}

hipError_t launch_topk_f32(const float* scores, const int32_t* nv, int R, int S, int k, int32_t* idx, float* val,
                           void* ws, hipStream_t st) {
  if (topk_use_mb(R, S)) return launch_topk_mb<float>(scores, nv, R, S, k, idx, val, ws, st);
  topk_row_kernel<float><<<R, TK_THREADS, 0, st>>>(scores, S, nv, nullptr, S, k, idx, val);
  return hipGetLastError();
}

hipError_t launch_topk_f64(const double* scores, int64_t row_stride, const int32_t* nv, const int32_t* ids, int R,
                           int S, int k, int32_t* idx, double* val, hipStream_t st) {
  topk_row_kernel<double><<<R, TK_THREADS, 0, st>>>(scores, row_stride, nv, ids, S, k, idx, val);
  return hipGetLastError();
}

size_t topk_f64_rows_ws_bytes(int R, int S) { return topk_use_mb(R, S) ? topk_mb_ws_bytes<double>(R, S) : 0; }

hipError_t launch_topk_f64_rows(const double* scores, const int32_t* nv, int R, int S, int k, int32_t* idx,
                                double* val, void* ws, hipStream_t st) {
  if (topk_use_mb(R, S)) return launch_topk_mb<double>(scores, nv, R, S, k, idx, val, ws, st);
  return launch_topk_f64(scores, S, nv, nullptr, R, S, k, idx, val, st);
}

bool topk_f64_rows_listed(int R, int S, int* region) {
  *region = TK_LOCAL_CHUNK;
  return topk_use_mb(R, S) && (S + TK_LOCAL_CHUNK - 1) / TK_LOCAL_CHUNK <= 256;
}

void topk_mb_layout_f64(void* ws, int R, int S, uint32_t** thresholds, uint32_t** bcnt, double** cval,
                        int32_t** cid) {
  uint8_t* p = (uint8_t*)ws;
  *thresholds = (uint32_t*)p;
  p += a256((size_t)R * 256 * 4);
  *bcnt = (uint32_t*)p;
  p += a256((size_t)R * 256 * 4);
  *cval = (double*)p;
  p += a256((size_t)R * S * sizeof(double));
  *cid = (int32_t*)p;
}

hipError_t launch_topk_finalize_f64(const double* scores, const int32_t* nv, int R, int S, int k, const uint32_t* bcnt,
                                    const double* cval, const int32_t* cid, int32_t* idx, double* val,
                                    const uint32_t* tau_used, hipStream_t st) {
  const int P = (S + TK_LOCAL_CHUNK - 1) / TK_LOCAL_CHUNK;
  topk_finalize_kernel<double><<<R, TK_THREADS, 0, st>>>(scores, nv, S, k, P, TK_LOCAL_CHUNK, bcnt, cval, cid, idx,
                                                         val, tau_used);
  return hipGetLastError();
}

// ---- static scratch for callers that cannot allocate ---------------------------
// The multi-workgroup selection's buffers (thresholds, region counts, candidate
// lists) in one file-scope device array per GPU.  Its name is a host-side stand-in
// in host code: the device address comes from hipGetSymbolAddress, looked up once
// per device and kept.  Every call on a device shares that device's array, which
// keeps the last call's contents (the kernels write every byte they read).
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int MAX_DEV = 64;
  static std::mutex mu;
  static void* addr[MAX_DEV] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace li
