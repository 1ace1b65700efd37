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
//      canonical order (score descending, id ascending), and they are written out.
// One workgroup of 1024 threads handles one row.
#include "common.h"
#include "launch.h"

namespace li {

constexpr int TK_THREADS = 1024;
constexpr int TK_BINS = 2048;  // 11-bit digits

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
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) sh_scan[wid] = v;
  __syncthreads();
  if (tid < 64) {
    uint32_t x = tid < TK_THREADS / 64 ? sh_scan[tid] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      uint32_t u = __shfl_up(x, o, 64);
      if (tid >= o) x += u;
    }
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

__device__ __forceinline__ bool sel_greater(const Sel& a, const Sel& b) {
  return a.key > b.key || (a.key == b.key && a.inv_id > b.inv_id);
}

template <typename S>
__global__ __launch_bounds__(TK_THREADS) void topk_row_kernel(const S* __restrict__ scores, int64_t row_stride,
                                                              const int32_t* __restrict__ nv,
                                                              const int32_t* __restrict__ ids, int S_len, int k,
                                                              int32_t* __restrict__ idx_out, S* __restrict__ val_out) {
  typedef typename ScoreTraits<S>::K K;
  constexpr int BITS = ScoreTraits<S>::BITS;
  __shared__ uint32_t hist[TK_BINS];
  __shared__ uint32_t sh_scan[64];
  __shared__ int sh_res[2];
  __shared__ uint32_t sh_count;
  __shared__ Sel list[LI_TOPK_MAX_DEV];

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const S* row = scores + (int64_t)r * row_stride;
  const int32_t* idrow = ids ? ids + (int64_t)r * row_stride : nullptr;
  int n = S_len;
  if (nv) n = min(max(nv[r], 0), S_len);
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
      for (int i = tid; i < n; i += TK_THREADS) {
        const K key = ScoreTraits<S>::ord(row[i]);
        if ((key & mask) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & dmask], 1u);
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
        for (int i = tid; i < n; i += TK_THREADS) {
          const K key = ScoreTraits<S>::ord(row[i]);
          if (key != prefix) continue;
          const uint32_t inv = ~(uint32_t)(idrow ? idrow[i] : i);
          if ((inv & imask) == iprefix) atomicAdd(&hist[(inv >> ishift) & dmask], 1u);
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
  // bitonic sort, descending
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
    idx_out[(int64_t)r * k + j] = oi;
    if (val_out) val_out[(int64_t)r * k + j] = ov;
  }
}

hipError_t launch_topk_f32(const float* scores, const int32_t* nv, int R, int S, int k, int32_t* idx, float* val,
                           hipStream_t st) {
  topk_row_kernel<float><<<R, TK_THREADS, 0, st>>>(scores, S, nv, nullptr, S, k, idx, val);
  return hipGetLastError();
}

hipError_t launch_topk_f64(const double* scores, int64_t row_stride, const int32_t* nv, const int32_t* ids, int R,
                           int S, int k, int32_t* idx, double* val, hipStream_t st) {
  topk_row_kernel<double><<<R, TK_THREADS, 0, st>>>(scores, row_stride, nv, ids, S, k, idx, val);
  return hipGetLastError();
}

}  // namespace li
