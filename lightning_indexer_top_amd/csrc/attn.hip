// Sparse attention over the selected latent rows for gfx950.
//
// "Long context", llm-serving.xyz lecture 03, section "The Architectural Answer",
// paragraph "Stage 2, sparse main attention": exact attention over only the top-k
// selected entries; section "Sparsity Is a Systems Feature: The Blast Radius",
// "Kernel layer": an MQA-shaped kernel that gathers the rows by token index.  Each
// selected row is a 576-element latent shared by every query head; keys use all 576
// elements and values the first 512.
//
// One workgroup of 8 waves handles one sequence and 32 query heads, two waves per
// SIMD.  Selected rows arrive 32 at a time (a chunk) by direct global-to-LDS loads
// into a ring of NBUF chunk buffers.  Per chunk:
//   logits  S^T[row, head] = K . Q^T as four 16 x 16 tiles (row half x head half),
//           each split over two waves by alternate 32-element K-steps
//           (v_mfma_f32_16x16x32_bf16); the second wave's partial sum goes
//           through LDS to the first, which owns the tile's softmax;
//   softmax in base 2 against a per-head reference maximum that moves only when a
//           logit exceeds it by more than 2^8 (then the outputs and sums are
//           rescaled), so the common chunk needs no cross-wave maximum;
//   values  O^T[dv, head] += V^T . P^T with v_mfma_f32_32x32x16_bf16, each wave
//           owning 64 of the 512 value columns; V^T comes from the same LDS rows by
//           transpose reads, P^T (bf16) from a small LDS tile.
// The chunks are software-pipelined: the logits of chunk c + 1 are computed beside
// the softmax of chunk c, with two workgroup barriers per chunk.

#include "common.h"
#include "launch.h"

namespace li {

constexpr int ATTN_NBUF = 4;  // chunk buffers

constexpr int AT_DQK = 576;
constexpr int AT_DV = 512;
constexpr int AT_CH = 32;                   // rows per chunk
constexpr int AT_RB = 2 * AT_DQK;           // bytes per row
constexpr int AT_PPR = AT_RB / 16;          // 16-byte pieces per row (72)
constexpr int AT_CHB = AT_CH * AT_RB;       // bytes per chunk buffer
constexpr int AT_KMAX = 2048;               // selected rows per sequence at most
constexpr int AT_PHS = 80;                  // LDS bytes per head of the probability tile
constexpr int AT_OSTR = 2 * AT_DV + 16;     // LDS bytes per head of the output staging
constexpr float AT_MARGIN = 8.0f;           // reference-maximum slack, base-2 units
static_assert(AT_CH * AT_PPR == 36 * 64, "36 load instructions of 64 pieces per chunk");

// The pieces of a row are swizzled inside each run of 8: piece p of row r sits in
// slot 72 r + (p & ~7) + ((p ^ at_sw(r)) & 7).  A row is 1152 bytes (9 x 128), so
// every row starts in the same 128-byte bank window and the swizzle alone spreads
// the reads: at_sw takes 8 different values over any 8 consecutive rows (the 16-byte
// logit operand reads of 8 lanes, 8 rows, one piece each), puts rows r and r + 8
// of one parity on complementary values (16 lanes over the 256-byte window), and
// gives rows 4 q .. 4 q + 3 four values that differ in bits 1 and 2 (a transpose
// read of 16 lanes: 4 rows x 2 adjacent pieces).
__device__ __forceinline__ int at_sw(int r) { return ((((r & 3) << 1) | ((r >> 2) & 1)) ^ ((r >> 2) & 2)); }

// Workgroup barrier after this wave's LDS accesses have completed.  Written out so
// that no fence makes the wave wait for its row loads still in flight.
__device__ __forceinline__ void at_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Reads of the chunk buffers are written out as well (the compiler would make each
// of them wait for every row load in flight), and wait for themselves before the
// statement ends: the nine 16-byte logit operands at ka + 128 i, then the eight
// transpose reads (ds_read_b64_tr_b16: in each group of 16 lanes, lane 4 a + b
// receives element b of the 4-element rows read by lanes a, a + 4, a + 8, a + 12)
// of the value operands, v[4 t + e] at a_t(e & 1) plus 16 rows (18432 bytes) for
// e >= 2; then six 4-byte reads of row indices (ia[i] -> id[i]) for the loads to come.
__device__ __forceinline__ void at_read_kv(i32x4 (&r)[9], i32x2 (&v)[8], int (&id)[6], uint32_t ka, uint32_t a00,
                                           uint32_t a01, uint32_t a10, uint32_t a11, const uint32_t (&ia)[6]) {
  asm volatile(
      "ds_read_b128 %0, %23\n\t"
      "ds_read_b128 %1, %23 offset:128\n\t"
      "ds_read_b128 %2, %23 offset:256\n\t"
      "ds_read_b128 %3, %23 offset:384\n\t"
      "ds_read_b128 %4, %23 offset:512\n\t"
      "ds_read_b128 %5, %23 offset:640\n\t"
      "ds_read_b128 %6, %23 offset:768\n\t"
      "ds_read_b128 %7, %23 offset:896\n\t"
      "ds_read_b128 %8, %23 offset:1024\n\t"
      "ds_read_b64_tr_b16 %9, %24\n\t"
      "ds_read_b64_tr_b16 %10, %25\n\t"
      "ds_read_b64_tr_b16 %11, %24 offset:18432\n\t"
      "ds_read_b64_tr_b16 %12, %25 offset:18432\n\t"
      "ds_read_b64_tr_b16 %13, %26\n\t"
      "ds_read_b64_tr_b16 %14, %27\n\t"
      "ds_read_b64_tr_b16 %15, %26 offset:18432\n\t"
      "ds_read_b64_tr_b16 %16, %27 offset:18432\n\t"
      "ds_read_b32 %17, %28\n\t"
      "ds_read_b32 %18, %29\n\t"
      "ds_read_b32 %19, %30\n\t"
      "ds_read_b32 %20, %31\n\t"
      "ds_read_b32 %21, %32\n\t"
      "ds_read_b32 %22, %33\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
        "=&v"(r[8]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
        "=&v"(v[7]), "=&v"(id[0]), "=&v"(id[1]), "=&v"(id[2]), "=&v"(id[3]), "=&v"(id[4]), "=&v"(id[5])
      : "v"(ka), "v"(a00), "v"(a01), "v"(a10), "v"(a11), "v"(ia[0]), "v"(ia[1]), "v"(ia[2]), "v"(ia[3]), "v"(ia[4]),
        "v"(ia[5])
      : "memory");
}

// The probability operands of the value product (two 16-byte reads) and the
// rescale flag, read together.
__device__ __forceinline__ void at_read_p(i32x4& p0, i32x4& p1, int& flag, uint32_t pa, uint32_t fa) {
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b128 %1, %3 offset:32\n\t"
      "ds_read_b32 %2, %4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(p0), "=&v"(p1), "=&v"(flag)
      : "v"(pa), "v"(fa)
      : "memory");
}

// The nine 16-byte operands at a + 128 i (the query's, read once).
__device__ __forceinline__ void at_read_k(i32x4 (&r)[9], uint32_t a) {
  asm volatile(
      "ds_read_b128 %0, %9\n\t"
      "ds_read_b128 %1, %9 offset:128\n\t"
      "ds_read_b128 %2, %9 offset:256\n\t"
      "ds_read_b128 %3, %9 offset:384\n\t"
      "ds_read_b128 %4, %9 offset:512\n\t"
      "ds_read_b128 %5, %9 offset:640\n\t"
      "ds_read_b128 %6, %9 offset:768\n\t"
      "ds_read_b128 %7, %9 offset:896\n\t"
      "ds_read_b128 %8, %9 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
        "=&v"(r[8])
      : "v"(a)
      : "memory");
}

// s_waitcnt vmcnt(n) for the counts the row-load pipeline uses (0 and multiples
// of 4 or 5 up to 15); any other count waits for everything.
__device__ __forceinline__ void at_wait_loads(int n) {
  switch (n) {
    case 15: LI_WAIT_VMCNT(15); break;
    case 12: LI_WAIT_VMCNT(12); break;
    case 10: LI_WAIT_VMCNT(10); break;
    case 8: LI_WAIT_VMCNT(8); break;
    case 5: LI_WAIT_VMCNT(5); break;
    case 4: LI_WAIT_VMCNT(4); break;
    default: LI_WAIT_VMCNT(0); break;
  }
}

__device__ __forceinline__ void at_write_zero(uint32_t a) {
  const i32x4 z = {0, 0, 0, 0};
  asm volatile("ds_write_b128 %0, %1" : : "v"(a), "v"(z) : "memory");
}

// PAGED: the latent rows live in a pool read at page size 1 ("Long context",
// section "Sparsity Is a Systems Feature: The Blast Radius", paragraph "KV-cache
// management": the token-level sparse read takes pages of one token);
// slot_table[b * max_slots + s] is the pool row of token s of sequence b.  Slots
// outside [0, num_slots) are clamped into it.
template <int NBUF, bool PAGED>
__global__ __launch_bounds__(512) void sparse_attn_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ kv,
                                                          const int32_t* __restrict__ idx, int B, int Hq, int S, int k,
                                                          float tau, uint16_t* __restrict__ out,
                                                          float* __restrict__ lse,
                                                          const int32_t* __restrict__ slot_table, int max_slots,
                                                          int num_slots) {
  __shared__ __attribute__((aligned(1024))) uint8_t kvbuf[NBUF * AT_CHB];
  __shared__ int sidx[AT_KMAX];
  __shared__ f32x4 spart[4][64];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[32 * AT_PHS];
  __shared__ float mx[2][32];
  __shared__ int sflag;

  // block -> (sequence, head tile): the head tiles of one sequence land on blocks
  // 8 apart, which the dispatcher places on the same XCD, so they share its L2.
  const int nt = Hq / 32;
  const int L = blockIdx.x;
  const int xcd = L & 7, round = L >> 3;
  const int ht = round % nt;
  const int b = (round / nt) * 8 + xcd;
  if (b >= B) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;  // 16 x 16 tile: lane group, column
  const int hf = lane >> 5, ho = lane & 31;  // 32 x 32 tile: lane half, column (= head)
  const int tile = wave & 3, rh = tile >> 1, hh = tile & 1, kh = wave >> 2;
  const int hs = 16 * hh + c16;  // head of this lane's logits
  i32x4 qb[9];                   // Q^T operands, read from LDS in the prologue

  // the selected rows' indices, -1 for entries that select nothing
  {
    const int32_t* irow = idx + (int64_t)b * k;
    for (int i = tid; i < k; i += 512) {
      const int id = irow[i];
      int v = (id >= 0 && id < S) ? id : -1;
      if constexpr (PAGED) {
        if (v >= 0) v = min(max(slot_table[(int64_t)b * max_slots + v], 0), num_slots - 1);
      }
      sidx[i] = v;
    }
  }
  if (tid == 0) sflag = 0;
  LI_WAIT_VMCNT(0);  // no index load is left in the row-load counts
  __syncthreads();

  // Row loads: load instruction j (0..35) of a chunk fills slots 64 j .. 64 j + 63;
  // wave w issues j = w + 8 u.  Skipped and missing rows load row 0 and are zeroed
  // once landed.
  const int nd = wave < 4 ? 5 : 4;
  int drow[5], doff[5];
#pragma unroll
  for (int u = 0; u < 5; ++u) {
    const int s = 64 * (wave + 8 * u) + lane;
    const int r = s / AT_PPR;
    const int ps = s - AT_PPR * r;
    drow[u] = r;
    doff[u] = 16 * ((ps & ~7) | ((ps ^ at_sw(r)) & 7));
  }
  const uint8_t* kvb = (const uint8_t*)(kv + (PAGED ? 0 : (int64_t)b * S * AT_DQK));
  const uint32_t kv_lds = lds_addr(kvbuf);
  const int nch = (k + AT_CH - 1) / AT_CH;
  // the row indices of this wave's loads of chunk c (LDS reads), then the loads
  auto row_ids = [&](int c, int (&id)[5]) {
    const int c0 = c * AT_CH;
#pragma unroll
    for (int u = 0; u < 5; ++u) {
      const int row = c0 + drow[u];
      const int v = sidx[min(row, k - 1)];
      id[u] = row < k ? v : -1;
    }
  };
  auto issue_ids = [&](int c, const int* id) {  // id[0..4]
    const uint32_t lb = kv_lds + (uint32_t)((c % NBUF) * AT_CHB) + 1024u * wave;
#pragma unroll
    for (int u = 0; u < 5; ++u) {
      if (u < 4 || wave < 4) {
        const uint8_t* src = kvb + (int64_t)max(id[u], 0) * AT_RB + doff[u];
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(uintptr_t)(lb + 8192u * u), 16, 0, 0);
      }
    }
  };
  auto issue = [&](int c) {
    int id[5];
    row_ids(c, id);
    issue_ids(c, id);
  };
  // the 32 heads' query rows, laid out like a chunk, into buffer NBUF - 1 (before
  // that buffer's first chunk): the same slots, row = head
  auto issue_q = [&]() {
    const uint8_t* qb0 = (const uint8_t*)(q + ((int64_t)b * Hq + 32 * ht) * AT_DQK);
    const uint32_t lb = kv_lds + (uint32_t)((NBUF - 1) * AT_CHB) + 1024u * wave;
#pragma unroll
    for (int u = 0; u < 5; ++u) {
      if (u < 4 || wave < 4) {
        const uint8_t* src = qb0 + drow[u] * AT_RB + doff[u];
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(uintptr_t)(lb + 8192u * u), 16, 0, 0);
      }
    }
  };

  // per-lane LDS offsets inside a chunk buffer
  const int R = 16 * rh + c16;  // logit operand row
  const uint32_t koff = 16u * (AT_PPR * R + ((g ^ at_sw(R)) ^ (4 * kh)));
  uint32_t voff[2][2];
  {
    const int R0 = 4 * hf + ((lane >> 2) & 3);
    const int x = 2 * ((lane >> 4) & 1) + ((lane >> 1) & 1);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e1 = 0; e1 < 2; ++e1) {
        const int sw = at_sw(R0 + 8 * e1);  // the same for the rows 16 on
        voff[t][e1] = 16u * (AT_PPR * (R0 + 8 * e1) + 8 * wave + ((x ^ sw) ^ (4 * t))) + 8u * (lane & 1);
      }
  }
  const uint32_t pw_off = hs * AT_PHS + 2 * (16 * rh + 8 * (g & 1) + 4 * (g >> 1));
  const int pr_off = ho * AT_PHS + 16 * hf;

  // rows of chunk c that select something (bit r: row 32 c + r): the index read,
  // then the vote
  auto row_index = [&](int c) -> int {
    const int row = c * AT_CH + lane;
    const int id = sidx[min(row, k - 1)];
    return lane < AT_CH && row < k ? id : -1;
  };
  auto valid_rows = [&](int id) -> uint32_t { return (uint32_t)__ballot(id >= 0); };
  // once this wave's loads of chunk c have landed: zero the slots of the rows that
  // select nothing (vr: valid_rows(c))
  auto zero_fill = [&](int c, uint32_t vr) {
    if (vr != 0xFFFFFFFFu) {
      const uint32_t lb = kv_lds + (uint32_t)((c % NBUF) * AT_CHB) + 1024u * wave + 16u * lane;
#pragma unroll
      for (int u = 0; u < 5; ++u)
        if ((u < 4 || wave < 4) && !((vr >> drow[u]) & 1u)) at_write_zero(lb + 8192u * u);
    }
  };
  // chunk c's operands: the logit rows of this wave's 9 K-steps and the V^T values,
  // together with the row indices of chunk c + NBUF (this wave's loads, id[0..4])
  // and of chunk c + 1 (row c + 1 + lane, id[5])
  const uint32_t sidx_lds = lds_addr(sidx);
  auto read_chunk = [&](int c, i32x4 (&ka)[9], i32x2 (&vv)[8], int (&id)[6]) {
    const uint32_t bufa = kv_lds + (uint32_t)((c % NBUF) * AT_CHB);
    uint32_t ia[6];
#pragma unroll
    for (int u = 0; u < 5; ++u) ia[u] = sidx_lds + 4u * (uint32_t)min((c + NBUF) * AT_CH + drow[u], k - 1);
    ia[5] = sidx_lds + 4u * (uint32_t)min((c + 1) * AT_CH + lane, k - 1);
    at_read_kv(ka, vv, id, bufa + koff, bufa + voff[0][0], bufa + voff[0][1], bufa + voff[1][0], bufa + voff[1][1],
               ia);
#pragma unroll
    for (int u = 0; u < 5; ++u)
      if ((c + NBUF) * AT_CH + drow[u] >= k) id[u] = -1;
    if (lane >= AT_CH || (c + 1) * AT_CH + lane >= k) id[5] = -1;
  };
  // partial logits over the 9 K-steps, two accumulation chains
  auto logit_mfma = [&](const i32x4 (&ka)[9], f32x4& s0, f32x4& s1) {
    s0 = (f32x4){};
    s1 = (f32x4){};
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, ka[i]), bq = __builtin_bit_cast(bf16x8, qb[i]);
      if (i & 1)
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq, s1, 0, 0, 0);
      else
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq, s0, 0, 0, 0);
    }
  };
  auto write_p = [&](const float (&p)[4]) {
    const bf16x4 v = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
    *(bf16x4*)(pbuf + pw_off) = v;
  };

  // softmax in base 2: exp(tau x - m) == 2^(tau log2(e) x - m / ln 2)
  const float tau2 = tau * 1.4426950408889634f;
  float m_s = -INFINITY, l_s = 0.0f, m_o = -INFINITY;
  f32x16 o[2];
  o[0] = (f32x16){};
  o[1] = (f32x16){};
  f32x4 sown;  // this wave's partial logits of the next chunk
  uint32_t vr_c = 0, vr_c1 = 0;  // valid rows of the current and the next chunk
  const uint32_t pr_lds = lds_addr(pbuf) + pr_off, flag_lds = lds_addr(&sflag);

  // One step of the software pipeline over chunks.  Chunk c is loaded during step
  // c - NBUF - 1 (the first NBUF + 1 up front); its logit and value operands are
  // read in phase A of step c - 1, which frees its buffer for chunk c + NBUF; its
  // softmax runs in phase A and its value product in phase B of step c.  Two
  // barriers per step: Y (partial logits and probabilities are in LDS) and X (the
  // chunk after next has landed).  vcur: chunk c's value operands; vnext receives
  // chunk c + 1's.
  auto step = [&](int c, const i32x2 (&vcur)[8], i32x2 (&vnext)[8]) {
    // ---- phase A: logits of chunk c + 1 (MFMA) beside the softmax of chunk c
    f32x4 s = sown;
    const uint32_t vrow = vr_c;
    if (!kh) s += spart[tile][lane];
    // (with the operands: the row indices of the loads issued after barrier Y, and
    // chunk c + 2's)
    int nid[6];
    nid[5] = -1;
    const bool load_next = c + NBUF + 1 < nch;
    f32x4 s0, s1;
    const bool more = c + 1 < nch;
    if (more) {
      i32x4 ka[9];
      read_chunk(c + 1, ka, vnext, nid);
      logit_mfma(ka, s0, s1);
    }
    const int rid2 = nid[5];
    // the tile's owner: logits of rows 16 rh + 4 g + j (j < 4), head hs
    float st[4], lsum = 0.0f;
    if (!kh) {
      bool ex = false;
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * rh + 4 * g + j;
        st[j] = ((vrow >> row) & 1u) ? s[j] * tau2 : -INFINITY;
        ex |= st[j] > m_s + AT_MARGIN;
        p[j] = st[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(st[j] - m_s);
        lsum += p[j];
      }
      write_p(p);
      if (__ballot(ex) != 0ull && lane == 0) sflag = c + 1;
    }
    if (more) sown = s0 + s1;
    at_barrier();
    // chunk c + 1 has been read by every wave: its buffer takes chunk c + NBUF + 1
    if (load_next) issue_ids(c + NBUF + 1, nid);

    // ---- phase B: value product of chunk c, loads of chunk c + NBUF + 1
    i32x4 pp0, pp1;
    int flag;
    at_read_p(pp0, pp1, flag, pr_lds, flag_lds);
    if (flag == c + 1) {
      // some logit passed its head's reference maximum by the margin: move the
      // references to the exact maxima and recompute this chunk's probabilities
      if (!kh) {
        float ml = fmaxf(fmaxf(st[0], st[1]), fmaxf(st[2], st[3]));
        ml = fmaxf(ml, __shfl_xor(ml, 16, WAVE));
        ml = fmaxf(ml, __shfl_xor(ml, 32, WAVE));
        if (g == 0) mx[rh][hs] = ml;
      }
      at_barrier();
      {
        const float mn = fmaxf(m_o, fmaxf(mx[0][ho], mx[1][ho]));
        const float al = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_o - mn);
        m_o = mn;
        if (__ballot(al != 1.0f) != 0ull) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[t][r] *= al;
        }
      }
      if (!kh) {
        const float mn = fmaxf(m_s, fmaxf(mx[0][hs], mx[1][hs]));
        const float al = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_s - mn);
        m_s = mn;
        float p[4];
        lsum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[j] = st[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(st[j] - mn);
          lsum += p[j];
        }
        l_s = l_s * al + lsum;
        write_p(p);
      }
      at_barrier();
      pp0 = *(const i32x4*)(pbuf + pr_off);
      pp1 = *(const i32x4*)(pbuf + pr_off + 32);
    } else if (!kh) {
      l_s += lsum;
    }
    // O^T[dv, head] += V^T . P^T over the chunk's two 16-row K-steps
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const i32x4 a4 = {vcur[4 * t + 2 * s2].x, vcur[4 * t + 2 * s2].y, vcur[4 * t + 2 * s2 + 1].x,
                          vcur[4 * t + 2 * s2 + 1].y};
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4),
                                                       __builtin_bit_cast(bf16x8, s2 ? pp1 : pp0), o[t], 0, 0, 0);
      }
    }
    // the second wave of each tile hands over its partial logits of chunk c + 1
    // (read in phase A of the next step)
    if (kh && more) spart[tile][lane] = sown;
    const uint32_t vr2 = valid_rows(rid2);
    if (c + 2 < nch) {
      at_wait_loads(nd * (min(nch - 1, c + NBUF + 1) - (c + 2)));
      zero_fill(c + 2, vr2);
    }
    vr_c = vr_c1;
    vr_c1 = vr2;
    at_barrier();
  };

  // prologue: chunks 0 and 1, the query rows (into buffer NBUF - 1) and chunks
  // 2 .. NBUF - 2 in flight; once chunks 0, 1 and the query have landed, the Q^T
  // operands and chunk 0's operands and logits; then chunks NBUF - 1 and NBUF
  i32x2 va[8], vb[8];
  issue(0);
  if (1 < nch) issue(1);
  issue_q();
  for (int c = 2; c < NBUF - 1 && c < nch; ++c) issue(c);
  vr_c = valid_rows(row_index(0));
  vr_c1 = valid_rows(row_index(1));
  at_wait_loads(nd * max(0, min(nch - 1, NBUF - 2) - 1));
  zero_fill(0, vr_c);
  if (1 < nch) zero_fill(1, vr_c1);
  at_barrier();
  {
    // Q^T operand of this wave's K-steps 2 i + kh (dims 64 i + 32 kh + 8 g .. + 7 of
    // head hs)
    at_read_k(qb, kv_lds + (uint32_t)((NBUF - 1) * AT_CHB) + 16u * (AT_PPR * hs + ((g ^ at_sw(hs)) ^ (4 * kh))));
    i32x4 ka[9];
    int unused[6];
    f32x4 s0, s1;
    read_chunk(0, ka, va, unused);
    logit_mfma(ka, s0, s1);
    sown = s0 + s1;
    if (kh) spart[tile][lane] = sown;
  }
  at_barrier();
  // every wave has its query operands and chunk 0's: their buffers take chunks
  // NBUF - 1 and NBUF (chunk 1 has landed and is zero-filled already)
  for (int c = NBUF - 1; c <= NBUF && c < nch; ++c) issue(c);
  for (int c = 0; c < nch; c += 2) {
    step(c, va, vb);
    if (c + 1 < nch) step(c + 1, vb, va);
  }

  // the softmax sums: the four lane groups of each tile owner, then the two row
  // halves (the last step ended with a barrier, so mx is free)
  if (!kh) {
    float l = l_s;
    l += __shfl_xor(l, 16, WAVE);
    l += __shfl_xor(l, 32, WAVE);
    if (g == 0) mx[rh][hs] = l;
  }
  at_barrier();
  const float lt = mx[0][ho] + mx[1][ho];
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  // normalised outputs staged through LDS as [head][dv] bf16, then stored 16 bytes
  // per lane
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dv = 64 * wave + 32 * t + 8 * r4 + 4 * hf;
      const bf16x4 v = {(__bf16)(o[t][4 * r4] * inv), (__bf16)(o[t][4 * r4 + 1] * inv),
                        (__bf16)(o[t][4 * r4 + 2] * inv), (__bf16)(o[t][4 * r4 + 3] * inv)};
      *(bf16x4*)(kvbuf + ho * AT_OSTR + 2 * dv) = v;
    }
  }
  at_barrier();
  uint16_t* obase = out + ((int64_t)b * Hq + 32 * ht) * AT_DV;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int pc = tid + 512 * u;
    const int h = pc >> 6, part = pc & 63;
    *(uint4*)(obase + (int64_t)h * AT_DV + 8 * part) = *(const uint4*)(kvbuf + h * AT_OSTR + 16 * part);
  }
  if (lse && wave == 0 && hf == 0)
    lse[(int64_t)b * Hq + 32 * ht + ho] = lt > 0.0f ? (m_o + log2f(lt)) * 0.6931471805599453f : -INFINITY;
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
  sparse_attn_kernel<ATTN_NBUF, false><<<blocks, 512, 0, st>>>(q, kv, idx, B, Hq, S, k, sm_scale, out, lse, nullptr, 0,
                                                               0);
  return hipGetLastError();
}

hipError_t launch_attn_paged(const uint16_t* q, const uint16_t* kv_pool, const int32_t* slot_table, int max_slots,
                             int num_slots, const int32_t* idx, int B, int Hq, int S, int k, float sm_scale,
                             uint16_t* out, float* lse, hipStream_t st) {
  const int nt = Hq / 32;
  const int blocks = ((B + 7) / 8) * 8 * nt;
  sparse_attn_kernel<ATTN_NBUF, true><<<blocks, 512, 0, st>>>(q, kv_pool, idx, B, Hq, S, k, sm_scale, out, lse,
                                                              slot_table, max_slots, num_slots);
  return hipGetLastError();
}

}  // namespace li
