// Sparse attention over the selected latent rows for gfx950.
//
// "Long context", llm-serving.xyz lecture 03, section "The Architectural Answer",
// paragraph "Stage 2, sparse main attention": exact attention over only the top-k
// selected entries; section "Sparsity Is a Systems Feature: The Blast Radius",
// "Kernel layer": an MQA-shaped kernel that gathers the rows by token index.  Each
// selected row is a 576-element latent shared by every query head; keys use all 576
// elements and values the first 512.
//
// One workgroup of 8 waves handles one sequence and 32 query heads, as two
// independent halves of four waves: half h takes chunks h, h + 2, h + 4, ... (a
// chunk is 32 selected rows), each into its own two of the four LDS chunk buffers
// (direct global-to-LDS loads, the next chunk in flight while one is computed), and
// its four waves meet at barriers of their own (an LDS counter), so the two waves
// that share a SIMD belong to different halves and one runs while the other waits.
// Per chunk, wave w of a half:
//   logits  one 16 x 16 tile S^T[row, head] = K . Q^T (rows 16 (w >> 1) .., heads
//           16 (w & 1) ..) over all 18 K-steps (v_mfma_f32_16x16x32_bf16), the
//           query operand in VGPRs;
//   softmax in base 2 against a per-head reference maximum that moves only when a
//           logit exceeds it by more than 2^8 (a flag in LDS then sends the half's
//           waves through the rescale path), probabilities (bf16) into the half's
//           LDS tile;
//   values  O^T[dv, head] += V^T . P^T for its 128 of the 512 value columns and all
//           32 heads (v_mfma_f32_32x32x16_bf16), V^T by transpose reads
//           (ds_read_b64_tr_b16).
// At the end the halves' outputs, reference maxima and sums are merged through LDS.

#include "common.h"
#include "launch.h"

namespace li {

constexpr int AT_DQK = 576;
constexpr int AT_DV = 512;
constexpr int AT_CH = 32;                   // rows per chunk
constexpr int AT_RB = 2 * AT_DQK;           // bytes per row
constexpr int AT_PPR = AT_RB / 16;          // 16-byte pieces per row (72)
constexpr int AT_CHB = AT_CH * AT_RB;       // bytes per chunk buffer
constexpr int AT_NBUF = 4;                  // chunk buffers: two per half
constexpr int AT_KMAX = 2048;               // selected rows per sequence at most
constexpr int AT_PHS = 80;                  // LDS bytes per head of the probability tile
constexpr int AT_OSTR = 2 * AT_DV + 16;     // LDS bytes per head of the output staging
constexpr float AT_MARGIN = 8.0f;           // reference-maximum slack, base-2 units
constexpr int AT_SPIN = 1 << 22;            // bound of a half-barrier wait (never reached)
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

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Workgroup barrier after this wave's LDS accesses have completed.  Written out so
// that no fence makes the wave wait for its row loads still in flight.
__device__ __forceinline__ void at_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Barrier of the four waves of a half: once this wave's LDS accesses have completed,
// one lane adds 1 to the half's counter, then the wave waits until the counter
// reaches `target` (4 x the number of such barriers the half has passed).  Every
// wave of the half passes the same sequence of barriers; the wait is bounded.
__device__ __forceinline__ void at_half_barrier(uint32_t ctr, uint32_t target, int lane) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (lane == 0) {
    const uint32_t one = 1;
    asm volatile("ds_add_u32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(ctr), "v"(one) : "memory");
  }
  // (no s_sleep between the reads: waking from it measured 0.6 us slower per launch)
  for (int i = 0; i < AT_SPIN; ++i) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(ctr) : "memory");
    if (__builtin_amdgcn_readfirstlane(v) >= target) break;
  }
}

// Reads of the chunk buffers are written out (the compiler would make each of them
// wait for every row load in flight) and wait for themselves before the statement
// ends.
// The nine 16-byte operands at a + 128 i.
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

// Eight transpose reads (ds_read_b64_tr_b16: in each group of 16 lanes, lane 4 a + b
// receives element b of the 4-element rows read by lanes a, a + 4, a + 8, a + 12) of
// value operands: v[4 t + e] at a_t(e & 1), plus 16 rows (18432 bytes) for e >= 2.
__device__ __forceinline__ void at_read_v(i32x2 (&v)[8], uint32_t a00, uint32_t a01, uint32_t a10, uint32_t a11) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:18432\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:18432\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %11\n\t"
      "ds_read_b64_tr_b16 %6, %10 offset:18432\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:18432\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(a00), "v"(a01), "v"(a10), "v"(a11)
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

__device__ __forceinline__ int at_read_i32(uint32_t a) {
  int r;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r) : "v"(a) : "memory");
  return r;
}

__device__ __forceinline__ float at_read_f32(uint32_t a) {
  float r;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r) : "v"(a) : "memory");
  return r;
}

__device__ __forceinline__ void at_write_f32(uint32_t a, float v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(a), "v"(v) : "memory");
}

// PAGED: the latent rows live in a pool read at page size 1 ("Long context",
// section "Sparsity Is a Systems Feature: The Blast Radius", paragraph "KV-cache
// management": the token-level sparse read takes pages of one token);
// slot_table[b * max_slots + s] is the pool row of token s of sequence b.  Slots
// outside [0, num_slots) are clamped into it.
template <bool PAGED>
__global__ __launch_bounds__(512) void sparse_attn_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ kv,
                                                          const int32_t* __restrict__ idx, int B, int Hq, int S, int k,
                                                          float tau, uint16_t* __restrict__ out,
                                                          float* __restrict__ lse,
                                                          const int32_t* __restrict__ slot_table, int max_slots,
                                                          int num_slots) {
  __shared__ __attribute__((aligned(1024))) uint8_t kvbuf[AT_NBUF * AT_CHB];
  __shared__ __attribute__((aligned(16))) int sidx[AT_KMAX];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][32 * AT_PHS];
  __shared__ float mx[2][2][32];
  __shared__ int sflag[2];
  __shared__ uint32_t hbar[2];

  // block -> (sequence, head tile): the head tiles of one sequence land on blocks
  // 8 apart, which the dispatcher places on the same XCD, so they share its L2.
  const int nt = Hq / 32;
  const int L = blockIdx.x;
  const int xcd = L & 7, round = L >> 3;
  const int ht = round % nt;
  const int b = (round / nt) * 8 + xcd;
  if (b >= B) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave >> 2, w4 = wave & 3;
  const int g = lane >> 4, c16 = lane & 15;  // 16 x 16 tile: lane group, column
  const int hf = lane >> 5, ho = lane & 31;  // 32 x 32 tile: lane half, column (= head)
  const int rh = w4 >> 1, hh = w4 & 1;       // this wave's logit tile
  const int hs = 16 * hh + c16;              // head of this lane's logits
  const int nch = (k + AT_CH - 1) / AT_CH;

  // the selected rows' indices (pool rows when paged), -1 for entries that select nothing
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
  if (tid < 2) {
    sflag[tid] = 0;
    hbar[tid] = 0;
  }
  LI_WAIT_VMCNT(0);  // no index load is left in the row-load counts
  __syncthreads();

  const uint8_t* kvb = (const uint8_t*)(kv + (PAGED ? 0 : (int64_t)b * S * AT_DQK));
  const uint32_t kv_lds = lds_addr(kvbuf), sidx_lds = lds_addr(sidx);
  // Row loads of a half's chunk: load instruction j (0..35) fills slots 64 j ..
  // 64 j + 63; wave w4 of the half issues j = w4 + 4 u.  Rows that select nothing load
  // row 0 and are zeroed once landed.
  // lane l's row of load u: (64 (w4 + 4 u) + l) / 72, i.e. row r0(u) for lanes below
  // bnd(u) and r0(u) + 1 above (a load instruction spans at most two rows)
  int drow[9];
  uint32_t doff[9];
#pragma unroll
  for (int u = 0; u < 9; ++u) {
    const int s = 64 * (w4 + 4 * u) + lane;
    const int r = s / AT_PPR;
    const int ps = s - AT_PPR * r;
    drow[u] = r;
    doff[u] = 16u * (uint32_t)((ps & ~7) | ((ps ^ at_sw(r)) & 7));
  }
  // the half's chunk c sits in buffer 2 half + (c / 2) % 2
  auto buf_of = [&](int c) -> uint32_t { return kv_lds + (uint32_t)((2 * half + ((c >> 1) & 1)) * AT_CHB); };
  // issue this wave's loads of chunk c; returns the chunk's valid rows (bit r: row
  // 32 c + r selects something), from one index read per lane
  auto issue = [&](int c) -> uint32_t {
    const int row = c * AT_CH + (lane & 31);
    int idv = at_read_i32(sidx_lds + 4u * (uint32_t)min(row, k - 1));
    if (row >= k) idv = -1;
    const uint32_t lb = buf_of(c) + 1024u * w4;
#pragma unroll
    for (int u = 0; u < 9; ++u) {
      const int j = w4 + 4 * u;
      const int r0 = (64 * j) / AT_PPR;
      const int bnd = AT_PPR * (r0 + 1) - 64 * j;
      const int i0 = __builtin_amdgcn_readlane(idv, r0), i1 = __builtin_amdgcn_readlane(idv, min(r0 + 1, 31));
      const int id = lane < bnd ? i0 : i1;
      const uint8_t* src = kvb + (int64_t)max(id, 0) * AT_RB + doff[u];
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(uintptr_t)(lb + 4096u * u), 16, 0, 0);
    }
    return (uint32_t)__ballot(lane < 32 && idv >= 0);
  };
  // once this wave's loads of chunk c have landed: zero the slots of the rows that
  // select nothing (vr: the chunk's valid rows)
  auto zero_fill = [&](int c, uint32_t vr) {
    if (vr != 0xFFFFFFFFu) {
      const uint32_t lb = buf_of(c) + 1024u * w4 + 16u * lane;
#pragma unroll
      for (int u = 0; u < 9; ++u) {
        if (!((vr >> drow[u]) & 1u)) {
          const i32x4 z = {0, 0, 0, 0};
          asm volatile("ds_write_b128 %0, %1" : : "v"(lb + 4096u * u), "v"(z) : "memory");
        }
      }
    }
  };

  // the 32 heads' query rows, laid out like a chunk, into buffer 3 (half 1's second
  // buffer) before its first chunk: every wave issues 4 or 5 of the 36 loads
  {
    const uint8_t* qb0 = (const uint8_t*)(q + ((int64_t)b * Hq + 32 * ht) * AT_DQK);
    const uint32_t lb = kv_lds + (uint32_t)(3 * AT_CHB) + 1024u * wave;
#pragma unroll
    for (int u = 0; u < 5; ++u) {
      if (u < 4 || wave < 4) {
        const int s = 64 * (wave + 8 * u) + lane;
        const int r = s / AT_PPR;
        const int ps = s - AT_PPR * r;
        const uint8_t* src = qb0 + r * AT_RB + 16 * ((ps & ~7) | ((ps ^ at_sw(r)) & 7));
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(uintptr_t)(lb + 8192u * u), 16, 0, 0);
      }
    }
  }
  // the first chunk of each half (buffers 0 and 2)
  uint32_t vr_cur = 0, vr_next = 0;
  if (half < nch) vr_cur = issue(half);

  // per-lane LDS offsets inside a chunk buffer
  // logit operand: row R = 16 rh + c16; K-steps 2 i (dims 64 i + 8 g ..) at koff0 +
  // 128 i, 2 i + 1 (dims 64 i + 32 + 8 g ..) at koff1 + 128 i
  const int R = 16 * rh + c16;
  const uint32_t koff0 = 16u * (uint32_t)(AT_PPR * R + (g ^ at_sw(R)));
  const uint32_t koff1 = 16u * (uint32_t)(AT_PPR * R + ((g ^ at_sw(R)) ^ 4));
  // value operands: columns 128 w4 + 64 tt + 32 t .. of rows R0 (+ 8 e1, + 16)
  uint32_t voff[2][2][2];
  {
    const int R0 = 4 * hf + ((lane >> 2) & 3);
    const int x = 2 * ((lane >> 4) & 1) + ((lane >> 1) & 1);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e1 = 0; e1 < 2; ++e1) {
          const int sw = at_sw(R0 + 8 * e1);  // the same for the rows 16 on
          voff[tt][t][e1] =
              16u * (uint32_t)(AT_PPR * (R0 + 8 * e1) + 16 * w4 + 8 * tt + ((x ^ sw) ^ (4 * t))) + 8u * (lane & 1);
        }
  }
  const uint32_t pb_lds = lds_addr(pbuf[half]);
  const uint32_t pw_off = pb_lds + (uint32_t)(hs * AT_PHS + 2 * (16 * rh + 8 * (g & 1) + 4 * (g >> 1)));
  const uint32_t pr_lds = pb_lds + (uint32_t)(ho * AT_PHS + 16 * hf);
  const uint32_t flag_lds = lds_addr(&sflag[half]), ctr_lds = lds_addr(&hbar[half]);
  uint32_t hgen = 0;  // half-barriers passed

  // the query operands, once the query rows (and the first chunks) have landed
  i32x4 qb0[9], qb1[9];
  LI_WAIT_VMCNT(0);
  if (half < nch) zero_fill(half, vr_cur);
  at_barrier();
  {
    const uint32_t qa = kv_lds + (uint32_t)(3 * AT_CHB) + 16u * (uint32_t)(AT_PPR * hs);
    at_read_k(qb0, qa + 16u * (uint32_t)(g ^ at_sw(hs)));
    at_read_k(qb1, qa + 16u * (uint32_t)((g ^ at_sw(hs)) ^ 4));
  }
  at_barrier();  // buffer 3 is free for half 1's second chunk

  // softmax in base 2: exp(tau x - m) == 2^(tau log2(e) x - m / ln 2)
  const float tau2 = tau * 1.4426950408889634f;
  float m_s = -INFINITY, l_s = 0.0f, m_o = -INFINITY;
  f32x16 o[2][2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int t = 0; t < 2; ++t) o[tt][t] = (f32x16){};

  for (int c = half; c < nch; c += 2) {
    // ---- the half's chunk c has landed (this wave's loads); zero the rows that
    // select nothing; every wave of the half is past chunk c - 2
    LI_WAIT_VMCNT(0);
    if (c != half) zero_fill(c, vr_cur);
    at_half_barrier(ctr_lds, 4u * ++hgen, lane);
    // its buffer of chunk c - 2 takes chunk c + 2
    if (c + 2 < nch) vr_next = issue(c + 2);
    const uint32_t buf = buf_of(c);

    // ---- logits of rows 16 rh + 4 g + j, head hs, over all 18 K-steps
    f32x4 s0 = {}, s1 = {};
    {
      i32x4 ka[9];
      at_read_k(ka, buf + koff0);
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, ka[i]), bq = __builtin_bit_cast(bf16x8, qb0[i]);
        if (i & 1)
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq, s1, 0, 0, 0);
        else
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq, s0, 0, 0, 0);
      }
      at_read_k(ka, buf + koff1);
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, ka[i]), bq = __builtin_bit_cast(bf16x8, qb1[i]);
        if (i & 1)
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq, s0, 0, 0, 0);
        else
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq, s1, 0, 0, 0);
      }
    }
    const f32x4 s = s0 + s1;
    float st[4], lsum = 0.0f;
    {
      bool ex = false;
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool valid = (vr_cur >> (16 * rh + 4 * g + j)) & 1u;
        st[j] = valid ? s[j] * tau2 : -INFINITY;
        ex |= st[j] > m_s + AT_MARGIN;
        p[j] = st[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(st[j] - m_s);
        lsum += p[j];
      }
      const bf16x4 v = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
      asm volatile("ds_write_b64 %0, %1" : : "v"(pw_off), "v"(__builtin_bit_cast(i32x2, v)) : "memory");
      if (__ballot(ex) != 0ull && lane == 0) {
        const int f = c + 1;
        asm volatile("ds_write_b32 %0, %1" : : "v"(flag_lds), "v"(f) : "memory");
      }
    }
    at_half_barrier(ctr_lds, 4u * ++hgen, lane);

    // ---- probabilities and flag; the rescale path when some logit passed its head's
    // reference maximum by the margin
    i32x4 pp0, pp1;
    int flag;
    at_read_p(pp0, pp1, flag, pr_lds, flag_lds);
    if (flag == c + 1) {
      // move the references to the exact maxima and recompute this chunk's probabilities
      float ml = fmaxf(fmaxf(st[0], st[1]), fmaxf(st[2], st[3]));
      ml = fmaxf(ml, __shfl_xor(ml, 16, WAVE));
      ml = fmaxf(ml, __shfl_xor(ml, 32, WAVE));
      if (g == 0) at_write_f32(lds_addr(&mx[half][rh][hs]), ml);
      at_half_barrier(ctr_lds, 4u * ++hgen, lane);
      {
        const float mn = fmaxf(m_o, fmaxf(at_read_f32(lds_addr(&mx[half][0][ho])),
                                          at_read_f32(lds_addr(&mx[half][1][ho]))));
        const float al = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_o - mn);
        m_o = mn;
        if (__ballot(al != 1.0f) != 0ull) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int r = 0; r < 16; ++r) o[tt][t][r] *= al;
        }
      }
      {
        const float mn = fmaxf(m_s, fmaxf(at_read_f32(lds_addr(&mx[half][0][hs])),
                                          at_read_f32(lds_addr(&mx[half][1][hs]))));
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
        const bf16x4 v = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
        asm volatile("ds_write_b64 %0, %1" : : "v"(pw_off), "v"(__builtin_bit_cast(i32x2, v)) : "memory");
      }
      at_half_barrier(ctr_lds, 4u * ++hgen, lane);
      at_read_p(pp0, pp1, flag, pr_lds, flag_lds);
    } else {
      l_s += lsum;
    }

    // ---- O^T[dv, head] += V^T . P^T over the chunk's two 16-row K-steps, for this
    // wave's two 64-column blocks
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      i32x2 vv[8];
      at_read_v(vv, buf + voff[tt][0][0], buf + voff[tt][0][1], buf + voff[tt][1][0], buf + voff[tt][1][1]);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const i32x4 a4 = {vv[4 * t + 2 * s2].x, vv[4 * t + 2 * s2].y, vv[4 * t + 2 * s2 + 1].x,
                            vv[4 * t + 2 * s2 + 1].y};
          o[tt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4),
                                                             __builtin_bit_cast(bf16x8, s2 ? pp1 : pp0), o[tt][t], 0,
                                                             0, 0);
        }
      }
    }
    vr_cur = vr_next;
  }

  // ---- merge the two halves: the softmax sums of each half (four lane groups of a
  // tile, then its two row halves), the reference maxima and the outputs of half 1
  // through LDS into half 0, which normalises and stores
  {
    float l = l_s;
    l += __shfl_xor(l, 16, WAVE);
    l += __shfl_xor(l, 32, WAVE);
    if (g == 0) at_write_f32(lds_addr(&mx[half][rh][hs]), l);
  }
  LI_WAIT_VMCNT(0);
  at_barrier();
  const float lh = at_read_f32(lds_addr(&mx[half][0][ho])) + at_read_f32(lds_addr(&mx[half][1][ho]));
  // half 1's outputs (64 per lane), reference maxima and sums, after the ring
  float* mg = (float*)kvbuf + (size_t)w4 * 66 * 64;
  if (half == 1) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mg[((tt * 2 + t) * 16 + r) * 64 + lane] = o[tt][t][r];
    mg[64 * 64 + lane] = m_o;
    mg[65 * 64 + lane] = lh;
  }
  __syncthreads();
  const float m1 = mg[64 * 64 + lane], l1 = mg[65 * 64 + lane];
  const float mm = fmaxf(m_o, m1);
  const float a0 = m_o == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_o - mm);
  const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - mm);
  const float lt = lh * a0 + l1 * a1;
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (half == 0) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          o[tt][t][r] = (o[tt][t][r] * a0 + mg[((tt * 2 + t) * 16 + r) * 64 + lane] * a1) * inv;
  }
  __syncthreads();  // the merge area is read; the staging below reuses the ring
  // normalised outputs staged through LDS as [head][dv] bf16, then stored 16 bytes
  // per lane
  if (half == 0) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int dv = 128 * w4 + 64 * tt + 32 * t + 8 * r4 + 4 * hf;
          const bf16x4 v = {(__bf16)o[tt][t][4 * r4], (__bf16)o[tt][t][4 * r4 + 1], (__bf16)o[tt][t][4 * r4 + 2],
                            (__bf16)o[tt][t][4 * r4 + 3]};
          *(bf16x4*)(kvbuf + ho * AT_OSTR + 2 * dv) = v;
        }
  }
  __syncthreads();
  uint16_t* obase = out + ((int64_t)b * Hq + 32 * ht) * AT_DV;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int pc = tid + 512 * u;
    const int h = pc >> 6, part = pc & 63;
    *(uint4*)(obase + (int64_t)h * AT_DV + 8 * part) = *(const uint4*)(kvbuf + h * AT_OSTR + 16 * part);
  }
  if (lse && half == 0 && w4 == 0 && hf == 0)
    lse[(int64_t)b * Hq + 32 * ht + ho] = lt > 0.0f ? (mm + log2f(lt)) * 0.6931471805599453f : -INFINITY;
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
  sparse_attn_kernel<false><<<blocks, 512, 0, st>>>(q, kv, idx, B, Hq, S, k, sm_scale, out, lse, nullptr, 0, 0);
  return hipGetLastError();
}

hipError_t launch_attn_paged(const uint16_t* q, const uint16_t* kv_pool, const int32_t* slot_table, int max_slots,
                             int num_slots, const int32_t* idx, int B, int Hq, int S, int k, float sm_scale,
                             uint16_t* out, float* lse, hipStream_t st) {
  const int nt = Hq / 32;
  const int blocks = ((B + 7) / 8) * 8 * nt;
  sparse_attn_kernel<true><<<blocks, 512, 0, st>>>(q, kv_pool, idx, B, Hq, S, k, sm_scale, out, lse, slot_table,
                                                   max_slots, num_slots);
  return hipGetLastError();
}

}  // namespace li
