// C ABI of the lightning-indexer library: host-side argument validation,
// workspace sizing and kernel launches on the caller's stream.  Nothing here
// allocates device memory or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/li.h"
#include "launch.h"

static_assert(LI_TOPK_NOALLOC_SCRATCH_BYTES == li::NOALLOC_SCRATCH_BYTES, "header and library agree");

namespace {

thread_local char g_err[256] = "";

li_status fail(li_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

li_status ok() {
  g_err[0] = 0;
  return LI_OK;
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

li_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LI_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// Shared validation of the indexer scoring arguments.
li_status check_score_args(const void* q, li_dtype qt, const float* w, const void* k, li_dtype kt, const float* ks,
                           const int32_t* nv, int B, int T, int S, int H, int d) {
  if (!q || !w || !k) return fail(LI_ERR_NULL, "q, w and k must be non-NULL");
  if (qt != LI_BF16 && qt != LI_F32) return fail(LI_ERR_DTYPE, "q_type must be LI_BF16 or LI_F32");
  if (kt != LI_BF16 && kt != LI_F32 && kt != LI_FP8_E4M3)
    return fail(LI_ERR_DTYPE, "k_type must be LI_FP8_E4M3, LI_BF16 or LI_F32");
  if (kt == LI_FP8_E4M3 && !ks) return fail(LI_ERR_NULL, "fp8 keys need k_scale");
  if (kt != LI_FP8_E4M3 && ks) return fail(LI_ERR_DTYPE, "k_scale is only accepted with fp8 keys");
  if (d != LI_INDEX_DIM) return fail(LI_ERR_SHAPE, "d must be %d (got %d)", LI_INDEX_DIM, d);
  if (H < 1 || H > 128) return fail(LI_ERR_SHAPE, "H must be in [1, 128] (got %d)", H);
  if (B < 1 || T < 1 || S < 1) return fail(LI_ERR_SHAPE, "B, T and S must be >= 1");
  if ((int64_t)B * T >= (1ll << 31) || (int64_t)B * T * S >= (1ll << 40))
    return fail(LI_ERR_SHAPE, "B*T*S too large");
  if (misaligned(q) || misaligned(w) || misaligned(k) || misaligned(ks) || misaligned(nv))
    return fail(LI_ERR_ALIGN, "device pointers must be 16-byte aligned");
  return LI_OK;
}

}  // namespace

extern "C" {

const char* li_status_string(li_status s) {
  switch (s) {
    case LI_OK: return "ok";
    case LI_ERR_NULL: return "null pointer";
    case LI_ERR_SHAPE: return "unsupported shape";
    case LI_ERR_DTYPE: return "unsupported dtype";
    case LI_ERR_ALIGN: return "misaligned pointer";
    case LI_ERR_WORKSPACE: return "workspace too small";
    case LI_ERR_LAUNCH: return "launch failed";
  }
  return "unknown status";
}

const char* li_last_error(void) { return g_err; }

const char* li_version(void) { return "lightning-indexer-gfx950 0.1"; }

li_status li_indexer_score(const void* q, li_dtype q_type, const float* w, const void* k, li_dtype k_type,
                           const float* k_scale, const int32_t* nv, int B, int T, int S, int H, int d, float* scores,
                           hipStream_t stream) {
  li_status s = check_score_args(q, q_type, w, k, k_type, k_scale, nv, B, T, S, H, d);
  if (s != LI_OK) return s;
  if (!scores) return fail(LI_ERR_NULL, "scores must be non-NULL");
  if (misaligned(scores)) return fail(LI_ERR_ALIGN, "scores must be 16-byte aligned");
  return launched(li::launch_score(q, q_type, w, k, k_type, k_scale, nv, B, T, S, H, scores, stream),
                  "li_indexer_score");
}

size_t li_topk_workspace_bytes(int R, int S, int k) {
  if (R < 1 || S < 1 || k < 1) return 0;
  return li::topk_ws_bytes(R, S, k);
}

li_status li_topk_select(const float* scores, const int32_t* nv, int R, int S, int k, int32_t* idx, float* val,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!scores || !idx) return fail(LI_ERR_NULL, "scores and idx must be non-NULL");
  if (R < 1 || S < 1) return fail(LI_ERR_SHAPE, "R and S must be >= 1");
  if (k < 1 || k > LI_TOPK_MAX) return fail(LI_ERR_SHAPE, "k must be in [1, %d] (got %d)", LI_TOPK_MAX, k);
  if ((int64_t)R * S >= (1ll << 40)) return fail(LI_ERR_SHAPE, "R*S too large");
  if (misaligned(scores) || misaligned(nv) || misaligned(idx) || misaligned(val))
    return fail(LI_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t need = li_topk_workspace_bytes(R, S, k);
  if (need && (!ws || ws_bytes < need)) return fail(LI_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if (misaligned(ws)) return fail(LI_ERR_ALIGN, "workspace must be 16-byte aligned");
  return launched(li::launch_topk_f32(scores, nv, R, S, k, idx, val, ws, stream), "li_topk_select");
}

li_status li_topk_select_noalloc(const float* scores, const int32_t* nv, int R, int S, int k, int32_t* idx,
                                 float* val, hipStream_t stream) {
  if (!scores || !idx) return fail(LI_ERR_NULL, "scores and idx must be non-NULL");
  if (R < 1 || S < 1) return fail(LI_ERR_SHAPE, "R and S must be >= 1");
  if (k < 1 || k > LI_TOPK_MAX) return fail(LI_ERR_SHAPE, "k must be in [1, %d] (got %d)", LI_TOPK_MAX, k);
  if ((int64_t)R * S >= (1ll << 40)) return fail(LI_ERR_SHAPE, "R*S too large");
  if (misaligned(scores) || misaligned(nv) || misaligned(idx) || misaligned(val))
    return fail(LI_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t need = li_topk_workspace_bytes(R, S, k);
  if (need > li::NOALLOC_SCRATCH_BYTES)
    return fail(LI_ERR_WORKSPACE, "this shape needs %zu bytes of scratch, more than the %zu of the static scratch",
                need, (size_t)li::NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need) {
    const hipError_t e = li::noalloc_scratch(&ws);
    if (e != hipSuccess) return fail(LI_ERR_LAUNCH, "static scratch lookup: %s", hipGetErrorString(e));
  }
  return launched(li::launch_topk_f32(scores, nv, R, S, k, idx, val, ws, stream), "li_topk_select_noalloc");
}

size_t li_indexer_topk_workspace_bytes(li_dtype q_type, li_dtype k_type, int B, int T, int S, int H, int topk) {
  if (B < 1 || T < 1 || S < 1 || H < 1 || topk < 1) return 0;
  return li::indexer_topk_ws_bytes(q_type, k_type, B, T, S, H, topk);
}

li_status li_indexer_topk(const void* q, li_dtype q_type, const float* w, const void* k, li_dtype k_type,
                          const float* k_scale, const int32_t* nv, int B, int T, int S, int H, int d, int topk,
                          int32_t* idx, float* val, void* ws, size_t ws_bytes, hipStream_t stream) {
  li_status s = check_score_args(q, q_type, w, k, k_type, k_scale, nv, B, T, S, H, d);
  if (s != LI_OK) return s;
  if (!idx) return fail(LI_ERR_NULL, "idx must be non-NULL");
  if (topk < 1 || topk > LI_TOPK_MAX) return fail(LI_ERR_SHAPE, "topk must be in [1, %d]", LI_TOPK_MAX);
  if (misaligned(idx) || misaligned(val)) return fail(LI_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t need = li::indexer_topk_ws_bytes(q_type, k_type, B, T, S, H, topk);
  if (need && (!ws || ws_bytes < need)) return fail(LI_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if (misaligned(ws)) return fail(LI_ERR_ALIGN, "workspace must be 16-byte aligned");
  return launched(li::launch_indexer_topk(q, q_type, w, k, k_type, k_scale, nv, B, T, S, H, topk, idx, val, ws,
                                          stream),
                  "li_indexer_topk");
}

li_status li_pool_keys(const void* k, li_dtype k_type, int B, int L, int d, int pool, uint8_t* codes,
                       float* scales, hipStream_t stream) {
  if (k_type != LI_BF16) return fail(LI_ERR_DTYPE, "token keys must be LI_BF16");
  if (d != LI_INDEX_DIM) return fail(LI_ERR_SHAPE, "d must be %d", LI_INDEX_DIM);
  if (pool != 1 && pool != 2 && pool != 4 && pool != 8) return fail(LI_ERR_SHAPE, "pool must be 1, 2, 4 or 8");
  if (B < 1 || L < 0) return fail(LI_ERR_SHAPE, "need B >= 1 and L >= 0");
  if ((int64_t)B * L >= (1ll << 40)) return fail(LI_ERR_SHAPE, "B*L too large");
  if (L / pool == 0) return ok();  // no complete block: nothing to write
  if (!k || !codes || !scales) return fail(LI_ERR_NULL, "k, codes and scales must be non-NULL");
  if (misaligned(k) || misaligned(codes) || misaligned(scales))
    return fail(LI_ERR_ALIGN, "device pointers must be 16-byte aligned");
  return launched(li::launch_pool_keys((const uint16_t*)k, B, L, pool, codes, scales, stream), "li_pool_keys");
}

size_t li_pooled_indexer_topk_workspace_bytes(int B, int T, int Sp, int H, int topk) {
  if (B < 1 || T < 1 || Sp < 1 || H < 1 || topk < 1) return 0;
  return li::pooled_topk_ws_bytes(B, T, Sp, H, topk);
}

li_status li_pooled_indexer_topk(const void* q, li_dtype q_type, const float* w, const uint8_t* codes,
                                 const float* scales, const int32_t* nv_tokens, int B, int T, int Sp, int H, int d,
                                 int pool, int topk, int32_t* idx_tokens, float* val_blocks, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  if (q_type != LI_BF16) return fail(LI_ERR_DTYPE, "q_type must be LI_BF16");
  li_status s = check_score_args(q, q_type, w, codes, LI_FP8_E4M3, scales, nv_tokens, B, T, Sp, H, d);
  if (s != LI_OK) return s;
  if (!idx_tokens) return fail(LI_ERR_NULL, "idx_tokens must be non-NULL");
  if (pool != 1 && pool != 2 && pool != 4 && pool != 8) return fail(LI_ERR_SHAPE, "pool must be 1, 2, 4 or 8");
  if (topk < 1 || topk > LI_TOPK_MAX) return fail(LI_ERR_SHAPE, "topk must be in [1, %d]", LI_TOPK_MAX);
  if ((int64_t)Sp * pool >= (1ll << 31)) return fail(LI_ERR_SHAPE, "Sp * pool must fit in int32");
  if (misaligned(idx_tokens) || misaligned(val_blocks) || misaligned(ws))
    return fail(LI_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t need = li::pooled_topk_ws_bytes(B, T, Sp, H, topk);
  if (!ws || ws_bytes < need) return fail(LI_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  return launched(li::launch_pooled_topk((const uint16_t*)q, w, codes, scales, nv_tokens, B, T, Sp, H, pool, topk,
                                         idx_tokens, val_blocks, ws, stream),
                  "li_pooled_indexer_topk");
}

namespace {
li_status check_paged_args(const int32_t* page_table, int page_size, int max_pages, int num_pages, int S) {
  if (!page_table) return fail(LI_ERR_NULL, "page_table must be non-NULL");
  if (page_size != LI_INDEX_PAGE) return fail(LI_ERR_SHAPE, "page_size must be %d", LI_INDEX_PAGE);
  if (num_pages < 1 || (int64_t)num_pages * LI_INDEX_PAGE >= (1ll << 31))
    return fail(LI_ERR_SHAPE, "num_pages must be in [1, 2^31 / %d)", LI_INDEX_PAGE);
  if ((int64_t)max_pages * LI_INDEX_PAGE < S) return fail(LI_ERR_SHAPE, "max_pages * %d must cover S", LI_INDEX_PAGE);
  if (misaligned(page_table)) return fail(LI_ERR_ALIGN, "page_table must be 16-byte aligned");
  return LI_OK;
}
}  // namespace

li_status li_indexer_score_paged(const void* q, li_dtype q_type, const float* w, const uint8_t* k_pool,
                                 const float* k_scale_pool, const int32_t* page_table, int page_size, int max_pages,
                                 int num_pages, const int32_t* nv, int B, int T, int S, int H, int d, float* scores,
                                 hipStream_t stream) {
  if (q_type != LI_BF16) return fail(LI_ERR_DTYPE, "q_type must be LI_BF16");
  li_status s = check_score_args(q, q_type, w, k_pool, LI_FP8_E4M3, k_scale_pool, nv, B, T, S, H, d);
  if (s != LI_OK) return s;
  s = check_paged_args(page_table, page_size, max_pages, num_pages, S);
  if (s != LI_OK) return s;
  if (!scores) return fail(LI_ERR_NULL, "scores must be non-NULL");
  if (misaligned(scores)) return fail(LI_ERR_ALIGN, "scores must be 16-byte aligned");
  return launched(li::launch_score_paged((const uint16_t*)q, w, k_pool, k_scale_pool, page_table, max_pages,
                                         num_pages, nv, B, T, S, H, scores, stream),
                  "li_indexer_score_paged");
}

size_t li_indexer_topk_paged_workspace_bytes(int B, int T, int S, int H, int topk) {
  if (B < 1 || T < 1 || S < 1 || H < 1 || topk < 1) return 0;
  return li::indexer_topk_paged_ws_bytes(B, T, S, H, topk);
}

li_status li_indexer_topk_paged(const void* q, li_dtype q_type, const float* w, const uint8_t* k_pool,
                                const float* k_scale_pool, const int32_t* page_table, int page_size, int max_pages,
                                int num_pages, const int32_t* nv, int B, int T, int S, int H, int d, int topk,
                                int32_t* idx, float* val, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (q_type != LI_BF16) return fail(LI_ERR_DTYPE, "q_type must be LI_BF16");
  li_status s = check_score_args(q, q_type, w, k_pool, LI_FP8_E4M3, k_scale_pool, nv, B, T, S, H, d);
  if (s != LI_OK) return s;
  s = check_paged_args(page_table, page_size, max_pages, num_pages, S);
  if (s != LI_OK) return s;
  if (!idx) return fail(LI_ERR_NULL, "idx must be non-NULL");
  if (topk < 1 || topk > LI_TOPK_MAX) return fail(LI_ERR_SHAPE, "topk must be in [1, %d]", LI_TOPK_MAX);
  if (misaligned(idx) || misaligned(val) || misaligned(ws))
    return fail(LI_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t need = li::indexer_topk_paged_ws_bytes(B, T, S, H, topk);
  if (!ws || ws_bytes < need) return fail(LI_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  return launched(li::launch_indexer_topk_paged((const uint16_t*)q, w, k_pool, k_scale_pool, page_table, max_pages,
                                                num_pages, nv, B, T, S, H, topk, idx, val, ws, stream),
                  "li_indexer_topk_paged");
}

li_status li_sparse_attn_gather_paged(const void* q, const void* kv_pool, const int32_t* slot_table, int max_slots,
                                      int num_slots, const int32_t* idx, int B, int Hq, int S, int k, int dqk, int dv,
                                      float sm_scale, void* out, float* lse, hipStream_t stream) {
  if (!q || !kv_pool || !slot_table || !idx || !out)
    return fail(LI_ERR_NULL, "q, kv_pool, slot_table, idx and out must be non-NULL");
  if (dqk != 576 || dv != 512) return fail(LI_ERR_SHAPE, "dqk must be 576 and dv 512");
  if (Hq < 1 || Hq > 128 || Hq % 32) return fail(LI_ERR_SHAPE, "Hq must be a multiple of 32 in [32, 128]");
  if (B < 1 || S < 1 || k < 1 || k > LI_TOPK_MAX)
    return fail(LI_ERR_SHAPE, "need B, S >= 1 and 1 <= k <= %d", LI_TOPK_MAX);
  if (max_slots < S) return fail(LI_ERR_SHAPE, "max_slots must cover S");
  if (num_slots < 1) return fail(LI_ERR_SHAPE, "num_slots must be >= 1");
  if ((int64_t)B * max_slots >= (1ll << 40)) return fail(LI_ERR_SHAPE, "B*max_slots too large");
  if (misaligned(q) || misaligned(kv_pool) || misaligned(slot_table) || misaligned(idx) || misaligned(out) ||
      misaligned(lse))
    return fail(LI_ERR_ALIGN, "device pointers must be 16-byte aligned");
  return launched(li::launch_attn_paged((const uint16_t*)q, (const uint16_t*)kv_pool, slot_table, max_slots,
                                        num_slots, idx, B, Hq, S, k, sm_scale, (uint16_t*)out, lse, stream),
                  "li_sparse_attn_gather_paged");
}

size_t li_layer_stream_buffer_bytes(int S, size_t kv_row_bytes) {
  if (S < 1) return 0;
  return li::layer_stream_buffer_bytes(S, kv_row_bytes);
}

li_status li_layer_stream_prefill(const void* q, const float* w, const int32_t* nv, const void* host_keys,
                                  const void* host_kv, size_t kv_row_bytes, void* host_new_keys, void* host_new_kv,
                                  int new_rows, void* buf0, void* buf1, size_t buf_bytes, int L, int T, int S, int H,
                                  int d, int topk, int32_t* idx, hipStream_t compute, hipStream_t copy,
                                  hipEvent_t* events) {
  if (!q || !w || !host_keys || !buf0 || !buf1 || !idx || !events)
    return fail(LI_ERR_NULL, "q, w, host_keys, buf0, buf1, idx and events must be non-NULL");
  for (int i = 0; i < 4; ++i)
    if (!events[i]) return fail(LI_ERR_NULL, "events must hold four events");
  if (kv_row_bytes && !host_kv) return fail(LI_ERR_NULL, "host_kv must be non-NULL when kv_row_bytes > 0");
  if (d != LI_INDEX_DIM) return fail(LI_ERR_SHAPE, "d must be %d", LI_INDEX_DIM);
  if (L < 1 || T < 1 || S < 1 || H < 1 || H > 128) return fail(LI_ERR_SHAPE, "need L, T, S >= 1 and H in [1, 128]");
  if ((int64_t)L * T * S >= (1ll << 40)) return fail(LI_ERR_SHAPE, "L*T*S too large");
  if (new_rows < 0 || new_rows > S) return fail(LI_ERR_SHAPE, "new_rows must be in [0, S]");
  if (topk < 1 || topk > LI_TOPK_MAX) return fail(LI_ERR_SHAPE, "topk must be in [1, %d]", LI_TOPK_MAX);
  if (!li::prefill_fused_apply(LI_BF16, LI_BF16, T, H, topk))
    return fail(LI_ERR_SHAPE, "the streamed layers run the fused prefill selection: T >= 16 and topk <= 512");
  if (buf_bytes < li::layer_stream_buffer_bytes(S, kv_row_bytes))
    return fail(LI_ERR_WORKSPACE, "each buffer needs %zu bytes", li::layer_stream_buffer_bytes(S, kv_row_bytes));
  if (misaligned(q) || misaligned(w) || misaligned(nv) || misaligned(buf0) || misaligned(buf1) || misaligned(idx))
    return fail(LI_ERR_ALIGN, "device pointers must be 16-byte aligned");
  uint8_t* const bufs[2] = {(uint8_t*)buf0, (uint8_t*)buf1};
  return launched(li::launch_layer_stream((const uint16_t*)q, w, nv, (const uint8_t*)host_keys,
                                          (const uint8_t*)host_kv, kv_row_bytes, (uint8_t*)host_new_keys,
                                          (uint8_t*)host_new_kv, new_rows, bufs, L, T, S, H, topk, idx, compute, copy,
                                          events),
                  "li_layer_stream_prefill");
}

size_t li_compact_workspace_bytes(int B, int S, int H, int m, int k) {
  if (B < 1 || S < 1 || H < 1 || m < 1) return 0;
  return li::compact_ws_bytes(B, S, H, m, k);
}

li_status li_compact_search_rerank(const void* q, const float* w, const float* P, const int8_t* ck,
                                   const float* ck_scale, const void* k_full, const int32_t* nv, int B, int S, int H,
                                   int d, int dc, int m, int k, int32_t* shortlist, int32_t* idx, double* val,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!q || !w || !P || !ck || !ck_scale || !k_full || !idx)
    return fail(LI_ERR_NULL, "q, w, P, ck, ck_scale, k_full and idx must be non-NULL");
  if (d != LI_INDEX_DIM) return fail(LI_ERR_SHAPE, "d must be %d", LI_INDEX_DIM);
  if (dc != LI_COMPACT_DIM) return fail(LI_ERR_SHAPE, "dc must be %d", LI_COMPACT_DIM);
  if (H < 1 || H > 128) return fail(LI_ERR_SHAPE, "H must be in [1, 128]");
  if (B < 1 || S < 1) return fail(LI_ERR_SHAPE, "B and S must be >= 1");
  if (k < 1 || m < k || m > LI_TOPK_MAX) return fail(LI_ERR_SHAPE, "need 1 <= k <= m <= %d", LI_TOPK_MAX);
  if ((int64_t)B * S >= (1ll << 40)) return fail(LI_ERR_SHAPE, "B*S too large");
  if (misaligned(q) || misaligned(w) || misaligned(P) || misaligned(ck) || misaligned(ck_scale) ||
      misaligned(k_full) || misaligned(nv) || misaligned(shortlist) || misaligned(idx) || misaligned(val) ||
      misaligned(ws))
    return fail(LI_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t need = li::compact_ws_bytes(B, S, H, m, k);
  if (!ws || ws_bytes < need) return fail(LI_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  return launched(li::launch_compact((const uint16_t*)q, w, P, ck, ck_scale, (const uint16_t*)k_full, nv, B, S, H, m,
                                     k, shortlist, idx, val, ws, stream),
                  "li_compact_search_rerank");
}

size_t li_pq_workspace_bytes(int B, int S, int H, int m, int k) {
  if (B < 1 || S < 1 || H < 1 || m < 1) return 0;
  return li::pq_ws_bytes(B, S, H, m, k);
}

li_status li_pq_search_rerank(const void* q, const float* w, const int8_t* codebook, float sigma,
                              const uint8_t* codes, const void* k_full, const int32_t* nv, int B, int S, int H, int d,
                              int m, int k, int32_t* shortlist, int32_t* idx, double* val, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  if (!q || !w || !codebook || !codes || !k_full || !idx)
    return fail(LI_ERR_NULL, "q, w, codebook, codes, k_full and idx must be non-NULL");
  if (d != LI_INDEX_DIM) return fail(LI_ERR_SHAPE, "d must be %d", LI_INDEX_DIM);
  if (H < 1 || H > 128) return fail(LI_ERR_SHAPE, "H must be in [1, 128]");
  if (B < 1 || S < 1) return fail(LI_ERR_SHAPE, "B and S must be >= 1");
  if (k < 1 || m < k || m > LI_TOPK_MAX) return fail(LI_ERR_SHAPE, "need 1 <= k <= m <= %d", LI_TOPK_MAX);
  if ((int64_t)B * S >= (1ll << 40)) return fail(LI_ERR_SHAPE, "B*S too large");
  if (!(sigma > 0.0f) || !(sigma < 3.0e38f)) return fail(LI_ERR_SHAPE, "sigma must be positive and finite");
  if (misaligned(q) || misaligned(w) || misaligned(codebook) || misaligned(codes) || misaligned(k_full) ||
      misaligned(nv) || misaligned(shortlist) || misaligned(idx) || misaligned(val) || misaligned(ws))
    return fail(LI_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t need = li::pq_ws_bytes(B, S, H, m, k);
  if (!ws || ws_bytes < need) return fail(LI_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  return launched(li::launch_pq((const uint16_t*)q, w, codebook, sigma, codes, (const uint16_t*)k_full, nv, B, S, H,
                                m, k, shortlist, idx, val, ws, stream),
                  "li_pq_search_rerank");
}

size_t li_sparse_attn_workspace_bytes(int B, int Hq, int k, int dv) { return li::attn_ws_bytes(B, Hq, k, dv); }

li_status li_sparse_attn_gather(const void* q, const void* kv, const int32_t* idx, int B, int Hq, int S, int k,
                                int dqk, int dv, float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  if (!q || !kv || !idx || !out) return fail(LI_ERR_NULL, "q, kv, idx and out must be non-NULL");
  if (dqk != 576 || dv != 512) return fail(LI_ERR_SHAPE, "dqk must be 576 and dv 512");
  if (Hq < 1 || Hq > 128 || Hq % 32) return fail(LI_ERR_SHAPE, "Hq must be a multiple of 32 in [32, 128]");
  if (B < 1 || S < 1 || k < 1 || k > LI_TOPK_MAX) return fail(LI_ERR_SHAPE, "need B, S >= 1 and 1 <= k <= %d",
                                                              LI_TOPK_MAX);
  if (misaligned(q) || misaligned(kv) || misaligned(idx) || misaligned(out) || misaligned(lse) || misaligned(ws))
    return fail(LI_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t need = li::attn_ws_bytes(B, Hq, k, dv);
  if (need && (!ws || ws_bytes < need)) return fail(LI_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  return launched(li::launch_attn((const uint16_t*)q, (const uint16_t*)kv, idx, B, Hq, S, k, sm_scale,
                                  (uint16_t*)out, lse, ws, stream),
                  "li_sparse_attn_gather");
}

}  // extern "C"
