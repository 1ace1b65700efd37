// Internal host-side launchers shared by the C ABI (capi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define LI_TOPK_MAX_DEV 2048

namespace li {

enum { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_I8 = 3 };

// scores [B*T, S] of q [B,T,H,128] against k [B,S,128]
hipError_t launch_score(const void* q, int q_type, const float* w, const void* k, int k_type, const float* ks,
                        const int32_t* nv, int B, int T, int S, int H, float* scores, hipStream_t st);

// per-row top-k of fp32 scores [R, S]; ws holds topk_ws_bytes(R, S, k) bytes
size_t topk_ws_bytes(int R, int S, int k);

// Size of the per-device static scratch of li_topk_select_noalloc, and its device
// address on the current device (looked up on first use, then kept).
constexpr size_t NOALLOC_SCRATCH_BYTES = (32u << 20) + (512u << 10);
hipError_t noalloc_scratch(void** ptr);
// whether rows of this shape take the multi-workgroup top-k (few, long rows)
bool topk_use_mb(int R, int S);
hipError_t launch_topk_f32(const float* scores, const int32_t* nv, int R, int S, int k, int32_t* idx, float* val,
                           void* ws, hipStream_t st);

// per-row top-k of fp64 scores (row r starts at r * row_stride); ids [R, row_stride]
// gives each entry's id (NULL = its position); ties go to the smaller id
hipError_t launch_topk_f64(const double* scores, int64_t row_stride, const int32_t* nv, const int32_t* ids, int R,
                           int S, int k, int32_t* idx, double* val, hipStream_t st);

// per-row top-k of dense fp64 scores [R, S] (ids = positions); few long rows take
// the many-workgroups-per-row path, whose buffers ws holds
size_t topk_f64_rows_ws_bytes(int R, int S);
hipError_t launch_topk_f64_rows(const double* scores, const int32_t* nv, int R, int S, int k, int32_t* idx,
                                double* val, void* ws, hipStream_t st);
// Whether launch_topk_f64_rows takes rows of S scores through per-region lists
// (regions of *region scores, each listed above a threshold of its own): a
// scoring kernel whose workgroups cover exactly those regions may list them itself
// (list_above_local_threshold into the buffers topk_mb_layout_f64 names in the
// same workspace) and then call launch_topk_finalize_f64.
bool topk_f64_rows_listed(int R, int S, int* region);
void topk_mb_layout_f64(void* ws, int R, int S, uint32_t** thresholds, uint32_t** bcnt, double** cval,
                        int32_t** cid);
hipError_t launch_topk_finalize_f64(const double* scores, const int32_t* nv, int R, int S, int k, const uint32_t* bcnt,
                                    const double* cval, const int32_t* cid, int32_t* idx, double* val,
                                    const uint32_t* tau_used, hipStream_t st);

// two-stage compact search (workspace layout in compact.hip)
size_t compact_ws_bytes(int B, int S, int H, int m, int k);
hipError_t launch_compact(const uint16_t* q, const float* w, const float* P, const int8_t* ck, const float* cks,
                          const uint16_t* kf, const int32_t* nv, int B, int S, int H, int m, int k,
                          int32_t* shortlist, int32_t* idx, double* val, void* ws, hipStream_t st);

// two-stage search over product-quantised keys (compact.hip)
size_t pq_ws_bytes(int B, int S, int H, int m, int k);
hipError_t launch_pq(const uint16_t* q, const float* w, const int8_t* cb, float sigma, const uint8_t* codes,
                     const uint16_t* kf, const int32_t* nv, int B, int S, int H, int m, int k, int32_t* shortlist,
                     int32_t* idx, double* val, void* ws, hipStream_t st);

// sparse attention over selected rows (workspace layout in attn.hip)
size_t attn_ws_bytes(int B, int Hq, int k, int dv);
hipError_t launch_attn(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int B, int Hq, int S, int k,
                       float sm_scale, uint16_t* out, float* lse, void* ws, hipStream_t st);

// scores of many query rows (prefill shapes: bf16 queries, bf16 or fp8 keys,
// T >= 16, H <= 128) by the MFMA-tiled kernel that also serves the fused selection
bool prefill_scores_apply(int q_type, int k_type, int T, int H);
hipError_t launch_prefill_scores(const uint16_t* q, const float* w, const void* k, int k_type, const float* ks,
                                 const int32_t* nv, int B, int T, int S, int H, float* scores, hipStream_t st);

// Few long rows, fp8 keys, 33-64 heads: the held-scores kernel lists each
// workgroup's entries above a threshold of its own (no waiting), the finalize
// selects exactly or over the whole row.
bool held_select_apply(int q_type, int k_type, int R, int S, int H, int topk);
hipError_t launch_score_held_select(const void* q, const float* w, const void* k, const float* ks, const int32_t* nv,
                                    int B, int T, int S, int H, int topk, float* scores, uint32_t* bcnt, float* cval,
                                    int32_t* cid, uint32_t* tau_used, int* P, int* chunk, hipStream_t st,
                                    const int32_t* page_table = nullptr, int max_pages = 0, int num_pages = 0);

// Paged fp8 keys: k_pool [num_pages, 64, 128] codes, ks_pool [num_pages, 64]
// scales, page_table [B, max_pages] (pool page of keys 64 p .. 64 p + 63 of b).
hipError_t launch_score_paged(const uint16_t* q, const float* w, const uint8_t* k_pool, const float* ks_pool,
                              const int32_t* page_table, int max_pages, int num_pages, const int32_t* nv, int B,
                              int T, int S, int H, float* scores, hipStream_t st);
size_t indexer_topk_paged_ws_bytes(int B, int T, int S, int H, int topk);
hipError_t launch_indexer_topk_paged(const uint16_t* q, const float* w, const uint8_t* k_pool, const float* ks_pool,
                                     const int32_t* page_table, int max_pages, int num_pages, const int32_t* nv,
                                     int B, int T, int S, int H, int topk, int32_t* idx, float* val, void* ws,
                                     hipStream_t st);
// Paged latent rows (page size 1): kv_pool [num_slots, 576], slot_table [B, max_slots]
hipError_t launch_attn_paged(const uint16_t* q, const uint16_t* kv_pool, const int32_t* slot_table, int max_slots,
                             int num_slots, const int32_t* idx, int B, int Hq, int S, int k, float sm_scale,
                             uint16_t* out, float* lse, hipStream_t st);
void topk_mb_layout(void* ws, int R, int S, uint32_t** thresholds, uint32_t** bcnt, float** cval, int32_t** cid);
// The exact selection over per-region candidate lists (regions of `chunk` keys, P
// per row, counts bcnt [R, P]); tau_used: the thresholds each region listed above
// ([R, 256]: P thresholds, then with P <= 128 the regions' largest keys at 128),
// or NULL when every region used one threshold that at least k entries cleared.
hipError_t launch_topk_finalize_f32(const float* scores, const int32_t* nv, int R, int S, int k, int P, int chunk,
                                    const uint32_t* bcnt, const float* cval, const int32_t* cid, int32_t* idx,
                                    float* val, const uint32_t* tau_used, hipStream_t st);

// fused scoring + selection for many query rows (prefill); falls back to
// score-then-select where the fused kernel does not apply
size_t indexer_topk_ws_bytes(int q_type, int k_type, int B, int T, int S, int H, int topk);
hipError_t launch_indexer_topk(const void* q, int q_type, const float* w, const void* k, int k_type, const float* ks,
                               const int32_t* nv, int B, int T, int S, int H, int topk, int32_t* idx, float* val,
                               void* ws, hipStream_t st);

// pooled indexer keys (pooled.hip): pool bf16 token keys [B, L, 128] into fp8
// codes [B, L / pool, 128] + scales; score the pooled keys, select the top blocks
// and expand them to token indices
hipError_t launch_pool_keys(const uint16_t* k, int B, int L, int pool, uint8_t* codes, float* scales,
                            hipStream_t st);
size_t pooled_topk_ws_bytes(int B, int T, int Sp, int H, int topk);
hipError_t launch_pooled_topk(const uint16_t* q, const float* w, const uint8_t* codes, const float* scales,
                              const int32_t* nv_tokens, int B, int T, int Sp, int H, int pool, int topk,
                              int32_t* idx_tokens, float* val_blocks, void* ws, hipStream_t st);

// layer-streamed prefill (stream.hip)
size_t layer_stream_buffer_bytes(int S, size_t kv_row_bytes);
hipError_t launch_layer_stream(const uint16_t* q, const float* w, const int32_t* nv, const uint8_t* host_keys,
                               const uint8_t* host_kv, size_t kv_row_bytes, uint8_t* host_new_keys,
                               uint8_t* host_new_kv, int new_rows, uint8_t* const buf[2], int L, int T, int S, int H,
                               int topk, int32_t* idx, hipStream_t compute, hipStream_t copy, hipEvent_t const ev[4]);
bool prefill_fused_apply(int q_type, int k_type, int T, int H, int topk);

}  // namespace li
