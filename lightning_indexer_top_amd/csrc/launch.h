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

// two-stage compact search (workspace layout in compact.hip)
size_t compact_ws_bytes(int B, int S, int H, int m, int k);
hipError_t launch_compact(const uint16_t* q, const float* w, const float* P, const int8_t* ck, const float* cks,
                          const uint16_t* kf, const int32_t* nv, int B, int S, int H, int m, int k,
                          int32_t* shortlist, int32_t* idx, double* val, void* ws, hipStream_t st);

// sparse attention over selected rows (workspace layout in attn.hip)
size_t attn_ws_bytes(int B, int Hq, int k, int dv);
hipError_t launch_attn(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int B, int Hq, int S, int k,
                       float sm_scale, uint16_t* out, float* lse, void* ws, hipStream_t st);

// scores of many query rows (prefill shapes: bf16 queries and keys, T >= 16,
// H <= 128) by the MFMA-tiled kernel that also serves the fused selection
bool prefill_scores_apply(int q_type, int k_type, int T, int H);
hipError_t launch_prefill_scores(const uint16_t* q, const float* w, const uint16_t* k, const int32_t* nv, int B,
                                 int T, int S, int H, float* scores, hipStream_t st);

// Few long rows (decode): the scoring kernel also lists each row's candidates.
// Its workgroups take the row's threshold from the first 32-key tile of every wave
// (published with one flag per wave, counters[r * 1024 + wave]) and list their own
// range's entries at or above it into the multi-workgroup top-k's regions (bcnt /
// cval / cid, P regions of chunk keys per row); the first to compute a row's
// threshold publishes it (taupub[16 r], one word per 128-byte line) for the later ones, and
// every region records the threshold it used (tau_used[r * 256 + p]); the finalize
// then selects exactly (if all of a row's regions used one threshold) and clears
// the row's flags (reset).
// select_score_apply tells whether the shape takes this path.
bool select_score_apply(int q_type, int k_type, int R, int S, int H, int topk);
hipError_t launch_score_select(const void* q, int k_type, const float* w, const void* k, const float* ks,
                               const int32_t* nv, int B, int T, int S, int H, int topk, float* scores,
                               uint32_t* counters, uint32_t* bcnt, float* cval, int32_t* cid, uint64_t* taupub,
                               uint32_t* tau_used, int* P, int* chunk, hipStream_t st);
void topk_mb_layout(void* ws, int R, int S, uint32_t** counters, uint32_t** bcnt, float** cval, int32_t** cid);
hipError_t launch_topk_finalize_f32(const float* scores, const int32_t* nv, int R, int S, int k, int P, int chunk,
                                    const uint32_t* bcnt, const float* cval, const int32_t* cid, int32_t* idx,
                                    float* val, uint32_t* reset, const uint32_t* tau_used, hipStream_t st);

// fused scoring + selection for many query rows (prefill); falls back to
// score-then-select where the fused kernel does not apply
size_t indexer_topk_ws_bytes(int B, int T, int S, int H, int topk);
hipError_t launch_indexer_topk(const void* q, int q_type, const float* w, const void* k, int k_type, const float* ks,
                               const int32_t* nv, int B, int T, int S, int H, int topk, int32_t* idx, float* val,
                               void* ws, hipStream_t st);

}  // namespace li
