// Scoring followed by per-row selection.
#include "common.h"
#include "launch.h"

namespace li {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t indexer_topk_ws_bytes(int B, int T, int S, int H, int topk) {
  (void)H;
  return align256((size_t)B * T * S * sizeof(float)) + topk_ws_bytes(B * T, S, topk);
}

hipError_t launch_indexer_topk(const void* q, int q_type, const float* w, const void* k, int k_type, const float* ks,
                               const int32_t* nv, int B, int T, int S, int H, int topk, int32_t* idx, float* val,
                               void* ws, hipStream_t st) {
  float* scores = (float*)ws;
  hipError_t e = launch_score(q, q_type, w, k, k_type, ks, nv, B, T, S, H, scores, st);
  if (e != hipSuccess) return e;
  return launch_topk_f32(scores, nv, B * T, S, topk, idx, val,
                         (uint8_t*)ws + align256((size_t)B * T * S * sizeof(float)), st);
}

}  // namespace li
