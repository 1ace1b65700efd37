// Layer-streamed prefill: a chunk of new queries moves through the layers one at a
// time, and only two layers' history is on the GPU at any moment (LeanSparse
// podcast transcript, cues 05:36-06:40: the indexer keys and compressed KV of every
// layer sit in host memory; one GPU buffer serves the current layer while the other
// loads the next layer's history; the full compressed KV is loaded because the
// picks are not known in advance; new state goes back to the host through a
// staging path).  The transfer hides behind the layer's compute when loading takes
// less time than scoring (cues 06:44-07:09).
//
// Host side only: copies on the caller's copy stream, the fused prefill scoring +
// selection (prefill_select_kernel) on the caller's compute stream, ordered by four
// caller-owned events:
//
//   copy:     H2D(layer 0 -> buf 0); record loaded[0]
//   layer l:  compute waits loaded[l % 2]; select(layer l, buf l % 2); record done[l % 2]
//             copy waits done[(l + 1) % 2] (layer l - 1 has finished with that
//             buffer), D2H of layer l - 1's new rows from it, H2D(layer l + 1 ->
//             it); record loaded[(l + 1) % 2]
//   end:      copy waits done of layers L - 2 and L - 1; D2H of their new rows
//
// Nothing is allocated and nothing synchronises the host.
#include "launch.h"

namespace li {

size_t layer_stream_buffer_bytes(int S, size_t kv_row_bytes) {
  const size_t keys = (size_t)S * 128 * 2;
  return ((keys + 255) & ~(size_t)255) + (size_t)S * kv_row_bytes;
}

hipError_t launch_layer_stream(const uint16_t* q, const float* w, const int32_t* nv, const uint8_t* host_keys,
                               const uint8_t* host_kv, size_t kv_row_bytes, uint8_t* host_new_keys,
                               uint8_t* host_new_kv, int new_rows, uint8_t* const buf[2], int L, int T, int S, int H,
                               int topk, int32_t* idx, hipStream_t compute, hipStream_t copy,
                               hipEvent_t const ev[4]) {
  const size_t key_bytes = (size_t)S * 128 * 2;
  const size_t kv_bytes = (size_t)S * kv_row_bytes;
  const size_t kv_off = (key_bytes + 255) & ~(size_t)255;
  hipEvent_t loaded[2] = {ev[0], ev[1]}, done[2] = {ev[2], ev[3]};
  auto load = [&](int l, int slot) -> hipError_t {
    hipError_t e = hipMemcpyAsync(buf[slot], host_keys + (size_t)l * key_bytes, key_bytes, hipMemcpyHostToDevice, copy);
    if (e == hipSuccess && kv_bytes)
      e = hipMemcpyAsync(buf[slot] + kv_off, host_kv + (size_t)l * kv_bytes, kv_bytes, hipMemcpyHostToDevice, copy);
    if (e == hipSuccess) e = hipEventRecord(loaded[slot], copy);
    return e;
  };
  // the chunk's new rows (the last new_rows keys and kv rows) of layer l, back to
  // the host from the buffer that served it
  auto store = [&](int l, int slot) -> hipError_t {
    if (new_rows <= 0) return hipSuccess;
    const size_t r0 = (size_t)(S - new_rows);
    hipError_t e = hipSuccess;
    if (host_new_keys)
      e = hipMemcpyAsync(host_new_keys + (size_t)l * new_rows * 256, buf[slot] + r0 * 256, (size_t)new_rows * 256,
                         hipMemcpyDeviceToHost, copy);
    if (e == hipSuccess && host_new_kv && kv_row_bytes)
      e = hipMemcpyAsync(host_new_kv + (size_t)l * new_rows * kv_row_bytes, buf[slot] + kv_off + r0 * kv_row_bytes,
                         (size_t)new_rows * kv_row_bytes, hipMemcpyDeviceToHost, copy);
    return e;
  };
  hipError_t e = load(0, 0);
  if (e != hipSuccess) return e;
  for (int l = 0; l < L; ++l) {
    const int cur = l & 1, nxt = cur ^ 1;
    e = hipStreamWaitEvent(compute, loaded[cur], 0);
    if (e != hipSuccess) return e;
    e = launch_indexer_topk(q + (size_t)l * T * H * 128, DT_BF16, w + (size_t)l * T * H, buf[cur], DT_BF16, nullptr,
                            nv, 1, T, S, H, topk, idx + (size_t)l * T * topk, nullptr, nullptr, compute);
    if (e != hipSuccess) return e;
    e = hipEventRecord(done[cur], compute);
    if (e != hipSuccess) return e;
    if (l + 1 < L) {
      if (l >= 1) {
        // buffer nxt served layer l - 1: wait for it, write its new rows back
        e = hipStreamWaitEvent(copy, done[nxt], 0);
        if (e == hipSuccess) e = store(l - 1, nxt);
        if (e != hipSuccess) return e;
      }
      e = load(l + 1, nxt);
      if (e != hipSuccess) return e;
    }
  }
  // the loop wrote back layers 0 .. L - 3; the last two buffers still hold layers
  // L - 2 and L - 1
  if (L >= 2) {
    e = hipStreamWaitEvent(copy, done[(L - 2) & 1], 0);
    if (e == hipSuccess) e = store(L - 2, (L - 2) & 1);
    if (e != hipSuccess) return e;
  }
  e = hipStreamWaitEvent(copy, done[(L - 1) & 1], 0);
  if (e == hipSuccess) e = store(L - 1, (L - 1) & 1);
  return e;
}

}  // namespace li
