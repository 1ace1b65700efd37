/*
 * li_probe.h -- roofline probes of liblightning_indexer_probe.so (gfx950).
 *
 * These are measurement tools, not part of the indexer path: they give the
 * measured ceilings (HBM read rate, bf16 matrix-core rate) that the benchmark
 * reports beside the datasheet peaks.  All pointers are device pointers owned by
 * the caller; work is enqueued on `stream` and nothing synchronises.  Each call
 * returns 0 on success, 1 for a bad argument (nothing launched) and 2 when the
 * launch failed.
 */
#ifndef LIGHTNING_INDEXER_LI_PROBE_H
#define LIGHTNING_INDEXER_LI_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups (of 256 threads) of the read probe at `blocks_per_cu` per compute
 * unit; `sink` holds that many uint32 words. */
int li_probe_read_blocks(int blocks_per_cu);

/* Reads all `bytes` of `buf` once with 16-byte loads, no stores but one word per
 * workgroup into sink.  mode 0: grid-stride loads into registers, 8 in flight per
 * lane; 1: a contiguous range per wave, 8 consecutive 1 KB wave loads in flight;
 * 2: a contiguous range per wave by DMA into LDS, 12 in flight; 3: as 2 with the
 * non-temporal cache policy; 4: a contiguous range per workgroup whose four waves
 * take 4 KB tiles in turn, 3 tiles in flight per wave, DMA into LDS, non-temporal
 * (bytes a multiple of 16 KB).  buf 16-byte aligned, bytes a multiple of 16,
 * 1 <= blocks_per_cu <= 16; returns 0, or 1 for invalid arguments. */
int li_probe_read(const void *buf, size_t bytes, uint32_t *sink, int mode, int blocks_per_cu, hipStream_t stream);

/* Workgroups of the matrix-core probe (4 waves each); `sink` holds 4 floats per
 * workgroup. */
int li_probe_mfma_blocks(void);

/* Floating-point operations one li_probe_mfma_bf16 launch performs for `iters`. */
double li_probe_mfma_flop(int iters);

/* `iters` x 16 v_mfma_f32_32x32x16_bf16 per wave from register operands: constant
 * operand bits (random = 0) or pseudo-random normal-range bf16 values (random = 1). */
int li_probe_mfma_bf16(int iters, int random, float *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_INDEXER_LI_PROBE_H */
