/*
 * mla_peaks.h -- attainable-peak microbenchmarks for MI355X (gfx950).
 *
 * The decode kernel is priced against the chip's published peaks (8 TB/s
 * HBM, 2.5 PFLOP/s dense bf16).  These kernels measure what the same box
 * attains, so that a second roofline column can be stated against measured
 * peaks: a streaming HBM read, a gather of random 1152-byte cache rows moved
 * exactly the way the decode moves them (one row = the 512 latent + 64 rotary
 * bf16 values of a cached position, the row the "Query-key similarity" page's
 * scores and the "Apply value weights" page's mix read), and dense
 * bf16 MFMA throughput.  They compute nothing of the method.
 *
 * Conventions: device pointers owned by the caller; `stream` is a hipStream_t
 * (NULL = default stream); each call enqueues ONE launch and returns without
 * synchronising.  Return value: 0 = launched, 1 = argument rejected (nothing
 * launched), 2 = the launch failed (HIP error).
 */
#ifndef MLA_PEAKS_H
#define MLA_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes at `src` (16-byte aligned, bytes a positive multiple of
 * 16) with 16-byte vector loads, grid-stride over `num_wg` workgroups of 256
 * threads.  `sink` (one uint32, device) is written only if an impossible
 * checksum comes up; it keeps the loads live. */
int mlap_stream_read(const void* src, size_t bytes, int32_t num_wg, uint32_t* sink, void* stream);

/* Gather rows of 1152 bytes: workgroup w (of num_wg, 256 threads) moves rows
 * rows[w * rows_per_wg + i], i < rows_per_wg, from `cache` (row r at byte
 * 1152 r) into LDS by LDS-DMA, 32 rows per block, 8 lanes per 128-byte line,
 * a ring of four 36 KB buffers with up to three blocks in flight and a
 * barrier per block.  rows_per_wg is a multiple of 32 in [32, 1024];
 * cache_bytes <= UINT32_MAX (rows are addressed with 32-bit byte offsets; a
 * row past cache_bytes reads zeros, never memory).  rows: device int32
 * [num_wg * rows_per_wg]. */
int mlap_row_gather(const void* cache, size_t cache_bytes, const int32_t* rows, int32_t num_wg,
                    int32_t rows_per_wg, uint32_t* sink, void* stream);

/* Dense bf16 matrix-core throughput: each of the 4 waves of each of num_wg
 * workgroups issues `iters` rounds of 16 independent 32x32x16 bf16 MFMAs
 * (32768 FLOP each).  sink: device float[num_wg * 256]. */
int mlap_mfma_bf16(int32_t num_wg, int32_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PEAKS_H */
