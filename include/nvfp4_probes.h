/*
 * nvfp4_probes.h -- C ABI of libnvfp4_probes, the measurement aids that sit
 * beside the NVFP4 decode projection (libnvfp4, nvfp4.h) without being part
 * of it.  The benchmark times them to put the GEMV's numbers in context; no
 * entry point of nvfp4.h calls them and the GEMV library does not link them.
 *
 * The pages judge their projection kernels against a read ceiling they
 * measured with STREAM on the same machine (spark_model::layers page, doc
 * comment of w4a16_k64_min_k), and split one launch into memory-pipe time and
 * exposed dequant time (doc comment of K64_N64_MAX_WIDE_CTAS).  These probes
 * give the MI355X counterparts: a plain read of the same bytes
 * (nvfp4_probe_read_stream), the cost of a launch that does nothing
 * (nvfp4_probe_empty), the arithmetic rate of the per-block work on
 * register data (nvfp4_probe_block_rate) and the time of the activation
 * staging alone (nvfp4_probe_x_stage).
 *
 * Conventions are those of nvfp4.h: DEVICE pointers, asynchronous on `stream`
 * (a hipStream_t, NULL = default stream), validation on the host before any
 * HIP call, nvfp4_status return codes (nvfp4_strerror of libnvfp4 names
 * them), no allocation, no synchronisation.
 */
#ifndef NVFP4_PROBES_H
#define NVFP4_PROBES_H

#include <stddef.h>
#include <stdint.h>

#include "nvfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Paths of nvfp4_probe_block_rate. */
#define NVFP4_RATE_MFMA 0
#define NVFP4_RATE_VALU 1

/* The issue rate of the arithmetic for one 16-element block of a 16-row group
 * times n tokens, on register data (no memory traffic), for the two ways to
 * do it on gfx950.  NVFP4_RATE_MFMA is nvfp4_gemv's sequence (two fp4->bf16
 * converts, one 16x16x16 bf16 MFMA with the tokens as M, ceil(n/4) scale
 * FMAs); NVFP4_RATE_VALU the best VALU form found (the same converts, then
 * per token an LDS read of its 4 activations, two v_dot2_f32_bf16 and one
 * scale FMA).  This is the measurement behind choosing MFMA for n = 1..16 (the
 * pages' kernels are CUDA-core / tensor-core designs for another GPU).  Runs
 * 256 workgroups of 8 waves (two per SIMD), each wave `blocks` blocks
 * (rounded down to a multiple of 8, independent codes per block as loaded
 * tiles have); the launch time divided by that count is the time of one
 * block on every SIMD of the chip, two waves at once.  n in {1, 2, 4, 8, 12,
 * 16}.  sink: DEVICE, at least 256*512*4 bytes, 4-byte aligned, receives
 * meaningless values.  Errors: NULL, RANGE (path, n, blocks < 8, sink_bytes),
 * ALIGN, LAUNCH. */
int nvfp4_probe_block_rate(int path, int n, int blocks, float *sink, size_t sink_bytes,
                           void *stream);

/* Reads `bytes` bytes of `buf` (DEVICE, 16-byte aligned, bytes a positive
 * multiple of 16) once with the streaming pattern that reads fastest on
 * MI355X (1024-thread workgroups over contiguous chunks of about 40 KiB, at
 * least 256 workgroups, four 16-byte non-temporal loads in flight per lane)
 * and writes to *sink (DEVICE, 4
 * bytes, 4-byte aligned) only if a checksum of the data equals a value the
 * benchmark's data never produces, so that no load is dead and nothing is
 * written in practice.  Timing it over the bytes of one weight gives the
 * achievable read ceiling of that size; over a buffer of 1 GiB or more, the
 * streaming rate without the per-launch ramp.  Errors: NULL, RANGE (bytes,
 * or more than 2^31 - 1 workgroups), ALIGN, DEVICE, LAUNCH. */
int nvfp4_probe_read_stream(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* Modes of nvfp4_probe_x_stage. */
#define NVFP4_XSTAGE_LOADS 0   /* the activation loads alone                       */
#define NVFP4_XSTAGE_FULL 1    /* loads, per-wave LDS tile, read-back into MFMA layout */

/* The activation staging nvfp4_gemv does at the start of a launch, alone, as
 * one more part of the launch split (spark_model::layers page, doc comment of
 * K64_N64_MAX_WIDE_CTAS): `workgroups` workgroups of 8 waves (1 .. 65536),
 * wave w taking the 128-column tiles w, w + 8, w + 16, ... of K for the n
 * token rows of X (bf16 [n][K], DEVICE, 16-byte aligned) with whole-line
 * 16-byte loads, `reps` times per launch (1 .. 1024).  NVFP4_XSTAGE_LOADS
 * stops after the loads; NVFP4_XSTAGE_FULL also writes each tile to the
 * wave's LDS tile and reads it back in the MFMA operand layout, as the GEMV
 * does (only the groups of four token rows that hold a token are written,
 * and only the lanes that carry a token read back).  Every workgroup reads the same X, so after the first repetition it
 * comes from L2: the launch time over reps is one staging on every compute
 * unit at once, bounded by what each XCD's L2 delivers.  n in 1 .. 16, K a
 * multiple of 128 from 128 to 8192 (one pass of the GEMV).  *sink (DEVICE, 4
 * bytes, 4-byte aligned) is written only if a checksum of the data equals a
 * value the benchmark's data never produces.  Errors: NULL, RANGE, ALIGN,
 * LAUNCH. */
int nvfp4_probe_x_stage(const uint16_t *X, int n, int K, int workgroups, int reps, int mode,
                        uint32_t *sink, void *stream);

/* Launches `workgroups` workgroups (1 .. 65536) of 512 threads that do
 * nothing: the fixed cost of one launch of the GEMV's shape (its dispatch,
 * wave launch and retirement), to set beside the GEMV's time.  Errors: RANGE,
 * LAUNCH. */
int nvfp4_probe_empty(int workgroups, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_PROBES_H */
