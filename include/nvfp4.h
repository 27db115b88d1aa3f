/*
 * nvfp4.h -- C ABI of libnvfp4, the MI355X (gfx950) NVFP4 weight-only
 * projection GEMV of batched LLM decode.
 *
 * The operation (Atlas PR #266, PR description "What it does"): for n
 * concurrent decode tokens, one projection computes
 *
 *     Y[t][r] = gscale * sum_k X[t][k] * e2m1(code[r][k]) * e4m3(scale[r][k/16])
 *
 * for t < n, r < N.  The page's point is that a tile of tokens shares one read
 * of the weight matrix instead of one read per token; its greedy tiling into
 * 3-token tiles is available as an explicit schedule (nvfp4_gemv_sched),
 * while the default launch reads the weight once for all n <= 16 tokens.
 *
 * Number formats: the pages name NVFP4 without defining its bits.  Codes are
 * OCP FP4 E2M1 (sign bit 3, magnitudes {0,.5,1,1.5,2,3,4,6}), block scales OCP
 * FP8 E4M3FN (bias 7, max 448, 0x7F/0xFF NaN), one scale per 16 consecutive k
 * of a row, and one fp32 tensor multiplier gscale.  X and Y are bf16 bit
 * patterns, accumulation is fp32, Y is rounded to nearest even.
 *
 * Conventions for every entry point:
 *   - all array pointers are DEVICE pointers of the current device (the
 *     one hipSetDevice selected), where every launch runs; calls are
 *     asynchronous on `stream` (a hipStream_t of that device; NULL is its
 *     default stream);
 *   - the caller allocates and owns every buffer; the GEMV entry points
 *     allocate nothing, cache no pointer and never synchronise;
 *   - arguments are validated on the host before any HIP call; a failed
 *     validation returns a status and launches nothing;
 *   - no exception crosses the ABI; nvfp4_strerror names every status.
 *
 * Layouts:
 *   canonical codes  [N][K/2] u8: element (r,k) in byte r*K/2 + k/2, low
 *                    nibble for even k, high nibble for odd k;
 *   canonical scales [N][K/16] u8: one E4M3 byte per 16 consecutive k;
 *   packed (device)  layout written by nvfp4_pack and read by the GEMV
 *                    entry points: rows padded to a multiple of 16 and K to
 *                    a multiple of 128 with zero codes, stored as 16-row x
 *                    128-column tiles whose 1 KiB of codes is one 16-byte
 *                    load per lane of a 64-lane wavefront; its byte sizes
 *                    are nvfp4_packed_codes_bytes / nvfp4_packed_scales_bytes;
 *   X [n][K] bf16 row-major (token-major), Y [n][N] bf16 row-major.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = 1,      /* a required pointer is NULL                      */
    NVFP4_ERR_RANGE = 2,     /* n outside [1,16], N or K not positive, bad rows */
    NVFP4_ERR_ALIGN = 3,     /* a pointer is not aligned as documented          */
    NVFP4_ERR_SHAPE = 4,     /* K not a multiple of 16, or a size limit         */
    NVFP4_ERR_SCHEDULE = 5,  /* an explicit tile schedule is invalid            */
    NVFP4_ERR_LAUNCH = 6,    /* the HIP runtime rejected a launch               */
    NVFP4_ERR_DEVICE = 7,    /* the current device is not a gfx950 GPU          */
    NVFP4_ERR_WORKSPACE = 8, /* a required workspace is NULL or too small       */
    NVFP4_ERR_SCRATCH = 9    /* beyond the fixed scratch of nvfp4_gemv_ws_static */
} nvfp4_status;

/* Largest number of tokens one launch covers (the decode batch of the pages:
 * up to 16 concurrent sequences, Atlas PR #266 A/B table, C = 1..16). */
#define NVFP4_MAX_TOKENS 16

/* Byte sizes of the packed device layout for an N x K weight: the weight in
 * the order the GEMV kernels load it, built once at load time.  The pages
 * trace their fast path to exactly this: the wide kernel ran fast only on a
 * weight copy laid out for it, and the fix they propose is to emit that copy
 * when the weight is (re)quantised (Atlas PR #266 automated review page,
 * "Tiebreaker" comment and the "Complete picture" follow-up).  Rows are padded
 * to 16 and K to 128, so the sizes are ceil(N/16)*16 * ceil(K/128)*128 / 2
 * bytes of codes and a sixteenth of that count of scale bytes, computed in
 * 64-bit arithmetic.  0 if N <= 0 or K <= 0 or K % 16 != 0. */
size_t nvfp4_packed_codes_bytes(int N, int K);
size_t nvfp4_packed_scales_bytes(int N, int K);

/* Quantise an fp32 weight W [N][K] (device, row-major, finite values) to the
 * canonical NVFP4 layout with the recipe: gscale = fp32(amax / (6*448));
 * per 16-block scale = E4M3 round-to-nearest-even of amax_block/(6*gscale),
 * saturating at 448; code = sign(w) | E2M1 round-to-nearest-even of
 * |w| / (scale*gscale) (magnitude 0 when that product is 0).
 * tensor_scale: device float[2]; [0] receives gscale, [1] the tensor amax.
 * codes: [N][K/2], scales: [N][K/16] (canonical).  Requires K % 16 == 0,
 * W 16-byte aligned.  Errors: NULL, RANGE, SHAPE, ALIGN, LAUNCH. */
int nvfp4_quantize(const float *W, int N, int K, uint8_t *codes, uint8_t *scales,
                   float *tensor_scale, void *stream);

/* Input element types of nvfp4_quantize_packed. */
#define NVFP4_DTYPE_F32 0
#define NVFP4_DTYPE_BF16 1

/* The same recipe as nvfp4_quantize, writing the packed device layout
 * directly (no canonical copy, no nvfp4_pack pass): the pages' runtime
 * requantisation, whose fix emits the layout the GEMV reads during the
 * requant (Atlas PR #266 review and follow-up on the transposed copy).  W is
 * [N][K] row-major, fp32 (dtype NVFP4_DTYPE_F32, finite) or bf16 bit patterns
 * (NVFP4_DTYPE_BF16, widened to fp32 exactly, so the result is the fp32
 * recipe on the widened values), 16-byte aligned.  codes_packed /
 * scales_packed: device buffers of nvfp4_packed_*_bytes(N, K), 16-byte
 * aligned, byte-identical to nvfp4_pack(nvfp4_quantize(W)) including the zero
 * padding.  tensor_scale: device float[2] = {gscale, amax}.  Errors: NULL,
 * RANGE (N, K, dtype), SHAPE (K % 16), ALIGN, DEVICE, LAUNCH. */
int nvfp4_quantize_packed(const void *W, int dtype, int N, int K, uint8_t *codes_packed,
                          uint8_t *scales_packed, float *tensor_scale, void *stream);

/* Reorder canonical codes/scales (device) into the packed device layout
 * (device buffers of nvfp4_packed_*_bytes; the padding is written as zeros):
 * the one-time layout step the pages ask for, the weight copy the fast kernel
 * reads, made once at load instead of on every call (Atlas PR #266 automated
 * review page, "Tiebreaker" comment: the wide GEMM's fast path needs such a
 * copy, and emitting it at load is named as the fix).  A pure byte gather
 * (nibble order unchanged), so packing loses nothing.  Errors: NULL, RANGE,
 * SHAPE, ALIGN (packed buffers must be 16-byte aligned), LAUNCH, DEVICE. */
int nvfp4_pack(const uint8_t *codes, const uint8_t *scales, int N, int K,
               uint8_t *codes_packed, uint8_t *scales_packed, void *stream);

/* Y[n][N] = X[n][K] . dequant(W)^T for 1 <= n <= 16 tokens: one projection
 * of n concurrent decode tokens that reads the weight once for all of them
 * (Atlas PR #266 conversation page, PR description "What it does": a tile of
 * tokens shares one read of the projection weight instead of one read per
 * token).  Here the tile is the whole batch of up to 16 tokens.
 * Wq / Wscale: packed layout (nvfp4_pack), 16-byte aligned.
 * X: bf16 [n][K], 16-byte aligned.  Y: bf16 [n][N], 2-byte aligned.
 * Each token's result is bit-identical to the same token computed alone
 * (n = 1) and under any schedule of nvfp4_gemv_sched.  Any N >= 1 and any
 * K % 16 == 0 up to 262144; K beyond 8192 runs in several K-chunk passes
 * inside the one launch.  Errors: NULL, RANGE, SHAPE (K % 16, K > 262144, or
 * a workgroup's share of the weight beyond 2 GiB), ALIGN, LAUNCH, DEVICE. */
int nvfp4_gemv(const uint8_t *Wq, const uint8_t *Wscale, float gscale,
               const uint16_t *X, uint16_t *Y, int n, int N, int K, void *stream);

/* nvfp4_gemv with the K dimension cut into ks parts, for long-K projections
 * such as a dense FFN's down projection (the dense-FFN decode paths of the
 * spark_model::layers page's FfnComponent dispatch).  One launch computes the
 * fp32 partial of each (K part, 16-row group) unit into `workspace`
 * ([ks][n][N] fp32, DEVICE, 16-byte aligned, at least
 * nvfp4_gemv_workspace_bytes(n, N, K, ks) bytes, owned by the caller); a
 * second launch on the same stream adds the parts in part
 * order, scales by gscale and rounds to bf16.  The parts fill the chip where
 * N alone has fewer 16-row groups than there are compute units and cut the
 * share of X each compute unit loads.  ks = 0 takes nvfp4_gemv_kparts(N, K);
 * ks = 1 is exactly nvfp4_gemv (no workspace needed, none touched).  The sum
 * order depends only on (N, K, ks), so each token's result is bit-identical
 * to the same token alone (n = 1) at the same ks; across different ks the
 * rounding order differs (all within the documented fp32 error bound).
 * Calls that share a workspace on different streams race.  Errors: as
 * nvfp4_gemv; RANGE (ks < 0 or ks > 64), SHAPE (with T = ceil(K/128) and
 * tp = ceil(T/ks) tiles per part: a part would be empty, ks > T or
 * (ks-1)*tp >= T, or longer than one pass, ks > 1 and tp > 64),
 * WORKSPACE (ks > 1 and workspace NULL or too small), ALIGN (workspace). */
int nvfp4_gemv_ws(const uint8_t *Wq, const uint8_t *Wscale, float gscale,
                  const uint16_t *X, uint16_t *Y, int n, int N, int K, int ks,
                  void *workspace, size_t workspace_bytes, void *stream);

/* nvfp4_gemv_ws for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results (bit for bit) as nvfp4_gemv_ws, except
 * that the fp32 partials go to a fixed scratch array inside the library
 * instead of a caller workspace: nvfp4_gemv_static_scratch_bytes() bytes
 * (8 MiB) of device memory per GPU the library runs on, held until the
 * process ends.  Its address on a device is looked up on the first call with
 * ks > 1 on that device (make that first call outside graph capture); no call
 * allocates or frees anything.  Every element the reduction reads is written
 * earlier in the same call, so nothing needs clearing between calls.  All
 * calls on one GPU share the array: calls that overlap on one GPU (other
 * streams, other threads) race and give wrong results; calls ordered on one
 * stream are safe.  Errors: as nvfp4_gemv_ws (no WORKSPACE), SCRATCH when
 * ks * n * N * 4 bytes exceed the scratch (checked before any HIP call),
 * DEVICE if the scratch address cannot be looked up. */
int nvfp4_gemv_ws_static(const uint8_t *Wq, const uint8_t *Wscale, float gscale,
                         const uint16_t *X, uint16_t *Y, int n, int N, int K, int ks,
                         void *stream);

/* Bytes of the fixed scratch nvfp4_gemv_ws_static uses (8 MiB).  Pure host
 * function. */
size_t nvfp4_gemv_static_scratch_bytes(void);

/* K parts nvfp4_gemv_ws takes for ks = 0, from the shape alone: 1 while K <=
 * 8192 (one pass of the 8 waves' X slices); beyond, the part count that
 * minimises (rounds of 16-row groups per compute unit of MI355X's 256) x
 * (128-column tiles per part) with every part within one pass, the fewest on
 * a tie (4 for 5120 x 17408).  Pure host function; returns ks >= 1 or a
 * negative status (-RANGE, -SHAPE). */
int nvfp4_gemv_kparts(int N, int K);

/* Bytes of workspace nvfp4_gemv_ws needs for (n, N, K, ks): ks * n * N * 4
 * for ks > 1 (ks = 0: nvfp4_gemv_kparts), 0 for ks = 1 and for invalid
 * arguments.  Pure host function. */
size_t nvfp4_gemv_workspace_bytes(int n, int N, int K, int ks);

/* Fused QKV projection (Atlas PR #266, PR description, multi_seq/qkv.rs
 * bullet: one fused weight whose q, k and v rows land at fixed offsets of a
 * per-sequence buffer).  W has N = rows[0]+rows[1]+rows[2] rows: rows
 * [0,rows[0]) are q, the next rows[1] are k, the last rows[2] are v.  Token t's
 * q/k/v outputs are written straight to Y + t*ldy + out_off[p] + j (j < rows[p])
 * with no scratch buffer and no device-to-device copy.  The three output
 * ranges must not overlap and must fit in ldy (ldy >= out_off[p] + rows[p]).
 * rows / out_off are HOST arrays read during the call.  Same bit-identity
 * guarantees as nvfp4_gemv; results equal the three slices of nvfp4_gemv on
 * the same weight bit for bit.  Errors: as nvfp4_gemv, RANGE for bad
 * rows/out_off/ldy. */
int nvfp4_gemv_qkv(const uint8_t *Wq, const uint8_t *Wscale, float gscale,
                   const uint16_t *X, uint16_t *Y, int n, int K,
                   const int32_t rows[3], const int64_t out_off[3], int64_t ldy,
                   void *stream);

/* nvfp4_gemv under an explicit token-tile schedule: tile_widths (HOST array
 * of ntiles entries, each in [1,16], summing to n) splits the n tokens into
 * consecutive tiles, each one launch that reads the whole weight once.  This
 * is how the pages' greedy [3,3,...,2|1] tiling (Atlas PR #266 description)
 * is reproduced for comparison.  Errors: as nvfp4_gemv, SCHEDULE for a bad
 * schedule (never a silent fallback). */
int nvfp4_gemv_sched(const uint8_t *Wq, const uint8_t *Wscale, float gscale,
                     const uint16_t *X, uint16_t *Y, int n, int N, int K,
                     const uint8_t *tile_widths, int ntiles, void *stream);

/* The dispatcher's schedule for (n, N, K): writes the tile widths nvfp4_gemv
 * uses into widths (HOST, capacity max_tiles) and returns their count, or a
 * negative status (RANGE, SHAPE for a shape nvfp4_gemv refuses, SCHEDULE for
 * no room).  Pure host function. */
int nvfp4_schedule(int n, int N, int K, uint8_t *widths, int max_tiles);

/* The pages' greedy schedule (Atlas PR #266 description): as many tiles of
 * `width` tokens as fit, then one tile with the remaining tokens; with width 3
 * a batch of 8 tokens takes 3 weight reads.  Returns the tile count or a
 * negative status.  Pure host function. */
int nvfp4_schedule_greedy(int n, int width, uint8_t *widths, int max_tiles);

/* Launch geometry the library uses for (n, N, K): workgroups, waves per
 * workgroup and 128-column tiles per wave.  Pure host function; returns a
 * status. */
int nvfp4_launch_geometry(int n, int N, int K, int *workgroups, int *waves,
                          int *tiles_per_wave);

/* The GEMV kernel a call launches for (n, N, K) with ks K parts (ks = 1:
 * nvfp4_gemv, nvfp4_gemv_qkv and every tile of nvfp4_gemv_sched; ks = 0: the
 * part count nvfp4_gemv_ws takes, nvfp4_gemv_kparts(N, K); ks > 1: that many
 * parts of nvfp4_gemv_ws).  The kernel is specialised on five values, which
 * variant (HOST int[5]) receives: [0] 128-column tiles of each wave's K-slice
 * in one pass (1 .. 8), [1] groups of four tokens carried, ceil(n/4), [2] 1 if
 * every wave owns exactly [0] tiles of every pass (no column predication),
 * [3] K-chunk passes inside the launch (1 = one pass), [4] K parts.  Lets a
 * caller, and the tests, know which specialisation serves a shape (the tile
 * schedule and its variants are the dispatch the PR description describes,
 * here picked from the shape).  Pure host function; returns a status (RANGE,
 * SHAPE as nvfp4_gemv_ws would). */
int nvfp4_gemv_variant(int n, int N, int K, int ks, int *variant);

/* Largest token count of one nvfp4_gemm call. */
#define NVFP4_MAX_GEMM_TOKENS (1 << 20)

/* Prefill / many-token form of the same operation (the step after decode as
 * n grows: the spark_model::layers page's W4A16 tile GEMMs for prefill, with
 * tile shapes picked by an occupancy rule):
 *     Y[t][r] = gscale * sum_k X[t][k] * e2m1(code[r][k]) * e4m3(scale[r][k/16])
 * for any 1 <= n <= NVFP4_MAX_GEMM_TOKENS.  Same packed weight (nvfp4_pack),
 * X bf16 [n][K] and Y bf16 [n][N] (row-major, contiguous) as nvfp4_gemv.
 * The weight is dequantised exactly to bf16 once per token tile (32, 64 or
 * 128 tokens) and multiplied with MFMA, fp32 accumulation over all of K.
 * Each token's result is bit-identical whatever n and its place in the batch
 * (the sum over K runs in one fixed order), but it is a different rounding
 * order from nvfp4_gemv's (both within the documented fp32 error bound).
 * For n <= 16 nvfp4_gemv is the faster call: it splits K over the waves of a
 * workgroup and keeps many more weight bytes in flight (on MI355X, 14336 x
 * 5120 fused QKV at n = 16: about 10 us against 18.5 us; nvfp4_gemm takes
 * 18.4 - 18.7 us at any n <= 16, where it runs the 32-token tile).
 * Errors: NULL, RANGE (n, N, K), SHAPE (K % 16, K > 262144), ALIGN (Wq,
 * Wscale, X 16-byte; Y 2-byte), DEVICE, LAUNCH. */
int nvfp4_gemm(const uint8_t *Wq, const uint8_t *Wscale, float gscale,
               const uint16_t *X, uint16_t *Y, int n, int N, int K, void *stream);

/* Tile shape and grid nvfp4_gemm uses for (n, N, K) on MI355X: weight rows
 * and tokens per workgroup, workgroups along rows and along tokens.  Tokens:
 * the smallest of 32 / 64 / 128 holding n.  Rows: 256 (8 waves) when that grid
 * gives at least half of the 256 compute units a workgroup (also with 64-token
 * tiles instead of two or more 128-token tiles where only they get there),
 * else 64 (4 waves, or 8 waves sharing the row groups' tokens when there is
 * one 128-token tile).
 * Pure host function; returns a status. */
int nvfp4_gemm_geometry(int n, int N, int K, int *rows_per_workgroup,
                        int *tokens_per_workgroup, int *grid_x, int *grid_y);

/* Human-readable name of a status code (static storage). */
const char *nvfp4_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
