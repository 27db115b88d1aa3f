/* A plain C caller of libnvfp4: only include/nvfp4.h and the HIP runtime API,
 * no Python.  It reads a weight in the canonical layout (E2M1 code bytes and
 * E4M3 scale bytes) and n bf16 activation rows from files, packs the weight on
 * the GPU with nvfp4_pack, runs nvfp4_gemv and nvfp4_gemv_qkv (the same weight
 * split in three projections written at permuted offsets of a wider row), and
 * writes both outputs to files.  It also checks that a few invalid calls are
 * refused with the documented status before any GPU work.
 *
 * usage: gemv_client N K n gscale codes.bin scales.bin x.bin y.bin y_qkv.bin
 *   codes.bin: N*K/2 bytes, scales.bin: N*K/16 bytes, x.bin: n*K bf16,
 *   y.bin: n*N bf16 (out),
 *   y_qkv.bin: n rows of N+32 bf16 (out): 32 zeros, then v (the last
 *   N - N/2 - N/4 rows of W), q (the first N/2 rows), k (the next N/4 rows).
 * Exit status 0 on success; a message on stderr otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "nvfp4.h"

static int fail(const char *what, const char *detail)
{
    fprintf(stderr, "gemv_client: %s: %s\n", what, detail);
    return 1;
}

static void *read_file(const char *path, size_t bytes)
{
    FILE *f = fopen(path, "rb");
    if (!f)
        return NULL;
    void *buf = malloc(bytes ? bytes : 1);
    if (buf && fread(buf, 1, bytes, f) != bytes) {
        free(buf);
        buf = NULL;
    }
    fclose(f);
    return buf;
}

static int write_file(const char *path, const void *buf, size_t bytes)
{
    FILE *f = fopen(path, "wb");
    if (!f)
        return 0;
    size_t w = fwrite(buf, 1, bytes, f);
    fclose(f);
    return w == bytes;
}

#define HIP(call)                                                    \
    do {                                                             \
        hipError_t e_ = (call);                                      \
        if (e_ != hipSuccess)                                        \
            return fail(#call, hipGetErrorString(e_));               \
    } while (0)

#define NV(call)                                                     \
    do {                                                             \
        int s_ = (call);                                             \
        if (s_ != NVFP4_OK)                                          \
            return fail(#call, nvfp4_strerror(s_));                  \
    } while (0)

int main(int argc, char **argv)
{
    if (argc != 10)
        return fail("usage", "gemv_client N K n gscale codes.bin scales.bin x.bin y.bin y_qkv.bin");
    const int N = atoi(argv[1]), K = atoi(argv[2]), n = atoi(argv[3]);
    const float gscale = (float)atof(argv[4]);
    if (N < 3 || K < 16 || K % 16 != 0 || n < 1 || n > NVFP4_MAX_TOKENS)
        return fail("arguments", "need N >= 3, K a positive multiple of 16, 1 <= n <= 16");
    const size_t code_bytes = (size_t)N * K / 2, scale_bytes = (size_t)N * K / 16;
    const size_t x_bytes = (size_t)n * K * 2, y_bytes = (size_t)n * N * 2;
    uint8_t *codes = read_file(argv[5], code_bytes);
    uint8_t *scales = read_file(argv[6], scale_bytes);
    uint16_t *x = read_file(argv[7], x_bytes);
    if (!codes || !scales || !x)
        return fail("reading inputs", argv[5]);

    /* Invalid calls are refused before any GPU work (host-side validation). */
    if (nvfp4_gemv(NULL, NULL, 1.0f, NULL, NULL, 1, N, K, NULL) != NVFP4_ERR_NULL)
        return fail("validation", "NULL pointers not refused");
    if (nvfp4_packed_codes_bytes(N, K + 8) != 0)
        return fail("validation", "K % 16 != 0 not refused by nvfp4_packed_codes_bytes");

    const size_t pc = nvfp4_packed_codes_bytes(N, K), ps = nvfp4_packed_scales_bytes(N, K);
    uint8_t *d_codes, *d_scales, *d_pc, *d_ps;
    uint16_t *d_x, *d_y, *d_yq;
    /* ldy of the fused-QKV output: 32 bf16 of gap before the projections */
    const int64_t ldy = (int64_t)N + 32;
    HIP(hipMalloc((void **)&d_codes, code_bytes));
    HIP(hipMalloc((void **)&d_scales, scale_bytes));
    HIP(hipMalloc((void **)&d_pc, pc));
    HIP(hipMalloc((void **)&d_ps, ps));
    HIP(hipMalloc((void **)&d_x, x_bytes));
    HIP(hipMalloc((void **)&d_y, y_bytes));
    HIP(hipMalloc((void **)&d_yq, (size_t)n * ldy * 2));
    HIP(hipMemcpy(d_codes, codes, code_bytes, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_scales, scales, scale_bytes, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_x, x, x_bytes, hipMemcpyHostToDevice));
    HIP(hipMemset(d_yq, 0, (size_t)n * ldy * 2));

    if (nvfp4_gemv(d_pc, d_ps, gscale, d_x, d_y, 0, N, K, NULL) != NVFP4_ERR_RANGE)
        return fail("validation", "n = 0 not refused");

    NV(nvfp4_pack(d_codes, d_scales, N, K, d_pc, d_ps, NULL));
    NV(nvfp4_gemv(d_pc, d_ps, gscale, d_x, d_y, n, N, K, NULL));
    /* the same weight as q | k | v (rows split N/2, N/4, the rest), written in
     * the order v, q, k after a 32-element gap */
    const int32_t rows[3] = {N / 2, N / 4, N - N / 2 - N / 4};
    const int64_t off[3] = {32 + rows[2], 32 + rows[2] + rows[0], 32};
    NV(nvfp4_gemv_qkv(d_pc, d_ps, gscale, d_x, d_yq, n, K, rows, off, ldy, NULL));
    HIP(hipDeviceSynchronize());

    uint16_t *y = malloc(y_bytes), *yq = malloc((size_t)n * ldy * 2);
    if (!y || !yq)
        return fail("malloc", "output buffers");
    HIP(hipMemcpy(y, d_y, y_bytes, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(yq, d_yq, (size_t)n * ldy * 2, hipMemcpyDeviceToHost));
    if (!write_file(argv[8], y, y_bytes) || !write_file(argv[9], yq, (size_t)n * ldy * 2))
        return fail("writing outputs", argv[8]);

    hipFree(d_codes);
    hipFree(d_scales);
    hipFree(d_pc);
    hipFree(d_ps);
    hipFree(d_x);
    hipFree(d_y);
    hipFree(d_yq);
    free(codes);
    free(scales);
    free(x);
    free(y);
    free(yq);
    printf("gemv_client: ok N=%d K=%d n=%d\n", N, K, n);
    return 0;
}
