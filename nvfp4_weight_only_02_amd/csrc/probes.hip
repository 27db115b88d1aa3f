// libnvfp4_probes: measurement aids beside the NVFP4 decode projection, not
// part of it (C ABI in include/nvfp4_probes.h; libnvfp4 never calls them).
//
// nvfp4_probe_block_rate: the issue rate of the two ways to multiply one
// 16-element NVFP4 block of a 16-row group by n <= 16 decode tokens on gfx950,
// on register data with no memory traffic.
//
//  * MFMA (what nvfp4_gemv does): two v_cvt_scalef32_pk_bf16_fp4 (4 codes of
//    the lane's weight row -> exact bf16), one v_mfma_f32_16x16x16_bf16 with
//    the tokens as M, then ceil(n/4) fp32 FMAs applying the E4M3 block scale
//    (trailing the MFMA by two blocks), and one v_cvt_pk_f32_fp8 per two
//    blocks for the scales.
//  * VALU: the same conversions, then per token an 8-byte LDS read of the
//    token's 4 activations at the lane's K positions (the activation rows of
//    all n tokens cannot stay in registers), two v_dot2_f32_bf16 (4 MACs) and
//    one FMA with the block scale.
//
// Both run 8 waves per workgroup (two per SIMD, the GEMV's occupancy) on 256
// workgroups; each wave runs `blocks` blocks (rounded down to a multiple of
// 8) in groups of 8.  Each lane holds 8 code words; block j of a group uses
// word j XORed with the group's scalar counter (one VALU op, like a loaded
// tile: no block depends on the previous one, nothing can be hoisted).  A
// compiler barrier per group keeps the VALU path's LDS reads inside the loop.
// The outputs only feed a sink.
//
// nvfp4_probe_read_stream: one plain read of a buffer (the read ceiling the
// GEMV is compared with).  nvfp4_probe_empty: a launch that does nothing (the
// fixed cost of a launch).  nvfp4_probe_x_stage: the GEMV's staging of the
// activations alone (the loads, or the loads plus the per-wave LDS tile and
// the read-back into the MFMA operand layout), repeated inside one launch.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <type_traits>
#include <utility>

#include "../../include/nvfp4_probes.h"

namespace {

typedef unsigned int u32;
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kProbeWorkgroups = 256;
constexpr int kProbeThreads = 512;

__device__ __forceinline__ bf16x2 cvt_lo(u32 w) { return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0); }
__device__ __forceinline__ bf16x2 cvt_hi(u32 w) { return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1); }

template <typename F, int... J>
__device__ __forceinline__ void unroll_impl(F &&f, std::integer_sequence<int, J...>)
{
    (f(std::integral_constant<int, J>{}), ...);
}

template <int N, typename F>
__device__ __forceinline__ void unroll(F &&f)
{
    unroll_impl(f, std::make_integer_sequence<int, N>{});
}

template <int NT>
__global__ __launch_bounds__(kProbeThreads) void block_rate_mfma_kernel(u32 seed, int blocks, float *sink)
{
    constexpr int NV = (NT + 3) / 4;
    u32 wb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        wb[j] = (seed + (u32)j * 0x9E3779B9u) ^ (u32)(threadIdx.x * 2654435761u);
    const u32x2 xa = {wb[0] * 3u, wb[1] * 5u};
    const s16x4 aop = __builtin_bit_cast(s16x4, xa);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc = zero, p1 = zero, p2 = zero;
    float s1 = 0.f, s2 = 0.f;
    for (int b0 = 0; b0 + 8 <= blocks; b0 += 8) {
        float sc[2] = {1.f, 1.f};
        unroll<8>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const u32 w = wb[j] ^ (u32)b0;
            if constexpr ((j & 1) == 0) {
                const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)(w & 0x3F3F3F3Fu), false);
                sc[0] = f2[0];
                sc[1] = f2[1];
            }
            const u32x2 bw = {__builtin_bit_cast(u32, cvt_lo(w)), __builtin_bit_cast(u32, cvt_hi(w))};
            const f32x4 pr =
                __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aop, __builtin_bit_cast(s16x4, bw), zero, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < NV; ++v)
                acc[v] = __builtin_fmaf(s2, p2[v], acc[v]);
            p2 = p1;
            s2 = s1;
            p1 = pr;
            s1 = sc[j & 1];
            asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
        });
    }
    float r = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v)
        r += __builtin_fmaf(s1, p1[v], __builtin_fmaf(s2, p2[v], acc[v]));
    sink[blockIdx.x * kProbeThreads + threadIdx.x] = r;
}

template <int NT>
__global__ __launch_bounds__(kProbeThreads) void block_rate_valu_kernel(u32 seed, int blocks, float *sink)
{
    // Per wave: 8 blocks x 16 tokens x 16 columns of bf16 activations (4 KiB),
    // read back as the lane's 4 columns of each token.
    __shared__ u32x2 xs[kProbeThreads / 64][8][16][4];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    u32 wb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        wb[j] = (seed + (u32)j * 0x9E3779B9u) ^ (u32)(threadIdx.x * 2654435761u);
    for (int e = lane; e < 8 * 16 * 4; e += 64)
        xs[wave][e >> 6][(e >> 2) & 15][e & 3] = u32x2{wb[0] + (u32)e * 0x9E3779B9u, wb[1] ^ (u32)e};
    __syncthreads();
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        acc[t] = 0.f;
    for (int b0 = 0; b0 + 8 <= blocks; b0 += 8) {
        float sc[2] = {1.f, 1.f};
        asm volatile("" ::: "memory");
        unroll<8>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const u32 w = wb[j] ^ (u32)b0;
            if constexpr ((j & 1) == 0) {
                const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)(w & 0x3F3F3F3Fu), false);
                sc[0] = f2[0];
                sc[1] = f2[1];
            }
            const bf16x2 lo = cvt_lo(w), hi = cvt_hi(w);
            const float s = sc[j & 1];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const u32x2 x = xs[wave][j][t][g];
                // The words are copied to scalars first: __builtin_bit_cast of
                // an ext-vector element reads element 0 with this compiler.
                const u32 x0 = x[0], x1 = x[1];
                float part = __builtin_amdgcn_fdot2_f32_bf16(lo, __builtin_bit_cast(bf16x2, x0), 0.f, false);
                part = __builtin_amdgcn_fdot2_f32_bf16(hi, __builtin_bit_cast(bf16x2, x1), part, false);
                acc[t] = __builtin_fmaf(s, part, acc[t]);
            }
        });
    }
    float r = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
        r += acc[t];
    sink[blockIdx.x * kProbeThreads + threadIdx.x] = r;
}

typedef void (*ProbeKernel)(u32, int, float *);

template <int NT>
ProbeKernel pick_probe(int path)
{
    return path == NVFP4_RATE_MFMA ? block_rate_mfma_kernel<NT> : block_rate_valu_kernel<NT>;
}

ProbeKernel pick_probe_n(int path, int n)
{
    switch (n) {
    case 1: return pick_probe<1>(path);
    case 2: return pick_probe<2>(path);
    case 4: return pick_probe<4>(path);
    case 8: return pick_probe<8>(path);
    case 12: return pick_probe<12>(path);
    default: return pick_probe<16>(path);
    }
}

constexpr int kReadThreads = 1024;
constexpr int kReadUnroll = 4;

// Workgroup w reads its contiguous chunk of `chunk16` 16-byte words, four
// non-temporal loads in flight per lane; the xor of everything read goes to
// *sink only if it equals a value no real data produces here, so the loads
// stay live and nothing is written in practice.
__global__ __launch_bounds__(kReadThreads) void read_stream_kernel(const u32x4 *buf, size_t n16, size_t chunk16,
                                                                   unsigned *sink)
{
    const size_t s0 = (size_t)blockIdx.x * chunk16;
    const size_t s1 = s0 + chunk16 < n16 ? s0 + chunk16 : n16;
    u32 acc = 0;
    for (size_t o = s0 + threadIdx.x; o < s1; o += (size_t)kReadThreads * kReadUnroll) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const size_t q = o + (size_t)u * kReadThreads;
            v[u] = q < s1 ? __builtin_nontemporal_load(buf + q) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == 0x9E3779B9u)
        sink[0] = acc;
}

__global__ __launch_bounds__(512) void empty_kernel() {}

// The activation staging of nvfp4_gemv for a K-slice of MT 128-column tiles
// per wave (wave w: tiles w, w + 8, ...), `reps` times: whole-line 16-byte
// buffer loads of the token rows of each tile (lane l: row 4q + l/16, bytes
// 16 * (l % 16) of the tile's 256; a row beyond n or a column beyond K reads
// nothing, as in the GEMV), then with FULL the per-wave LDS tile and the
// read-back of each lane's MFMA A fragments (token 4(i%4) + i/4, columns
// 16b + 4g .. +3 of block b).  As in the GEMV, only the NV = ceil(n/4) groups
// of four token rows that hold a token are loaded and written, and only the
// lanes whose MFMA row carries a token read back.  Everything feeds a
// checksum that reaches *sink only for a value the benchmark's data never
// produces.
template <int MT, int NV, bool FULL>
__global__ __launch_bounds__(kProbeThreads) void x_stage_kernel(const u32x4 *__restrict__ x, int n, int K,
                                                                int reps, u32 *sink)
{
    // range-checked resource over X's n*K bf16 (gfx9 raw buffer word 3)
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4 *>(x), (short)0,
                                                                        n * K * 2, 0x00020000);
    __shared__ u32x4 xs[kProbeThreads / 64][16][17];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int i = lane & 15, g = lane >> 4, chunk = lane & 15;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const bool xlane = 4 * (i & 3) + (i >> 2) < 4 * NV;
    u32 acc = 0;
    for (int rep = 0; rep < reps; ++rep) {
        asm volatile("" ::: "memory");   // every repetition loads again
        u32x4 v[MT][4];
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = q * 4 + (lane >> 4);
                const int k = (w + 8 * t) * 128 + chunk * 8;
                v[t][q] = z;
                if (q < NV)
                    v[t][q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                            xr, row < n && k < K ? (unsigned)(row * K + k) * 2u
                                                                                 : 0x7FFFFFF0u, 0, 0));
            }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if constexpr (!FULL) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc ^= v[t][q][0] + 3u * v[t][q][1] + 5u * v[t][q][2] + 7u * v[t][q][3];
            } else {
#pragma unroll
                for (int q = 0; q < NV; ++q)
                    xs[w][q * 4 + (lane >> 4)][chunk] = v[t][q];
                const char *base = reinterpret_cast<const char *>(&xs[w][4 * (i & 3) + (i >> 2)][0]);
                if (xlane) {
#pragma unroll
                    for (int b = 0; b < 8; ++b) {
                        const u32x2 r = *reinterpret_cast<const u32x2 *>(base + (16 * b + 4 * g) * 2);
                        acc ^= r[0] + 3u * r[1];
                    }
                }
            }
        }
    }
    if (acc == 0x9E3779B9u)
        sink[0] = acc;
}

typedef void (*XStageKernel)(const u32x4 *, int, int, int, u32 *);

template <int MT, int NV>
XStageKernel pick_x_stage_mode(int mode)
{
    return mode == NVFP4_XSTAGE_FULL ? x_stage_kernel<MT, NV, true> : x_stage_kernel<MT, NV, false>;
}

template <int MT>
XStageKernel pick_x_stage_nv(int n, int mode)
{
    switch ((n + 3) / 4) {
    case 1: return pick_x_stage_mode<MT, 1>(mode);
    case 2: return pick_x_stage_mode<MT, 2>(mode);
    case 3: return pick_x_stage_mode<MT, 3>(mode);
    default: return pick_x_stage_mode<MT, 4>(mode);
    }
}

XStageKernel pick_x_stage(int mt, int n, int mode)
{
    switch (mt) {
    case 1: return pick_x_stage_nv<1>(n, mode);
    case 2: return pick_x_stage_nv<2>(n, mode);
    case 3: return pick_x_stage_nv<3>(n, mode);
    case 4: return pick_x_stage_nv<4>(n, mode);
    case 5: return pick_x_stage_nv<5>(n, mode);
    case 6: return pick_x_stage_nv<6>(n, mode);
    case 7: return pick_x_stage_nv<7>(n, mode);
    default: return pick_x_stage_nv<8>(n, mode);
    }
}

}  // namespace

extern "C" {

int nvfp4_probe_block_rate(int path, int n, int blocks, float *sink, size_t sink_bytes, void *stream)
{
    if (!sink)
        return NVFP4_ERR_NULL;
    if ((path != NVFP4_RATE_MFMA && path != NVFP4_RATE_VALU) || blocks < 8 ||
        (n != 1 && n != 2 && n != 4 && n != 8 && n != 12 && n != 16))
        return NVFP4_ERR_RANGE;
    if (sink_bytes < (size_t)kProbeWorkgroups * kProbeThreads * sizeof(float))
        return NVFP4_ERR_RANGE;
    if ((uintptr_t)sink % 4 != 0)
        return NVFP4_ERR_ALIGN;
    hipLaunchKernelGGL(pick_probe_n(path, n), dim3(kProbeWorkgroups), dim3(kProbeThreads), 0,
                       (hipStream_t)stream, 0x1234567u, blocks, sink);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

int nvfp4_probe_read_stream(const void *buf, size_t bytes, uint32_t *sink, void *stream)
{
    if (!buf || !sink)
        return NVFP4_ERR_NULL;
    if (bytes == 0 || bytes % 16 != 0)
        return NVFP4_ERR_RANGE;
    if ((uintptr_t)buf % 16 != 0 || (uintptr_t)sink % 4 != 0)
        return NVFP4_ERR_ALIGN;
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
        strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return NVFP4_ERR_DEVICE;
    // About 40 KiB per workgroup, at least 256 workgroups (measured best on
    // MI355X from 17 MB to 1 GiB: 1 GiB reads at 6.87 TB/s this way, at 6.26
    // TB/s with the grid capped at 2048 workgroups of 512 KiB each).
    const size_t n16 = bytes / 16;
    size_t grid = (bytes + 40959) / 40960;
    grid = grid < 256 ? 256 : grid;
    if (grid > 0x7FFFFFFF)
        return NVFP4_ERR_RANGE;
    const size_t chunk16 = (n16 + grid - 1) / grid;
    hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)grid), dim3(kReadThreads), 0, (hipStream_t)stream,
                       reinterpret_cast<const u32x4 *>(buf), n16, chunk16, sink);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

int nvfp4_probe_x_stage(const uint16_t *X, int n, int K, int workgroups, int reps, int mode, uint32_t *sink,
                        void *stream)
{
    if (!X || !sink)
        return NVFP4_ERR_NULL;
    if (n < 1 || n > 16 || K < 128 || K > 8192 || K % 128 != 0 || workgroups < 1 || workgroups > 65536 ||
        reps < 1 || reps > 1024 || (mode != NVFP4_XSTAGE_LOADS && mode != NVFP4_XSTAGE_FULL))
        return NVFP4_ERR_RANGE;
    if ((uintptr_t)X % 16 != 0 || (uintptr_t)sink % 4 != 0)
        return NVFP4_ERR_ALIGN;
    const int mt = (K / 128 + 7) / 8;
    hipLaunchKernelGGL(pick_x_stage(mt, n, mode), dim3((unsigned)workgroups), dim3(kProbeThreads), 0,
                       (hipStream_t)stream, reinterpret_cast<const u32x4 *>(X), n, K, reps, sink);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

int nvfp4_probe_empty(int workgroups, void *stream)
{
    if (workgroups < 1 || workgroups > 65536)
        return NVFP4_ERR_RANGE;
    hipLaunchKernelGGL(empty_kernel, dim3((unsigned)workgroups), dim3(512), 0, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

}  // extern "C"
