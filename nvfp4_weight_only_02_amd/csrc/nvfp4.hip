// libnvfp4: NVFP4 weight-only projection GEMV of batched LLM decode on MI355X
// (gfx950), behind the C ABI of include/nvfp4.h.
//
// What is computed (Atlas PR #266, PR description "What it does"): for n <= 16
// concurrent decode tokens, Y[t][r] = gscale * sum_k X[t][k] * w(r,k) with w an
// NVFP4 weight (E2M1 code times the E4M3 scale of its 16-element K-block), the
// weight matrix read once for all tokens.
//
// Design (gfx950-first; the pages' CUDA kernels are prior art only):
//  * Packed layout: 16-row x 128-column tiles.  A tile's 1 KiB of codes is one
//    16-byte load per lane of a 64-lane wavefront, laid out so that the bytes a
//    lane loads are exactly the MFMA operand fragments it feeds.  A wave's
//    block scales for one row group (its tiles' 128-byte scale rows, contiguous)
//    are one 16-byte load per lane, passed to the lanes that need them through
//    a small per-wave LDS buffer.
//  * Dequant in registers: v_cvt_scalef32_pk_bf16_fp4 turns two E2M1 codes into
//    two exact bf16 values per instruction.  The E4M3 block scale is NOT folded
//    into that conversion (the hardware applies only the exponent of its f32
//    scale operand); instead each 16-element K-block is one
//    v_mfma_f32_16x16x16_bf16 whose fp32 partial is multiplied by the block
//    scale with one fp32 FMA per output.
//  * Tokens are the MFMA M dimension, padded to 16, token t on MFMA row
//    4*(t%4) + t/4.  Accumulator component v of a lane then holds tokens
//    4v..4v+3, so a launch of n tokens runs the scale FMAs of the first
//    ceil(n/4) components only.  A token always sits on the same MFMA row and
//    its component runs the same instruction sequence whatever n is, so its
//    result never depends on n or on the other tokens (bit-identity with the
//    n = 1 result).
//  * Persistent workgroups, 8 waves each, one contiguous range of row groups
//    per workgroup with the ranges as even as the chip allows (every
//    workgroup runs the same number of rounds).  Each wave owns a fixed
//    K-slice, every 8th 128-column tile (wave w: tiles w, w+8, w+16, ...);
//    its slice of X sits in VGPRs for the whole launch (loaded once, straight
//    in MFMA A-operand layout, load instructions for token rows >= n
//    skipped), and it streams the weight tiles of its slice for consecutive
//    16-row groups, refilling each ring slot with the next row group's tile as
//    soon as it is consumed (a ring of one row group: measured faster than
//    deeper rings, whose loads return later and stall the compute behind them).
//    With interleaved slices the refills the 8 waves issue while they work
//    through a row group walk the next row group's tiles in ascending address
//    order (measured faster than contiguous slices, whose refills stride the
//    row group, at large n where the compute spreads them out).
//  * K-slice partials are summed through LDS in a fixed wave order, then
//    scaled by gscale and rounded to bf16 (RNE) in the epilogue, which writes
//    each projection's rows straight to its output offset (fused QKV).
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>
#include <type_traits>
#include <utility>

#include "../../include/nvfp4.h"

namespace {

typedef unsigned int u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kRowsPerGroup = 16;      // MFMA N dimension: weight rows per tile
constexpr int kTileK = 128;            // K columns per tile (8 NVFP4 blocks)
constexpr int kBlocksPerTile = kTileK / 16;
constexpr int kMaxTilesPerWave = 8;    // X slice of a wave: 16 VGPRs per tile
constexpr int kMaxTilesChunked = 7;    // per wave and K chunk when K needs several chunks
constexpr int kWaves = 8;            // waves per workgroup, one K-slice each
constexpr int kBufferWord3 = 0x00020000;   // gfx9 raw buffer resource: 32-bit data, no swizzle
constexpr unsigned kOutOfRange = 0x7FFFFFF0u;   // buffer offset past any resource: reads zeros
constexpr int kSlots = 8;                        // row-group partials parked in LDS
constexpr int kMaxK = 1 << 18;                   // keeps every buffer offset within 32 bits
constexpr int kMaxKParts = 64;                   // K parts of a split launch

// 16-row groups of N rows and 128-column tiles of K columns, rounded up in
// 64-bit arithmetic (no int near INT_MAX overflows).
constexpr long long row_groups(long long N)
{
    return (N + kRowsPerGroup - 1) / kRowsPerGroup;
}
constexpr long long k_tiles(long long K)
{
    return (K + kTileK - 1) / kTileK;
}

struct GemvParams {
    const u32x4 *codes;    // packed codes, [RG][T][64 lanes] x 16 B
    const u32x2 *scales;   // packed scales, [RG][T][16 rows] x 8 B
    const uint16_t *X;     // bf16 [n][K]
    uint16_t *Y;           // bf16 output, token stride ldy
    float gscale;
    int n, N, K, T, RG;
    int kc;                // K chunks (passes) of a K part: chunk c covers its tiles [c*8*MT, (c+1)*8*MT)
    int rg_base, rg_rem;   // row groups per workgroup: rg_base, +1 for the first rg_rem
    int start1, start2;    // first row of the 2nd and 3rd projection (N if absent)
    long long off0, off1, off2, ldy;
    // K split: workgroups [q*wpp, (q+1)*wpp) own the tiles [q*tp, min((q+1)*tp, T))
    // of K part q.  With P set they store fp32 partials P[q][t][r] (unscaled)
    // instead of Y; nvfp4_ksplit_reduce_kernel then sums the parts.
    int tp, wpp;
    float *P;
};

// Two E2M1 codes (byte `sel` of w) -> two bf16 values, unscaled (scale 1.0).
__device__ __forceinline__ u32 fp4x2_to_bf16x2(u32 w, int sel)
{
    bf16x2 v;
    switch (sel) {
    case 0: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0); break;
    case 1: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1); break;
    case 2: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2); break;
    default: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3); break;
    }
    return __builtin_bit_cast(u32, v);
}

// Calls f(std::integral_constant<int, j>) for j = 0 .. N-1.
template <typename F, int... J>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, J...>)
{
    (f(std::integral_constant<int, J>{}), ...);
}

template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// A raw buffer resource over [base, base + bytes) (gfx9 layout: 48-bit base,
// stride 0, byte-granular range check).
__device__ __forceinline__ u32x4 buffer_rsrc(const void *base, unsigned bytes)
{
    const unsigned long long a = (unsigned long long)base;
    return u32x4{(u32)a, (u32)(a >> 32) & 0xFFFFu, bytes, (u32)kBufferWord3};
}

// Loads whose completion is tracked by hand (see the vmcnt bookkeeping in
// the kernel).  Offsets past the resource's range return zeros.
__device__ __forceinline__ u32x4 buffer_load_b128(u32x4 rsrc, unsigned off)
{
    u32x4 v;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(off), "s"(rsrc));
    return v;
}

__device__ __forceinline__ u32x4 buffer_load_b128_nt(u32x4 rsrc, unsigned off)
{
    u32x4 v;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen nt" : "=v"(v) : "v"(off), "s"(rsrc));
    return v;
}

// Wait until at most N vector-memory operations are outstanding; the
// registers passed are the ones the wait makes valid (tied in and out, so no
// read of them can be scheduled before it).
template <int N>
__device__ __forceinline__ void vm_wait4(u32x4 &a, u32x4 &b, u32x4 &c, u32x4 &d, std::integral_constant<int, N>)
{
    static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit field");
    asm volatile("s_waitcnt vmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "n"(N));
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);   // v_cvt_pk_bf16_f32: RNE
}

template <int N>
__device__ __forceinline__ void vm_wait1(u32x4 &a, std::integral_constant<int, N>)
{
    static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit field");
    asm volatile("s_waitcnt vmcnt(%1)" : "+v"(a) : "n"(N));
}

// One launch covers every token (n <= 16) of one weight matrix.
//   MT    tiles of the K-slice each of the kWaves waves owns in one K chunk
//         (wave w: tiles cb + w + kWaves * t, t < MT, of the chunk that
//         starts at tile cb);
//   NV    ceil(n / 4): accumulator components that carry real tokens;
//   EXACT every wave owns exactly MT tiles of every chunk (of every K part)
//         (K == 128 * T, T == ks * tp, tp == kc * kWaves * MT), so no column
//         predication is needed;
//   CHUNKED K is longer than one chunk (8 waves x 8 tiles, whose X slices
//         fill the VGPRs): the launch runs kc passes over the workgroup's row
//         groups, one per K chunk, restaging X for each, and each wave adds
//         its chunk partials into its own LDS slots in chunk order;
//   SPLIT K is cut into parts of at most one chunk each: the workgroups of
//         part q cover its tiles only and store unscaled fp32 partials, which
//         nvfp4_ksplit_reduce_kernel sums in part order.
template <int MT, int NV, bool EXACT, bool CHUNKED, bool SPLIT>
__global__ __launch_bounds__(kWaves * 64) void nvfp4_gemv_kernel(GemvParams p)
{
    static_assert(!(SPLIT && CHUNKED), "a K part is one pass");
    constexpr int W = kWaves;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int i = lane & 15;   // MFMA row of A (token 4*(i%4) + i/4), weight row of B and C
    const int g = lane >> 4;   // K quarter of A and B, accumulator token offset of C

    const int kpart = SPLIT ? (int)blockIdx.x / p.wpp : 0;   // K part: tiles [pt0, pt1)
    const int wg = SPLIT ? (int)blockIdx.x - kpart * p.wpp : (int)blockIdx.x;
    const int pt0 = SPLIT ? kpart * p.tp : 0;
    const int pt1 = SPLIT ? min(p.T, pt0 + p.tp) : p.T;
    const int rg0 = wg * p.rg_base + min(wg, p.rg_rem);
    const int rg1 = rg0 + p.rg_base + (wg < p.rg_rem ? 1 : 0);
    // Wave w's slice of the K chunk that starts at tile cb: tiles w0 + W * t
    // (w0 = cb + w, t < MT), of which those before the part's end pt1 exist
    // (a prefix, since the tiles ascend with t).
    auto first_tile = [&](int cb) { return cb + wave; };
    auto tiles_in = [&](int w0) { return max(0, min(MT, (pt1 - w0 + W - 1) / W)); };
    int tw0 = first_tile(pt0);   // first tile of this wave's slice in the current K chunk
    int tw = MT;                 // tiles of it that exist

    // All vector-memory loads of the main path are inline buffer loads waited
    // for with explicit, compile-time vmcnt values: loads retire in issue
    // order, so "at most N newer loads outstanding" is exact bookkeeping, and
    // every read of a loaded register goes through the wait statement (its
    // operands are tied), so nothing reads a register whose load is still in
    // flight.  Buffer resources: X ends at row n, the weights at this
    // workgroup's last row group; loads past the end return zeros without a
    // memory access.
    const unsigned nrg = (unsigned)(rg1 - rg0);
    const u32x4 crsrc = buffer_rsrc(p.codes + (size_t)rg0 * p.T * 64, nrg * p.T * 1024u);
    const u32x4 srsrc = buffer_rsrc(reinterpret_cast<const char *>(p.scales) + (size_t)rg0 * p.T * 128,
                                    nrg * p.T * 128u);
    const u32x4 xrsrc = buffer_rsrc(p.X, (unsigned)(p.n * p.K * 2));

    // X first (it is cache-resident after the first workgroups touch it, so
    // its staging below never waits for an HBM load): lane (chunk, q) loads
    // the 16-byte chunk `chunk` of token row q*4 + lane/16 of each tile of
    // the slice (16 lanes cover one row's 256 bytes: whole-line loads).  Only
    // the NV = ceil(n/4) load instructions per tile whose four token rows hold
    // a real token are issued.
    constexpr int kStageRow = kTileK * 2 / 16 + 1;   // 16-byte chunks per row, +1 pad
    __shared__ u32x4 xstage[W][kRowsPerGroup][kStageRow];
    const int chunk = lane & 15;
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    u32x4 xg[MT][4];
    auto issue_x = [&]() {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xg[t][q] = z4;
                if (q < NV) {
                    const int row = q * 4 + (lane >> 4);
                    const int k = (tw0 + t * W) * kTileK + chunk * 8;
                    const bool ok = row < p.n && (EXACT || ((!SPLIT || t < tw) && k < p.K));
                    xg[t][q] = buffer_load_b128(xrsrc, ok ? (unsigned)(row * p.K + k) * 2u : kOutOfRange);
                }
            }
    };

    // Weight ring: one row group of this wave's K-slice, issued as
    // [scale chunk, code tile 0 .. MT-1].  The scale chunk is the 128 scale
    // bytes of each tile of the slice (lane l holds bytes 16(l%8) .. +15 of
    // local tile l/8), so local tile t's scales land at bytes 128t .. 128t+127.
    u32x4 wsc;
    u32x4 wc[MT];
    // Offsets of row group rgl of the K-slice whose first tile is w0 and
    // which holds wn tiles (w0, w0 + W, ...).
    auto scale_off_at = [&](int rgl, int w0, int wn) -> unsigned {
        return lane < 8 * wn ? (unsigned)((rgl * p.T + w0 + (lane >> 3) * W) * 128 + (lane & 7) * 16)
                             : kOutOfRange;
    };
    auto code_off_at = [&](int rgl, int t, int w0, int wn) -> unsigned {
        return (EXACT || t < wn) ? (unsigned)((rgl * p.T + w0 + t * W) * 1024 + lane * 16) : kOutOfRange;
    };
    auto scale_off = [&](int rgl) -> unsigned { return scale_off_at(rgl, tw0, tw); };
    auto code_off = [&](int rgl, int t) -> unsigned { return code_off_at(rgl, t, tw0, tw); };
    auto issue_ring = [&](int rgl) {
        wsc = buffer_load_b128_nt(srsrc, scale_off(rgl));
#pragma unroll
        for (int t = 0; t < MT; ++t)
            wc[t] = buffer_load_b128_nt(crsrc, code_off(rgl, t));
    };

    // Stage X through a per-wave LDS tile into MFMA A-operand layout: lane
    // (i, g) holds X[4*(i%4) + i/4][k .. k+3] with k = 16*block + 4*g, for
    // every block of the slice.  Every X load is older than the MT + 1 ring
    // loads; tile t is staged as soon as its own loads are in, while the
    // later tiles' X and the ring are still arriving.  The staging is
    // LDS-bandwidth bound (all waves of a CU stage at once), so only the NV
    // token quarters in use are written, and only the lanes whose MFMA row
    // carries one of them read (the other lanes' A rows stay zero; they only
    // feed outputs that are never stored).
    u32x2 xr[MT][kBlocksPerTile];
    const bool xlane = 4 * (i & 3) + (i >> 2) < 4 * NV;
    // RING_FIRST: this pass's ring was issued before its X loads (by the
    // previous pass), so only the later tiles' X loads are newer than tile t's.
    auto stage_x = [&](auto ring_first_tag) {
    constexpr bool RING_FIRST = decltype(ring_first_tag)::value;
    static_for<MT>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        // Newer than tile t's X loads: the later tiles' X loads and (unless
        // it was issued first) the ring.
        vm_wait4(xg[t][0], xg[t][1], xg[t][2], xg[t][3],
                 std::integral_constant<int, (MT - 1 - t) * NV + (RING_FIRST ? 0 : MT + 1)>{});
#pragma unroll
        for (int q = 0; q < NV; ++q)
            xstage[wave][q * 4 + (lane >> 4)][chunk] = xg[t][q];
        const char *base = reinterpret_cast<const char *>(&xstage[wave][4 * (i & 3) + (i >> 2)][0]);
#pragma unroll
        for (int b = 0; b < kBlocksPerTile; ++b)
            xr[t][b] = u32x2{0u, 0u};
        if (xlane) {
#pragma unroll
            for (int b = 0; b < kBlocksPerTile; ++b)
                xr[t][b] = *reinterpret_cast<const u32x2 *>(base + (16 * b + 4 * g) * 2);
        }
    });
    };

    // Partial sums of a batch of up to kSlots row groups wait in LDS (added
    // up over the K chunks) and are reduced together, so waves only meet at a
    // barrier once per batch (once per launch at the decode shapes) instead
    // of after every row group.
    __shared__ f32x4 part[kSlots][W][64];
    __shared__ u32x4 sstage[W][64];
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // One row group of this wave's K-slice.  REFILL: each ring slot is
    // refilled with the same slot of the next row group as soon as it is
    // consumed, so every wait has exactly MT newer loads (the ring); on the
    // last row group nothing is refilled and the counts fall as it drains.
    // Blocks run as a software pipeline (the scale FMA of a block trails its
    // MFMA by two blocks).
    auto rowgroup = [&](auto refill_tag, int rg, int nrgl, int nw0, int nwn) -> f32x4 {
        constexpr bool REFILL = decltype(refill_tag)::value;
        vm_wait1(wsc, std::integral_constant<int, MT>{});
        sstage[wave][lane] = wsc;
        asm volatile("" ::: "memory");
        if constexpr (REFILL)
            wsc = buffer_load_b128_nt(srsrc, scale_off_at(nrgl, nw0, nwn));
        const char *sbase = reinterpret_cast<const char *>(&sstage[wave][0]) + i * 8;
        f32x4 acc = zero, p1 = zero, p2 = zero;
        float s1 = 0.f, s2 = 0.f;
        static_for<MT>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            // E4M3 scales of blocks 0..7 of tile t for weight row i.
            const u32x2 sb = *reinterpret_cast<const u32x2 *>(sbase + t * 128);
            float sc[kBlocksPerTile];
            static_for<4>([&](auto hc) {
                constexpr int h = decltype(hc)::value;
                const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)sb[h >> 1], (h & 1) != 0);
                sc[2 * h] = f2[0];
                sc[2 * h + 1] = f2[1];
            });
            vm_wait1(wc[t], std::integral_constant<int, REFILL ? MT : MT - 1 - t>{});
            const u32x4 c = wc[t];
#pragma unroll
            for (int b = 0; b < kBlocksPerTile; ++b) {
                // B operand: W[row i][16*block + 4*g + e], e = 0..3, from
                // bytes 2*(b&1) and 2*(b&1)+1 of dword b/2.
                const u32 cw = c[b >> 1];
                const u32 lo = fp4x2_to_bf16x2(cw, (b & 1) * 2);
                const u32 hi = fp4x2_to_bf16x2(cw, (b & 1) * 2 + 1);
                const s16x4 bop = __builtin_bit_cast(s16x4, u32x2{lo, hi});
                const s16x4 aop = __builtin_bit_cast(s16x4, xr[t][b]);
                const f32x4 pr = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aop, bop, zero, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    acc[v] = __builtin_fmaf(s2, p2[v], acc[v]);
                p2 = p1;
                s2 = s1;
                p1 = pr;
                s1 = sc[b];
                // Pin the FMAs of this step here (instruction selection
                // would otherwise sink the whole FMA chain below every
                // MFMA and keep all partials live).
                asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
            }
            // Refill the slot once its codes are consumed, so the next
            // row group's tile lands in the same registers.
            if constexpr (REFILL)
                wc[t] = buffer_load_b128_nt(crsrc, code_off_at(nrgl, t, nw0, nwn));
        });
#pragma unroll
        for (int v = 0; v < NV; ++v)
            acc[v] = __builtin_fmaf(s1, p1[v], __builtin_fmaf(s2, p2[v], acc[v]));
        return acc;
    };

    // Sum the K-slices of row group rg in wave order 0..W-1, scale by gscale,
    // round to bf16 and store the row group's outputs.  Component v of lane
    // (g, i) is token 4v + g of weight row 16*rg + i.
    auto reduce_store = [&](int rg, int slot) {
        f32x4 sum = part[slot][0][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) {
            const f32x4 q = part[slot][w][lane];
#pragma unroll
            for (int v = 0; v < NV; ++v)
                sum[v] = sum[v] + q[v];
        }
        const int r = rg * kRowsPerGroup + i;
        if constexpr (SPLIT) {
            if (r < p.N) {
                float *dst = p.P + (long long)kpart * p.n * p.N + r;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const int tok = 4 * v + g;
                    if (tok < p.n)
                        dst[(long long)tok * p.N] = sum[v];
                }
            }
        } else if (r < p.N) {
            long long off;
            if (r >= p.start2)
                off = p.off2 + (r - p.start2);
            else if (r >= p.start1)
                off = p.off1 + (r - p.start1);
            else
                off = p.off0 + r;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int tok = 4 * v + g;
                if (tok < p.n)
                    p.Y[(long long)tok * p.ldy + off] = f32_to_bf16_bits(p.gscale * sum[v]);
            }
        }
    };

    // Add chunk c's partial of the row group in `slot` to this wave's LDS slot.
    auto park = [&](int slot, int c, const f32x4 acc) {
        if (c == 0) {
            part[slot][wave][lane] = acc;
        } else {
            f32x4 q = part[slot][wave][lane];
#pragma unroll
            for (int v = 0; v < NV; ++v)
                q[v] = q[v] + acc[v];
            part[slot][wave][lane] = q;
        }
    };

    // Row groups in batches of up to kSlots (one batch at the decode shapes).
    auto batch_end = [&](int b0, int b1) {
        __syncthreads();
        for (int sl = wave; sl < b1 - b0; sl += W)
            reduce_store(b0 + sl, sl);
        if (b1 < rg1)
            __syncthreads();
    };
    if constexpr (CHUNKED) {
        // Work items (batch of up to kSlots row groups, K chunk c, row group)
        // in order, one row-group call site: every row group refills the ring
        // with the next item's tiles -- the next row group of this pass, else
        // the first row group of the next pass (next chunk, else the next
        // batch's first chunk) -- so only the first pass starts on an empty
        // ring; after the last item the refill offsets lie past the buffer
        // resources (loads that read nothing) and are drained at the end.
        int b0 = rg0, b1 = min(rg0 + kSlots, rg1), c = 0, rg = rg0;
        tw = EXACT ? MT : tiles_in(tw0);
        issue_x();
        issue_ring(0);
        stage_x(std::false_type{});
        while (true) {
            int nb0 = b0, nb1 = b1, nc = c, nrg = rg + 1;
            if (nrg == b1) {
                nrg = b0;
                nc = c + 1;
                if (nc == p.kc) {
                    nc = 0;
                    nb0 = b1;
                    nb1 = min(b1 + kSlots, rg1);
                    nrg = nb0;
                }
            }
            const bool more = nb0 < rg1;
            const int nw0 = first_tile(pt0 + nc * W * MT);
            const int nwn = more ? (EXACT ? MT : tiles_in(nw0)) : 0;
            park(rg - b0, c, rowgroup(std::true_type{}, rg, more ? nrg - rg0 : rg1 - rg0, nw0, nwn));
            if (rg == b1 - 1 && c == p.kc - 1)
                batch_end(b0, b1);
            if (!more)
                break;
            const bool new_pass = nc != c || nb0 != b0;
            b0 = nb0;
            b1 = nb1;
            c = nc;
            rg = nrg;
            if (new_pass) {
                tw0 = nw0;
                tw = nwn;
                issue_x();
                stage_x(std::true_type{});
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
        // One K chunk: X is loaded and staged once for the whole launch, and
        // the ring runs on across batches (each slot refilled with the next
        // row group whatever batch it belongs to).
        tw = EXACT ? MT : tiles_in(tw0);
        issue_x();
        issue_ring(0);
        stage_x(std::false_type{});
        auto finish = [&](int rg, const f32x4 acc) {
            const int slot = (rg - rg0) % kSlots;
            park(slot, 0, acc);
            if (slot == kSlots - 1 || rg == rg1 - 1)
                batch_end(rg - slot, rg + 1);
        };
        for (int rg = rg0; rg < rg1 - 1; ++rg)
            finish(rg, rowgroup(std::true_type{}, rg, rg - rg0 + 1, tw0, tw));
        finish(rg1 - 1, rowgroup(std::false_type{}, rg1 - 1, 0, 0, 0));
    }
}

// K-split epilogue: Y[t][r] = bf16_RNE(gscale * (((P[0] + P[1]) + P[2]) + ...)),
// the K parts added in part order, so a token's result depends only on
// (N, K, ks), never on n.  Grid (ceil(N / 256), n): one thread per output,
// written at its projection's offset as in the single-launch epilogue.  The
// parts are loaded kReduceBatch at a time, all of a batch in flight together
// (a dependent load per part would pay one memory latency per part).
constexpr int kReduceBatch = 8;

__global__ __launch_bounds__(256) void nvfp4_ksplit_reduce_kernel(GemvParams p, int ks)
{
    const int r = blockIdx.x * 256 + threadIdx.x;
    const int t = blockIdx.y;
    if (r >= p.N)
        return;
    const long long count = (long long)p.n * p.N;
    const float *src = p.P + (long long)t * p.N + r;
    float s = 0.f;
    for (int q0 = 0; q0 < ks; q0 += kReduceBatch) {
        float v[kReduceBatch];
#pragma unroll
        for (int j = 0; j < kReduceBatch; ++j)
            v[j] = q0 + j < ks ? __builtin_nontemporal_load(src + (q0 + j) * count) : 0.f;
#pragma unroll
        for (int j = 0; j < kReduceBatch; ++j)
            if (q0 + j < ks)
                s = (q0 + j == 0) ? v[j] : s + v[j];
    }
    long long off;
    if (r >= p.start2)
        off = p.off2 + (r - p.start2);
    else if (r >= p.start1)
        off = p.off1 + (r - p.start1);
    else
        off = p.off0 + r;
    p.Y[(long long)t * p.ldy + off] = f32_to_bf16_bits(p.gscale * s);
}

// ---- prefill: token-tiled GEMM for n beyond one decode tile ----------------
//
// The step after the decode path as n grows (the pages' W4A16 tile GEMM
// family for prefill, sized by a measured occupancy rule): Y = X . dequant(W)^T
// for any number of tokens.  Here each wave dequantises its weight tile once
// per token tile, exactly, into bf16 (an E2M1 code times an E4M3 scale has at
// most 6 significant bits), so the block scale costs nothing per token and one
// v_mfma_f32_16x16x32_bf16 covers two 16-element blocks, with the fp32 sum
// carried in the accumulator across all of K.  The packed device layout is
// the decode path's: dword j of a lane's 16 code bytes holds its 4 + 4 codes
// of blocks 2j and 2j+1, which is exactly the B operand of one such MFMA when
// the lane's A operand holds X at the same K positions (a fixed permutation of
// K inside each pair of blocks, applied to X as it is staged into LDS).
struct GemmParams {
    const u32x4 *codes;    // packed codes, [RG][T][64 lanes] x 16 B
    const u32x2 *scales;   // packed scales, [RG][T][16 rows] x 8 B
    const uint16_t *X;     // bf16 [n][K]
    uint16_t *Y;           // bf16 [n][N]
    float gscale;
    int n, N, K, T, RG;
};


constexpr int kXRow = kTileK * 2 + 32;        // LDS bytes of one token's 128-column X slice, padded
                                              // (measured: half the bank conflicts of +16)

// A wave-uniform value the compiler cannot prove uniform, moved to SGPRs.
__device__ __forceinline__ u32x4 uniform(u32x4 v)
{
    return u32x4{(u32)__builtin_amdgcn_readfirstlane((int)v[0]), (u32)__builtin_amdgcn_readfirstlane((int)v[1]),
                 (u32)__builtin_amdgcn_readfirstlane((int)v[2]), (u32)__builtin_amdgcn_readfirstlane((int)v[3])};
}

__device__ __forceinline__ u32x2 buffer_load_b64_nt(u32x4 rsrc, unsigned off)
{
    u32x2 v;
    asm volatile("buffer_load_dwordx2 %0, %1, %2, 0 offen nt" : "=v"(v) : "v"(off), "s"(rsrc));
    return v;
}

// Exact bf16 of the 8 weights of one lane for blocks 2j and 2j+1: codes in
// dword `w` (bytes 0, 1: block 2j; bytes 2, 3: block 2j+1; low nibble first),
// E4M3 scales of the two blocks in bytes 2H, 2H+1 of `sw`.
template <bool H>
__device__ __forceinline__ u32x4 dequant_pair(u32 w, u32 sw)
{
    const auto s2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)sw, H);
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    const bf16x2 o0 = {(__bf16)(a[0] * s2[0]), (__bf16)(a[1] * s2[0])};
    const bf16x2 o1 = {(__bf16)(b[0] * s2[0]), (__bf16)(b[1] * s2[0])};
    const bf16x2 o2 = {(__bf16)(c[0] * s2[1]), (__bf16)(c[1] * s2[1])};
    const bf16x2 o3 = {(__bf16)(d[0] * s2[1]), (__bf16)(d[1] * s2[1])};
    return u32x4{__builtin_bit_cast(u32, o0), __builtin_bit_cast(u32, o1), __builtin_bit_cast(u32, o2),
                 __builtin_bit_cast(u32, o3)};
}

// Steps of K whose loads are in flight ahead of the one computing: X and
// weights share one distance (loads complete in issue order).  Smaller token
// tiles compute less per step, so they prefetch deeper.
template <int BMB>
constexpr int gemm_prefetch()
{
    return BMB == 2 ? 8 : (BMB == 4 ? 6 : 3);
}

// One workgroup: GW waves x RGW row groups (16*GW*RGW weight rows) times a tile of
// BM = 16*BMB tokens.  Per 128-column K step the workgroup stages the token
// tile's X slice in LDS (double-buffered), each wave converts its RGW code
// tiles to bf16 operands and runs 4 * RGW * BMB MFMAs.  The loads of step
// s + P are issued when step s has computed, into the register slot step s
// used (a ring of P steps; steps past the end of K load zeros without memory
// traffic, so every step issues the same loads and every wait count is a
// constant).  Each output's sum runs over K in the same order whatever n, the
// tile shape or the token's place in its tile.
template <int RGW, int BMB, int GW, int TS>
__global__ __launch_bounds__(GW * 64) void nvfp4_gemm_kernel(GemmParams p)
{
    constexpr int BM = BMB * 16;
    constexpr int WB = BMB / TS;   // token blocks per wave: TS waves share a row group's token tile
    static_assert(BMB % TS == 0 && GW % TS == 0, "token split");
    constexpr int P = gemm_prefetch<BMB>();
    constexpr int L = 4 * BMB / GW + 2 * RGW;   // loads per step and thread
    static_assert((P - 1) * L <= 63, "vmcnt is a 6-bit field");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: buffer resources in SGPRs
    const int i = lane & 15, g = lane >> 4;
    constexpr int XL = 4 * BMB / GW;   // X chunks per thread and step
    const int wtb0 = (wave % TS) * WB;                              // first token block of this wave
    const int rgw0 = (blockIdx.x * (GW / TS) + wave / TS) * RGW;   // first row group of this wave
    const int tok0 = blockIdx.y * BM;
    const int ntok = min(BM, p.n - tok0);
    const int nrg = max(0, min(RGW, p.RG - rgw0));
    const int rgb = min(rgw0, p.RG);
    // Loads past these ranges (row groups beyond RG, tokens beyond n, K
    // columns beyond K) read zeros without touching memory.
    const u32x4 crsrc = uniform(buffer_rsrc(p.codes + (size_t)rgb * p.T * 64, (unsigned)(nrg * p.T) * 1024u));
    const u32x4 srsrc = uniform(buffer_rsrc(reinterpret_cast<const char *>(p.scales) + (size_t)rgb * p.T * 128,
                                            (unsigned)(nrg * p.T) * 128u));
    const u32x4 xrsrc = uniform(buffer_rsrc(p.X + (size_t)tok0 * p.K, (unsigned)(ntok * p.K * 2)));

    // X staging: thread tid moves 16-byte chunk c = tid % 16 (columns
    // 8c .. 8c+7 of the step) of token rows tid/16 + 16u.  Columns 4g' .. 4g'+3
    // of block b go to the 16-byte A fragment of lane group g' for block pair
    // b/2, at byte 8*(b%2) of it.
    __shared__ __align__(16) char xs[2][BM * kXRow];
    const int c = tid & 15;
    const int xrow0 = tid >> 4;
    const int wofs = 64 * (c >> 2) + 32 * (c & 1) + 8 * ((c >> 1) & 1);
    u32x4 xg[P][XL];
    u32x4 cw[P][RGW];
    u32x2 sw[P][RGW];

    auto issue = [&](auto slot_c, int s) {
        constexpr int q = decltype(slot_c)::value;
        const bool live = s < p.T;
#pragma unroll
        for (int u = 0; u < XL; ++u) {
            const int row = xrow0 + 4 * GW * u;
            const int k = s * kTileK + 8 * c;
            xg[q][u] = buffer_load_b128(xrsrc, live && row < ntok && k < p.K ? (unsigned)(row * p.K + k) * 2u
                                                                           : kOutOfRange);
        }
#pragma unroll
        for (int r = 0; r < RGW; ++r) {
            cw[q][r] = buffer_load_b128_nt(crsrc, live ? (unsigned)(((r * p.T + s) * 64 + lane) * 16) : kOutOfRange);
            sw[q][r] = buffer_load_b64_nt(srsrc, live ? (unsigned)(((r * p.T + s) * 16 + i) * 8) : kOutOfRange);
        }
    };
    // Wait until the loads of slot q are in (the P - 1 newer steps' loads may
    // still be in flight; with DRAIN, wait for every load), then move its X
    // into LDS buffer `buf`.
    auto land = [&](auto slot_c, int buf, auto drain_c) {
        constexpr int q = decltype(slot_c)::value;
        if constexpr (decltype(drain_c)::value)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((P - 1) * L) : "memory");
#pragma unroll
        for (int u = 0; u < XL; ++u)
            asm volatile("" : "+v"(xg[q][u]));
#pragma unroll
        for (int r = 0; r < RGW; ++r)
            asm volatile("" : "+v"(cw[q][r]), "+v"(sw[q][r]));
#pragma unroll
        for (int u = 0; u < XL; ++u) {
            char *dst = xs[buf] + (xrow0 + 4 * GW * u) * kXRow + wofs;
            *reinterpret_cast<u32x2 *>(dst) = u32x2{xg[q][u][0], xg[q][u][1]};
            *reinterpret_cast<u32x2 *>(dst + 16) = u32x2{xg[q][u][2], xg[q][u][3]};
        }
    };

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[RGW][WB];
#pragma unroll
    for (int r = 0; r < RGW; ++r)
#pragma unroll
        for (int tb = 0; tb < WB; ++tb)
            acc[r][tb] = zero;

    // One K step from LDS buffer `buf` and weight slot q, software-pipelined
    // over its four 32-column substeps: the A fragments and the dequantised B
    // operands of substep j+1 are produced while substep j's MFMAs run.
    auto compute_pipe = [&](auto slot_c, int buf) {
        constexpr int q = decltype(slot_c)::value;
        const char *xb = xs[buf] + (wtb0 * 16 + i) * kXRow + 16 * g;
        bf16x8 a[2][WB], b[2][RGW];
#pragma unroll
        for (int tb = 0; tb < WB; ++tb)
            a[0][tb] = *reinterpret_cast<const bf16x8 *>(xb + tb * 16 * kXRow);
#pragma unroll
        for (int r = 0; r < RGW; ++r)
            b[0][r] = __builtin_bit_cast(bf16x8, dequant_pair<false>(cw[q][r][0], sw[q][r][0]));
        static_for<4>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr int cur = j & 1, nxt = cur ^ 1;
            if constexpr (j < 3) {
#pragma unroll
                for (int tb = 0; tb < WB; ++tb)
                    a[nxt][tb] = *reinterpret_cast<const bf16x8 *>(xb + tb * 16 * kXRow + 64 * (j + 1));
#pragma unroll
                for (int r = 0; r < RGW; ++r)
                    b[nxt][r] = __builtin_bit_cast(bf16x8, dequant_pair<((j + 1) & 1) != 0>(cw[q][r][j + 1], sw[q][r][(j + 1) >> 1]));
            }
#pragma unroll
            for (int tb = 0; tb < WB; ++tb)
#pragma unroll
                for (int r = 0; r < RGW; ++r)
                    acc[r][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[cur][tb], b[cur][r], acc[r][tb], 0, 0, 0);
            
        });
    };

    static_assert(RGW == 1 || GW == 8, "row tiles: 1 row group per wave, or 8 waves x 2");
    auto compute = [&](auto slot_c, int buf) { compute_pipe(slot_c, buf); };

    // K step s: compute from slot s % P, refill that slot with step s + P
    // (loads past the last step read nothing), land slot (s + 1) % P.  Whole
    // rounds of P steps run unguarded; the last T % P steps follow with
    // nested guards, no refills, and waits for every load in flight.  So the
    // code has no path on which a wait's count would not hold (no skipped
    // step is followed by a taken one, the loop's back edge follows a whole
    // round), which the build's static check of the wait counts relies on.
    auto step = [&](auto qc, int s) {
        constexpr int q = decltype(qc)::value;
        compute(qc, s & 1);
        issue(qc, s + P);
        land(std::integral_constant<int, (q + 1) % P>{}, (s + 1) & 1, std::false_type{});
        __syncthreads();
    };
    static_for<P>([&](auto qc) { issue(qc, decltype(qc)::value); });
    land(std::integral_constant<int, 0>{}, 0, std::false_type{});
    __syncthreads();
    int s0 = 0;
    for (; s0 + P <= p.T; s0 += P)
        static_for<P>([&](auto qc) { step(qc, s0 + decltype(qc)::value); });
    auto tail = [&](auto self, auto qc) {
        constexpr int q = decltype(qc)::value;
        if constexpr (q < P - 1) {
            if (s0 + q < p.T) {
                compute(qc, (s0 + q) & 1);
                land(std::integral_constant<int, q + 1>{}, (s0 + q + 1) & 1, std::true_type{});
                __syncthreads();
                self(self, std::integral_constant<int, q + 1>{});
            }
        }
    };
    tail(tail, std::integral_constant<int, 0>{});
    // Drain the last round's loads (they read nothing).  The slot registers
    // are used after the wait, so the compiler cannot hand them to other
    // values while those loads may still write them.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int q = 0; q < P; ++q) {
#pragma unroll
        for (int u = 0; u < XL; ++u)
            asm volatile("" : "+v"(xg[q][u]));
#pragma unroll
        for (int r = 0; r < RGW; ++r)
            asm volatile("" : "+v"(cw[q][r]), "+v"(sw[q][r]));
    }

    // Component v of lane (g, i) of acc[r][tb]: token tok0 + 16*(wtb0 + tb) +
    // 4*g + v, weight row 16*(rgw0 + r) + i.
#pragma unroll
    for (int r = 0; r < RGW; ++r) {
        const int row = (rgw0 + r) * kRowsPerGroup + i;
        if (row >= p.N)
            continue;
#pragma unroll
        for (int tb = 0; tb < WB; ++tb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = 16 * (wtb0 + tb) + 4 * g + v;
                if (t < ntok)
                    p.Y[(size_t)(tok0 + t) * p.N + row] = f32_to_bf16_bits(p.gscale * acc[r][tb][v]);
            }
    }
}

// ---- pack: canonical -> tiled device layout --------------------------------

// One thread per 16-byte lane chunk of a tile.
__global__ void nvfp4_pack_codes_kernel(const uint8_t *codes, int N, int K, int T, long long chunks,
                                        u32x4 *out)
{
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= chunks)
        return;
    const int l = (int)(idx & 63);
    const long long tile_lin = idx >> 6;
    const int tile = (int)(tile_lin % T);
    const long long rg = tile_lin / T;
    const int i = l & 15, g = l >> 4;
    const long long row = rg * kRowsPerGroup + i;
    u32 w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        // packed byte q holds K = tile*128 + 16*(q/2) + 4*g + 2*(q%2) (+0, +1)
        const int k = tile * kTileK + 16 * (q >> 1) + 4 * g + 2 * (q & 1);
        u32 byte = 0;
        if (row < N && k < K)
            byte = codes[row * (long long)(K / 2) + k / 2];
        w[q >> 2] |= byte << (8 * (q & 3));
    }
    out[idx] = u32x4{w[0], w[1], w[2], w[3]};
}

// One thread per (row group, tile, row): the 8 scale bytes of that row's tile.
__global__ void nvfp4_pack_scales_kernel(const uint8_t *scales, int N, int K, int T, long long items,
                                         u32x2 *out)
{
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= items)
        return;
    const int i = (int)(idx & 15);
    const long long tile_lin = idx >> 4;
    const int tile = (int)(tile_lin % T);
    const long long rg = tile_lin / T;
    const long long row = rg * kRowsPerGroup + i;
    const int nb = K / 16;
    u32 w[2] = {0u, 0u};
#pragma unroll
    for (int b = 0; b < kBlocksPerTile; ++b) {
        const int blk = tile * kBlocksPerTile + b;
        u32 byte = 0;
        if (row < N && blk < nb)
            byte = scales[row * (long long)nb + blk];
        w[b >> 2] |= byte << (8 * (b & 3));
    }
    out[idx] = u32x2{w[0], w[1]};
}

// ---- quantise (input recipe) --------------------------------------------------

__global__ void nvfp4_amax_init_kernel(float *ts)
{
    ts[1] = 0.0f;
}

__global__ void nvfp4_amax_kernel(const float4 *W, long long n4, float *ts)
{
    float m = 0.0f;
    for (long long j = (long long)blockIdx.x * blockDim.x + threadIdx.x; j < n4;
         j += (long long)gridDim.x * blockDim.x) {
        const float4 v = W[j];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    for (int o = 32; o > 0; o >>= 1)
        m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0)   // non-negative floats order like their bit patterns
        atomicMax(reinterpret_cast<unsigned int *>(ts + 1), __float_as_uint(m));
}

// E4M3FN byte (0x00..0x7E) -> exact value, from its fields.
__device__ __forceinline__ double e4m3_value(int s)
{
    const int e = (s >> 3) & 15, m = s & 7;
    return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
}

// Nearest E4M3FN byte for v >= 0, ties to even, saturating at 448.
__device__ __forceinline__ int e4m3_rne(double v)
{
    if (!(v < 448.0))
        return 0x7E;
    if (v < 0.015625)   // below 2^-6: subnormal grid of step 2^-9
        return (int)rint(v * 512.0);
    int e;
    const double f = frexp(v, &e);   // v = f * 2^e, f in [0.5, 1)
    int E = e + 6;
    int M = (int)rint((f * 2.0 - 1.0) * 8.0);
    if (M == 8) {
        E += 1;
        M = 0;
    }
    const int byte = (E << 3) | M;
    return byte > 0x7E ? 0x7E : byte;
}

// E2M1 magnitude index of a / d (a >= 0, d > 0), nearest with ties to the even
// index, by exact comparisons against the midpoints of the grid.
__device__ __forceinline__ int e2m1_rne(double a, double d)
{
    int idx = 0;
    idx += a > 0.25 * d;
    idx += a >= 0.75 * d;
    idx += a > 1.25 * d;
    idx += a >= 1.75 * d;
    idx += a > 2.5 * d;
    idx += a >= 3.5 * d;
    idx += a > 5.0 * d;
    return idx;
}

// One thread per 16-element K-block (flat index row*(K/16) + block).
__global__ void nvfp4_quantize_kernel(const float4 *W, long long nblocks, uint2 *codes,
                                      uint8_t *scales, float *ts)
{
    const long long blk = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const float amax = ts[1];
    const float gs = (float)((double)amax / 2688.0);
    if (blk == 0)
        ts[0] = gs;
    if (blk >= nblocks)
        return;
    float w[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float4 v = W[blk * 4 + j];
        w[4 * j] = v.x;
        w[4 * j + 1] = v.y;
        w[4 * j + 2] = v.z;
        w[4 * j + 3] = v.w;
    }
    double am = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        am = fmax(am, fabs((double)w[j]));
    const int s = gs > 0.0f ? e4m3_rne(am / (6.0 * (double)gs)) : 0;
    const double d = e4m3_value(s) * (double)gs;
    u32 c[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int mag = d > 0.0 ? e2m1_rne(fabs((double)w[j]), d) : 0;
        const u32 code = (u32)mag | (signbit(w[j]) ? 8u : 0u);
        c[j >> 3] |= code << (4 * (j & 7));
    }
    codes[blk] = make_uint2(c[0], c[1]);
    scales[blk] = (uint8_t)s;
}

// Fused recipe quantiser writing the packed device layout directly (the
// pages' runtime requantisation with its "emit the transposed copy during
// requant" fix, on this layout): one thread per (row group, tile, row) makes
// the tile's 8 block scales and 128 codes of that row with exactly the
// decisions of nvfp4_quantize_kernel and stores them where nvfp4_pack would:
// lane chunk g of the tile holds the row's columns 4g .. 4g+3 of every block
// (byte 2b + e/2 of the chunk, low nibble first), and the row's 8 scale bytes
// follow in block order.  Rows past N and blocks past K/16 are zero.
template <typename T>
__device__ __forceinline__ float load_w(const T *W, long long idx);
template <>
__device__ __forceinline__ float load_w<float>(const float *W, long long idx)
{
    return W[idx];
}
template <>
__device__ __forceinline__ float load_w<uint16_t>(const uint16_t *W, long long idx)
{
    return __uint_as_float((u32)W[idx] << 16);   // bf16 -> fp32, exact
}

template <typename T>
__global__ void nvfp4_quantize_packed_kernel(const T *W, int N, int K, int T_tiles, long long items,
                                             const float *ts, u32x4 *codes, u32x2 *scales)
{
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= items)
        return;
    const int i = (int)(idx & 15);
    const long long tile_lin = idx >> 4;
    const int tile = (int)(tile_lin % T_tiles);
    const long long rg = tile_lin / T_tiles;
    const long long row = rg * kRowsPerGroup + i;
    const int nb = K / 16;
    const float gs = (float)((double)ts[1] / 2688.0);
    u32 chunk[4][4] = {};
    u32 sb[2] = {0u, 0u};
#pragma unroll 1
    for (int b = 0; b < kBlocksPerTile; ++b) {
        const int blk = tile * kBlocksPerTile + b;
        if (row >= N || blk >= nb)
            continue;
        float w[16];
        const long long base = row * (long long)K + (long long)blk * 16;
#pragma unroll
        for (int e = 0; e < 16; ++e)
            w[e] = load_w<T>(W, base + e);
        double am = 0.0;
#pragma unroll
        for (int e = 0; e < 16; ++e)
            am = fmax(am, fabs((double)w[e]));
        const int sc = gs > 0.0f ? e4m3_rne(am / (6.0 * (double)gs)) : 0;
        const double d = e4m3_value(sc) * (double)gs;
        sb[b >> 2] |= (u32)sc << (8 * (b & 3));
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int mag = d > 0.0 ? e2m1_rne(fabs((double)w[e]), d) : 0;
            const u32 code = (u32)mag | (signbit(w[e]) ? 8u : 0u);
            const int g = e >> 2;
            const int byte = 2 * (b & 1) + ((e & 3) >> 1);
            chunk[g][b >> 1] |= code << (8 * byte + 4 * (e & 1));
        }
    }
    const long long tbase = (rg * T_tiles + tile) * 64;
#pragma unroll
    for (int g = 0; g < 4; ++g)
        codes[tbase + g * 16 + i] = u32x4{chunk[g][0], chunk[g][1], chunk[g][2], chunk[g][3]};
    scales[(rg * T_tiles + tile) * 16 + i] = u32x2{sb[0], sb[1]};
}

template <typename T>
__global__ void nvfp4_amax_any_kernel(const T *W, long long n, float *ts)
{
    float m = 0.0f;
    for (long long j = (long long)blockIdx.x * blockDim.x + threadIdx.x; j < n;
         j += (long long)gridDim.x * blockDim.x)
        m = fmaxf(m, fabsf(load_w<T>(W, j)));
    for (int o = 32; o > 0; o >>= 1)
        m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0)   // non-negative floats order like their bit patterns
        atomicMax(reinterpret_cast<unsigned int *>(ts + 1), __float_as_uint(m));
}

__global__ void nvfp4_gscale_kernel(float *ts)
{
    ts[0] = (float)((double)ts[1] / 2688.0);
}

// ---- host side ---------------------------------------------------------------

typedef void (*GemvKernel)(GemvParams);

template <int MT, int NV>
GemvKernel pick_exact(bool exact, bool chunked, bool split)
{
    // Several chunks imply more than 64 tiles cut into kc = ceil(T/56)
    // chunks, so MT = ceil(T/(8*kc)) is 5, 6 or 7 for every K up to 262144
    // (T = 65 .. 2048).  A K part is never chunked.
    if constexpr (MT >= 5 && MT <= kMaxTilesChunked) {
        if (chunked && !split)
            return exact ? nvfp4_gemv_kernel<MT, NV, true, true, false>
                         : nvfp4_gemv_kernel<MT, NV, false, true, false>;
    }
    if (chunked)
        return nullptr;
    if (split)
        return exact ? nvfp4_gemv_kernel<MT, NV, true, false, true> : nvfp4_gemv_kernel<MT, NV, false, false, true>;
    return exact ? nvfp4_gemv_kernel<MT, NV, true, false, false> : nvfp4_gemv_kernel<MT, NV, false, false, false>;
}

template <int NV>
GemvKernel pick_mt(int mt, bool exact, bool chunked, bool split)
{
    switch (mt) {
    case 1: return pick_exact<1, NV>(exact, chunked, split);
    case 2: return pick_exact<2, NV>(exact, chunked, split);
    case 3: return pick_exact<3, NV>(exact, chunked, split);
    case 4: return pick_exact<4, NV>(exact, chunked, split);
    case 5: return pick_exact<5, NV>(exact, chunked, split);
    case 6: return pick_exact<6, NV>(exact, chunked, split);
    case 7: return pick_exact<7, NV>(exact, chunked, split);
    default: return pick_exact<8, NV>(exact, chunked, split);
    }
}

// Kernel for n tokens (ceil(n/4) accumulator components), MT tiles per wave,
// several K chunks (one launch) or K parts (partials for the reduction).
GemvKernel pick_kernel(int n, int mt, bool exact, bool chunked, bool split)
{
    switch ((n + 3) / 4) {
    case 1: return pick_mt<1>(mt, exact, chunked, split);
    case 2: return pick_mt<2>(mt, exact, chunked, split);
    case 3: return pick_mt<3>(mt, exact, chunked, split);
    default: return pick_mt<4>(mt, exact, chunked, split);
    }
}

struct Geometry {
    int workgroups, mt, kc;
    int ks, tp, wpp;   // K parts, tiles per part, workgroups per part
    bool exact;
};

constexpr int kMaxDevices = 64;
int g_cus[kMaxDevices];
int g_is_gfx950[kMaxDevices];   // 0 unknown, 1 yes, -1 no
std::mutex g_dev_mutex;

// Compute units and architecture of the current device, looked up once.
int current_device_info(int *cus)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return NVFP4_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (g_is_gfx950[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return NVFP4_ERR_DEVICE;
        g_is_gfx950[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        g_cus[dev] = prop.multiProcessorCount;
    }
    if (g_is_gfx950[dev] != 1)
        return NVFP4_ERR_DEVICE;
    *cus = g_cus[dev];
    return NVFP4_OK;
}

// Launch shape for an N x K weight on `cus` compute units: 8 waves per
// workgroup splitting the K tiles evenly (MT each, the last waves possibly
// short), one workgroup per compute unit per round, and as few workgroups as
// keep the number of rounds (row groups per workgroup) at its minimum, so that
// every workgroup streams the same number of row groups where N allows it.
//
// With ks > 1 K parts, K's tiles are cut into ks parts of tp tiles (the last
// possibly shorter, none empty); each (part, row group) is one unit of work
// and every part gets the same number of workgroups (wpp), each a contiguous
// row-group range of its part.
bool geometry_for(int N, int K, int cus, int ks, Geometry *geo)
{
    const int T = (int)k_tiles(K);
    const long long RG = row_groups(N);
    if (ks < 1 || ks > T)
        return false;
    geo->ks = ks;
    geo->tp = (T + ks - 1) / ks;
    if ((long long)(ks - 1) * geo->tp >= T)
        return false;   // the last part would be empty
    if (ks > 1 && geo->tp > kWaves * kMaxTilesPerWave)
        return false;   // a K part is one pass
    // One chunk up to 8 tiles per wave; beyond, chunks of at most
    // kMaxTilesChunked tiles per wave (the chunked kernels keep one more
    // set of X registers live across passes).
    const int tp = geo->tp;
    const int per_chunk = tp <= kWaves * kMaxTilesPerWave ? kWaves * kMaxTilesPerWave : kWaves * kMaxTilesChunked;
    geo->kc = (tp + per_chunk - 1) / per_chunk;
    geo->mt = (tp + kWaves * geo->kc - 1) / (kWaves * geo->kc);
    geo->exact = K % kTileK == 0 && T == ks * tp && tp == geo->kc * kWaves * geo->mt;
    const long long rounds = (ks * RG + cus - 1) / cus;
    geo->wpp = (int)((RG + rounds - 1) / rounds);
    geo->workgroups = ks * geo->wpp;
    return true;
}

// K parts for an N x K weight, from the shape alone (so a token's result
// never depends on n or on the device): one part while a part's tiles fit in
// one pass (K <= 8192); beyond, the count that minimises the critical path
// (rounds of row groups per workgroup on MI355X's 256 compute units times the
// tiles per part) with one pass per part, the fewest parts on a tie.  A
// single launch restages X once per pass and leaves compute units idle when
// N has fewer row groups than the chip has units; parts fill the chip and
// halve (or better) the X each compute unit loads.
int ksplit_for(int N, int K)
{
    const int T = (int)k_tiles(K);
    const long long RG = row_groups(N);
    if (T <= kWaves * kMaxTilesPerWave)
        return 1;
    int best = 1;
    long long best_cost = -1;
    for (int ks = 2; ks <= T && ks <= kMaxKParts; ++ks) {
        const int tp = (T + ks - 1) / ks;
        if ((long long)(ks - 1) * tp >= T || tp > kWaves * kMaxTilesPerWave)
            continue;
        const long long cost = ((ks * RG + 255) / 256) * tp;
        if (best_cost < 0 || cost < best_cost) {
            best = ks;
            best_cost = cost;
        }
    }
    return best;
}

// Fixed device memory for callers that cannot allocate (nvfp4_gemv_ws_static):
// the K-part partials live in this file-scope array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` is only the symbol's host-side
// stand-in: kernels get the device address hipGetSymbolAddress returns for
// the current device, looked up once per device and kept in g_scratch.
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void *g_scratch[kMaxDevices];

// Device address of `scratch` on the current device.
int scratch_on_current_device(void **ptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return NVFP4_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return NVFP4_ERR_DEVICE;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return NVFP4_OK;
}

bool aligned(const void *p, size_t a)
{
    return ((uintptr_t)p % a) == 0;
}

int validate_common(const uint8_t *Wq, const uint8_t *Wscale, const uint16_t *X, const uint16_t *Y,
                    int n, int N, int K)
{
    if (!Wq || !Wscale || !X || !Y)
        return NVFP4_ERR_NULL;
    if (n < 1 || n > NVFP4_MAX_TOKENS || N < 1 || K < 1)
        return NVFP4_ERR_RANGE;
    if (K % 16 != 0)
        return NVFP4_ERR_SHAPE;
    if (K > kMaxK)
        return NVFP4_ERR_SHAPE;
    if (!aligned(Wq, 16) || !aligned(Wscale, 16) || !aligned(X, 16) || !aligned(Y, 2))
        return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

// Workspace of a launch with ks K parts: fp32 partials [ks][n][N].
size_t ksplit_workspace_bytes(int ks, int n, int N)
{
    return ks > 1 ? (size_t)ks * n * N * sizeof(float) : 0;
}

// One GEMV launch (ks == 1), or the K-part launch and its reduction (ks > 1,
// partials in `ws`, which the caller has checked to be large enough).
int launch_gemv(const GemvParams &p, hipStream_t stream, int ks = 1, void *ws = nullptr)
{
    int cus = 0;
    int st = current_device_info(&cus);
    if (st != NVFP4_OK)
        return st;
    Geometry geo;
    if (!geometry_for(p.N, p.K, cus, ks, &geo))
        return NVFP4_ERR_SHAPE;
    GemvKernel k = pick_kernel(p.n, geo.mt, geo.exact, geo.kc > 1, ks > 1);
    if (!k)
        return NVFP4_ERR_SHAPE;
    GemvParams q = p;
    q.rg_base = p.RG / geo.wpp;
    q.rg_rem = p.RG % geo.wpp;
    q.kc = geo.kc;
    q.tp = geo.tp;
    q.wpp = geo.wpp;
    q.P = ks > 1 ? static_cast<float *>(ws) : nullptr;
    if ((long long)(q.rg_base + 1) * p.T * 1024 > 0x7FFFFFFFLL)
        return NVFP4_ERR_SHAPE;   // a workgroup's codes must stay within a 32-bit buffer offset
    hipLaunchKernelGGL(k, dim3(geo.workgroups), dim3(kWaves * 64), 0, stream, q);
    if (hipGetLastError() != hipSuccess)
        return NVFP4_ERR_LAUNCH;
    if (ks > 1) {
        hipLaunchKernelGGL(nvfp4_ksplit_reduce_kernel, dim3((unsigned)((p.N + 255) / 256), (unsigned)p.n),
                           dim3(256), 0, stream, q, ks);
        if (hipGetLastError() != hipSuccess)
            return NVFP4_ERR_LAUNCH;
    }
    return NVFP4_OK;
}

typedef void (*GemmKernel)(GemmParams);

struct GemmGeometry {
    int rgw, gw, bmb;      // row groups per wave, waves per workgroup, 16-token blocks per token tile
    int ts;                // waves sharing one row group's token tile (token split)
    int grid_x, grid_y;    // row tiles, token tiles
};

// Tile shape of the prefill GEMM for n tokens of an N x K weight on `cus`
// compute units.  The token tile is the smallest of 32 / 64 / 128 tokens that
// holds n (capped at 128; for n > 128 see the 256-row choice below).  The row tile is 256 rows (8 waves x 2 row groups,
// one workgroup per compute unit), which shares each X tile among the most
// rows and measured the fastest per row, once its grid gives at least half
// the compute units a workgroup; below that, 64 rows (4 waves x 1 row group,
// two workgroups per compute unit), whose four times as many workgroups keep
// the longest one's work shorter.  A 128-row tile (4 x 2) never won: above the
// threshold it puts two workgroups on some compute unit, as long a critical
// path at a lower rate per row (fused QKV, n = 320 .. 512: 90 .. 97 us against
// 74 .. 82 us for 256 rows), below it the 64-row tile was as fast or faster.
// Beyond one 128-token tile (n > 128) the 256-row tile may also take 96- or
// 64-token tiles: more weight reads and a lower rate per token, but more
// workgroups in as few rounds.  Fused QKV: 96-token tiles at n = 288 .. 384
// take 65 .. 68 us against 75 .. 76 us, at n = 640 / 768 132 / 138 against
// 145 / 148 us; 64-token tiles at n = 160 .. 256 50 .. 54 us against 61 .. 63
// us for the 64-row tile.  With one 128-token tile (n <= 128) the token-split
// 64-row tile below is faster (n = 96 .. 128: 38.7 / 38.8 us against 38.9 /
// 39.7 us with 64-token tiles).
// The 64-row tile with a single 128-token tile runs 8 waves, two per row group,
// each on 64 of the tokens: twice the waves of the 4-wave form where the grid
// has one token tile (n = 96 .. 128 on the fused QKV: 36 us against 41 us).
// With more token tiles its registers (one such workgroup per compute unit)
// cost more than the waves gain, and with 32- or 64-token tiles it gains
// nothing.  Each output's sum over K runs in one wave in the same order
// whatever the tile, so every choice gives the same bits.
void gemm_geometry_for(int n, int N, int cus, GemmGeometry *geo)
{
    geo->bmb = n <= 32 ? 2 : (n <= 64 ? 4 : 8);
    const long long RG = row_groups(N);
    geo->grid_y = (n + 16 * geo->bmb - 1) / (16 * geo->bmb);
    const long long tiles256 = (RG + 15) / 16;
    bool wide = tiles256 * geo->grid_y * 2 >= cus;
    if (n > 128) {
        // Among the token tiles whose 256-row grid reaches half the compute
        // units, the least (rounds x tokens per tile / measured rate per token
        // of that tile: 1.0, 0.84, 0.70 for 128, 96, 64), 128 first on ties.
        static const int bms[3] = {8, 6, 4}, rate[3] = {100, 84, 70};
        long long best = -1;
        for (int j = 0; j < 3; ++j) {
            const long long gy = (n + 16 * bms[j] - 1) / (16 * bms[j]);
            const long long wgs = tiles256 * gy;
            if (wgs * 2 < cus)
                continue;
            const long long cost = (wgs + cus - 1) / cus * 16 * bms[j] * 10000 / rate[j];
            if (best < 0 || cost < best) {
                best = cost;
                geo->bmb = bms[j];
                geo->grid_y = (int)gy;
                wide = true;
            }
        }
    }
    geo->rgw = wide ? 2 : 1;
    geo->ts = !wide && geo->bmb == 8 && geo->grid_y == 1 ? 2 : 1;
    geo->gw = wide || geo->ts == 2 ? 8 : 4;
    const int rows_rg = geo->rgw * geo->gw / geo->ts;   // row groups per workgroup
    geo->grid_x = (int)((RG + rows_rg - 1) / rows_rg);
}

template <int RGW, int GW>
GemmKernel pick_gemm_bmb(int bmb)
{
    switch (bmb) {
    case 2: return nvfp4_gemm_kernel<RGW, 2, GW, 1>;
    case 4: return nvfp4_gemm_kernel<RGW, 4, GW, 1>;
    case 6:
        if constexpr (GW == 8)
            return nvfp4_gemm_kernel<RGW, 6, GW, 1>;   // 96-token tiles: 256-row tile only
        return nullptr;
    default: return nvfp4_gemm_kernel<RGW, 8, GW, 1>;
    }
}

GemmKernel pick_gemm(const GemmGeometry &geo)
{
    if (geo.rgw == 2)
        return pick_gemm_bmb<2, 8>(geo.bmb);
    if (geo.ts == 2)
        return nvfp4_gemm_kernel<1, 8, 8, 2>;
    return pick_gemm_bmb<1, 4>(geo.bmb);
}

int validate_gemm(const uint8_t *Wq, const uint8_t *Wscale, const uint16_t *X, const uint16_t *Y,
                  int n, int N, int K)
{
    if (!Wq || !Wscale || !X || !Y)
        return NVFP4_ERR_NULL;
    if (n < 1 || n > NVFP4_MAX_GEMM_TOKENS || N < 1 || K < 1)
        return NVFP4_ERR_RANGE;
    if (K % 16 != 0 || K > kMaxK)
        return NVFP4_ERR_SHAPE;
    if (!aligned(Wq, 16) || !aligned(Wscale, 16) || !aligned(X, 16) || !aligned(Y, 2))
        return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

GemvParams make_params(const uint8_t *Wq, const uint8_t *Wscale, float gscale, const uint16_t *X,
                       uint16_t *Y, int n, int N, int K)
{
    GemvParams p;
    p.codes = reinterpret_cast<const u32x4 *>(Wq);
    p.scales = reinterpret_cast<const u32x2 *>(Wscale);
    p.X = X;
    p.Y = Y;
    p.gscale = gscale;
    p.n = n;
    p.N = N;
    p.K = K;
    p.T = (int)k_tiles(K);
    p.RG = (int)row_groups(N);
    p.start1 = N;
    p.start2 = N;
    p.off0 = p.off1 = p.off2 = 0;
    p.ldy = N;
    p.tp = p.T;
    p.wpp = 1;
    p.P = nullptr;
    return p;
}

int check_schedule(int n, const uint8_t *tile_widths, int ntiles)
{
    if (!tile_widths || ntiles < 1 || ntiles > n)
        return NVFP4_ERR_SCHEDULE;
    int sum = 0;
    for (int j = 0; j < ntiles; ++j) {
        if (tile_widths[j] < 1 || tile_widths[j] > NVFP4_MAX_TOKENS)
            return NVFP4_ERR_SCHEDULE;
        sum += tile_widths[j];
    }
    return sum == n ? NVFP4_OK : NVFP4_ERR_SCHEDULE;
}

// Arguments of a K-part call (nvfp4_gemv_ws, nvfp4_gemv_ws_static); *ks = 0
// becomes the part count for the shape.
int validate_kparts(const uint8_t *Wq, const uint8_t *Wscale, const uint16_t *X, const uint16_t *Y, int n,
                    int N, int K, int *ks)
{
    int st = validate_common(Wq, Wscale, X, Y, n, N, K);
    if (st != NVFP4_OK)
        return st;
    if (*ks < 0 || *ks > kMaxKParts)
        return NVFP4_ERR_RANGE;
    if (*ks == 0)
        *ks = ksplit_for(N, K);
    const int T = (int)k_tiles(K);
    const int tp = (T + *ks - 1) / *ks;
    if (*ks > T || (long long)(*ks - 1) * tp >= T)
        return NVFP4_ERR_SHAPE;   // some K part would be empty
    if (*ks > 1 && tp > kWaves * kMaxTilesPerWave)
        return NVFP4_ERR_SHAPE;   // a K part longer than one pass (8192 columns)
    return NVFP4_OK;
}

}  // namespace

extern "C" {

size_t nvfp4_packed_codes_bytes(int N, int K)
{
    if (N <= 0 || K <= 0 || K % 16 != 0)
        return 0;
    const size_t RG = (size_t)row_groups(N);
    const size_t T = (size_t)k_tiles(K);
    return RG * T * 1024;
}

size_t nvfp4_packed_scales_bytes(int N, int K)
{
    if (N <= 0 || K <= 0 || K % 16 != 0)
        return 0;
    const size_t RG = (size_t)row_groups(N);
    const size_t T = (size_t)k_tiles(K);
    return RG * T * 128;
}

int nvfp4_quantize(const float *W, int N, int K, uint8_t *codes, uint8_t *scales,
                   float *tensor_scale, void *stream)
{
    if (!W || !codes || !scales || !tensor_scale)
        return NVFP4_ERR_NULL;
    if (N < 1 || K < 1)
        return NVFP4_ERR_RANGE;
    if (K % 16 != 0)
        return NVFP4_ERR_SHAPE;
    if (!aligned(W, 16) || !aligned(codes, 8) || !aligned(tensor_scale, 4))
        return NVFP4_ERR_ALIGN;
    int cus = 0;
    int st = current_device_info(&cus);
    if (st != NVFP4_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    const long long nblocks = (long long)N * (K / 16);
    hipLaunchKernelGGL(nvfp4_amax_init_kernel, dim3(1), dim3(1), 0, s, tensor_scale);
    const long long n4 = nblocks * 4;
    long long grid = (n4 + 255) / 256;
    if (grid > (long long)cus * 8)
        grid = (long long)cus * 8;
    hipLaunchKernelGGL(nvfp4_amax_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                       reinterpret_cast<const float4 *>(W), n4, tensor_scale);
    hipLaunchKernelGGL(nvfp4_quantize_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const float4 *>(W), nblocks, reinterpret_cast<uint2 *>(codes),
                       scales, tensor_scale);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

int nvfp4_quantize_packed(const void *W, int dtype, int N, int K, uint8_t *codes_packed,
                          uint8_t *scales_packed, float *tensor_scale, void *stream)
{
    if (!W || !codes_packed || !scales_packed || !tensor_scale)
        return NVFP4_ERR_NULL;
    if (N < 1 || K < 1 || (dtype != NVFP4_DTYPE_F32 && dtype != NVFP4_DTYPE_BF16))
        return NVFP4_ERR_RANGE;
    if (K % 16 != 0)
        return NVFP4_ERR_SHAPE;
    if (!aligned(W, 16) || !aligned(codes_packed, 16) || !aligned(scales_packed, 16) ||
        !aligned(tensor_scale, 4))
        return NVFP4_ERR_ALIGN;
    int cus = 0;
    int st = current_device_info(&cus);
    if (st != NVFP4_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    const long long n = (long long)N * K;
    long long grid = (n + 255) / 256;
    if (grid > (long long)cus * 8)
        grid = (long long)cus * 8;
    const int T = (int)k_tiles(K);
    const long long RG = row_groups(N);
    const long long items = RG * T * 16;
    const unsigned qgrid = (unsigned)((items + 255) / 256);
    hipLaunchKernelGGL(nvfp4_amax_init_kernel, dim3(1), dim3(1), 0, s, tensor_scale);
    if (dtype == NVFP4_DTYPE_F32) {
        const float *w = reinterpret_cast<const float *>(W);
        hipLaunchKernelGGL(nvfp4_amax_any_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s, w, n, tensor_scale);
        hipLaunchKernelGGL(nvfp4_quantize_packed_kernel<float>, dim3(qgrid), dim3(256), 0, s, w, N, K, T, items,
                           tensor_scale, reinterpret_cast<u32x4 *>(codes_packed),
                           reinterpret_cast<u32x2 *>(scales_packed));
    } else {
        const uint16_t *w = reinterpret_cast<const uint16_t *>(W);
        hipLaunchKernelGGL(nvfp4_amax_any_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, s, w, n,
                           tensor_scale);
        hipLaunchKernelGGL(nvfp4_quantize_packed_kernel<uint16_t>, dim3(qgrid), dim3(256), 0, s, w, N, K, T,
                           items, tensor_scale, reinterpret_cast<u32x4 *>(codes_packed),
                           reinterpret_cast<u32x2 *>(scales_packed));
    }
    hipLaunchKernelGGL(nvfp4_gscale_kernel, dim3(1), dim3(1), 0, s, tensor_scale);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

int nvfp4_pack(const uint8_t *codes, const uint8_t *scales, int N, int K, uint8_t *codes_packed,
               uint8_t *scales_packed, void *stream)
{
    if (!codes || !scales || !codes_packed || !scales_packed)
        return NVFP4_ERR_NULL;
    if (N < 1 || K < 1)
        return NVFP4_ERR_RANGE;
    if (K % 16 != 0)
        return NVFP4_ERR_SHAPE;
    if (!aligned(codes_packed, 16) || !aligned(scales_packed, 16))
        return NVFP4_ERR_ALIGN;
    int cus = 0;
    int st = current_device_info(&cus);
    if (st != NVFP4_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    const int T = (int)k_tiles(K);
    const long long RG = row_groups(N);
    const long long chunks = RG * T * 64;
    const long long items = RG * T * 16;
    hipLaunchKernelGGL(nvfp4_pack_codes_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                       codes, N, K, T, chunks, reinterpret_cast<u32x4 *>(codes_packed));
    hipLaunchKernelGGL(nvfp4_pack_scales_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s,
                       scales, N, K, T, items, reinterpret_cast<u32x2 *>(scales_packed));
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

int nvfp4_gemv(const uint8_t *Wq, const uint8_t *Wscale, float gscale, const uint16_t *X, uint16_t *Y,
               int n, int N, int K, void *stream)
{
    int st = validate_common(Wq, Wscale, X, Y, n, N, K);
    if (st != NVFP4_OK)
        return st;
    return launch_gemv(make_params(Wq, Wscale, gscale, X, Y, n, N, K), (hipStream_t)stream);
}

int nvfp4_gemv_kparts(int N, int K)
{
    if (N < 1 || K < 1)
        return -NVFP4_ERR_RANGE;
    if (K % 16 != 0 || K > kMaxK)
        return -NVFP4_ERR_SHAPE;
    return ksplit_for(N, K);
}

size_t nvfp4_gemv_workspace_bytes(int n, int N, int K, int ks)
{
    if (n < 1 || n > NVFP4_MAX_TOKENS || N < 1 || K < 1 || K % 16 != 0 || K > kMaxK || ks < 0)
        return 0;
    return ksplit_workspace_bytes(ks == 0 ? ksplit_for(N, K) : ks, n, N);
}

int nvfp4_gemv_ws(const uint8_t *Wq, const uint8_t *Wscale, float gscale, const uint16_t *X, uint16_t *Y,
                  int n, int N, int K, int ks, void *workspace, size_t workspace_bytes, void *stream)
{
    int st = validate_kparts(Wq, Wscale, X, Y, n, N, K, &ks);
    if (st != NVFP4_OK)
        return st;
    if (ks > 1) {
        if (!workspace || workspace_bytes < ksplit_workspace_bytes(ks, n, N))
            return NVFP4_ERR_WORKSPACE;
        if (!aligned(workspace, 16))
            return NVFP4_ERR_ALIGN;
    }
    return launch_gemv(make_params(Wq, Wscale, gscale, X, Y, n, N, K), (hipStream_t)stream, ks, workspace);
}

int nvfp4_gemv_ws_static(const uint8_t *Wq, const uint8_t *Wscale, float gscale, const uint16_t *X,
                         uint16_t *Y, int n, int N, int K, int ks, void *stream)
{
    int st = validate_kparts(Wq, Wscale, X, Y, n, N, K, &ks);
    if (st != NVFP4_OK)
        return st;
    if (ksplit_workspace_bytes(ks, n, N) > kScratchBytes)
        return NVFP4_ERR_SCRATCH;
    void *ws = nullptr;
    if (ks > 1) {
        st = scratch_on_current_device(&ws);
        if (st != NVFP4_OK)
            return st;
    }
    return launch_gemv(make_params(Wq, Wscale, gscale, X, Y, n, N, K), (hipStream_t)stream, ks, ws);
}

size_t nvfp4_gemv_static_scratch_bytes(void)
{
    return kScratchBytes;
}

int nvfp4_gemv_qkv(const uint8_t *Wq, const uint8_t *Wscale, float gscale, const uint16_t *X,
                   uint16_t *Y, int n, int K, const int32_t rows[3], const int64_t out_off[3],
                   int64_t ldy, void *stream)
{
    if (!rows || !out_off)
        return NVFP4_ERR_NULL;
    long long N = 0;
    for (int j = 0; j < 3; ++j) {
        if (rows[j] < 0 || out_off[j] < 0 || out_off[j] + rows[j] > ldy)
            return NVFP4_ERR_RANGE;
        N += rows[j];
    }
    if (N < 1 || N > 0x7FFFFFFF)
        return NVFP4_ERR_RANGE;
    for (int a = 0; a < 3; ++a)
        for (int b = a + 1; b < 3; ++b)
            if (rows[a] > 0 && rows[b] > 0 && out_off[a] < out_off[b] + rows[b] &&
                out_off[b] < out_off[a] + rows[a])
                return NVFP4_ERR_RANGE;   // output ranges overlap
    int st = validate_common(Wq, Wscale, X, Y, n, (int)N, K);
    if (st != NVFP4_OK)
        return st;
    GemvParams p = make_params(Wq, Wscale, gscale, X, Y, n, (int)N, K);
    p.start1 = rows[0];
    p.start2 = rows[0] + rows[1];
    p.off0 = out_off[0];
    p.off1 = out_off[1];
    p.off2 = out_off[2];
    p.ldy = ldy;
    return launch_gemv(p, (hipStream_t)stream);
}

int nvfp4_gemv_sched(const uint8_t *Wq, const uint8_t *Wscale, float gscale, const uint16_t *X,
                     uint16_t *Y, int n, int N, int K, const uint8_t *tile_widths, int ntiles,
                     void *stream)
{
    int st = validate_common(Wq, Wscale, X, Y, n, N, K);
    if (st != NVFP4_OK)
        return st;
    st = check_schedule(n, tile_widths, ntiles);
    if (st != NVFP4_OK)
        return st;
    int t0 = 0;
    for (int j = 0; j < ntiles; ++j) {
        GemvParams p = make_params(Wq, Wscale, gscale, X + (size_t)t0 * K, Y + (size_t)t0 * N,
                                   tile_widths[j], N, K);
        st = launch_gemv(p, (hipStream_t)stream);
        if (st != NVFP4_OK)
            return st;
        t0 += tile_widths[j];
    }
    return NVFP4_OK;
}

int nvfp4_gemm(const uint8_t *Wq, const uint8_t *Wscale, float gscale, const uint16_t *X, uint16_t *Y,
               int n, int N, int K, void *stream)
{
    int st = validate_gemm(Wq, Wscale, X, Y, n, N, K);
    if (st != NVFP4_OK)
        return st;
    int cus = 0;
    st = current_device_info(&cus);
    if (st != NVFP4_OK)
        return st;
    GemmGeometry geo;
    gemm_geometry_for(n, N, cus, &geo);
    GemmParams p;
    p.codes = reinterpret_cast<const u32x4 *>(Wq);
    p.scales = reinterpret_cast<const u32x2 *>(Wscale);
    p.X = X;
    p.Y = Y;
    p.gscale = gscale;
    p.n = n;
    p.N = N;
    p.K = K;
    p.T = (int)k_tiles(K);
    p.RG = (int)row_groups(N);
    GemmKernel kern = pick_gemm(geo);
    if (!kern)
        return NVFP4_ERR_SHAPE;
    hipLaunchKernelGGL(kern, dim3(geo.grid_x, geo.grid_y),
                       dim3(geo.gw * 64), 0,
                       (hipStream_t)stream, p);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

int nvfp4_gemm_geometry(int n, int N, int K, int *rows_per_workgroup, int *tokens_per_workgroup,
                        int *grid_x, int *grid_y)
{
    if (!rows_per_workgroup || !tokens_per_workgroup || !grid_x || !grid_y)
        return NVFP4_ERR_NULL;
    if (n < 1 || n > NVFP4_MAX_GEMM_TOKENS || N < 1 || K < 1)
        return NVFP4_ERR_RANGE;
    if (K % 16 != 0 || K > kMaxK)
        return NVFP4_ERR_SHAPE;
    GemmGeometry geo;
    gemm_geometry_for(n, N, 256, &geo);   // MI355X; the launch itself uses the queried count
    *rows_per_workgroup = geo.rgw * geo.gw / geo.ts * kRowsPerGroup;
    *tokens_per_workgroup = geo.bmb * 16;
    *grid_x = geo.grid_x;
    *grid_y = geo.grid_y;
    return NVFP4_OK;
}

int nvfp4_schedule(int n, int N, int K, uint8_t *widths, int max_tiles)
{
    if (!widths)
        return -NVFP4_ERR_NULL;
    if (n < 1 || n > NVFP4_MAX_TOKENS || N < 1 || K < 1)
        return -NVFP4_ERR_RANGE;
    if (K % 16 != 0 || K > kMaxK)
        return -NVFP4_ERR_SHAPE;   // a shape nvfp4_gemv refuses has no schedule
    if (max_tiles < 1)
        return -NVFP4_ERR_SCHEDULE;
    // One launch reads the weight once for every n <= 16; measured faster than
    // any split into several launches at every shape (each extra tile re-reads
    // the whole weight).
    widths[0] = (uint8_t)n;
    return 1;
}

int nvfp4_schedule_greedy(int n, int width, uint8_t *widths, int max_tiles)
{
    if (!widths)
        return -NVFP4_ERR_NULL;
    if (n < 1 || n > NVFP4_MAX_TOKENS || width < 1 || width > NVFP4_MAX_TOKENS)
        return -NVFP4_ERR_RANGE;
    int cnt = 0, left = n;
    while (left > 0) {
        if (cnt >= max_tiles)
            return -NVFP4_ERR_SCHEDULE;
        const int w = left < width ? left : width;
        widths[cnt++] = (uint8_t)w;
        left -= w;
    }
    return cnt;
}

int nvfp4_launch_geometry(int n, int N, int K, int *workgroups, int *waves, int *tiles_per_wave)
{
    if (!workgroups || !waves || !tiles_per_wave)
        return NVFP4_ERR_NULL;
    if (n < 1 || n > NVFP4_MAX_TOKENS || N < 1 || K < 1)
        return NVFP4_ERR_RANGE;
    if (K % 16 != 0 || K > kMaxK)
        return NVFP4_ERR_SHAPE;
    int cus = 256;   // MI355X; the launch itself uses the queried count
    Geometry geo;
    if (!geometry_for(N, K, cus, 1, &geo))
        return NVFP4_ERR_SHAPE;
    *workgroups = geo.workgroups;
    *waves = kWaves;
    *tiles_per_wave = geo.mt;
    return NVFP4_OK;
}

int nvfp4_gemv_variant(int n, int N, int K, int ks, int *variant)
{
    if (!variant)
        return NVFP4_ERR_NULL;
    if (n < 1 || n > NVFP4_MAX_TOKENS || N < 1 || K < 1 || ks < 0 || ks > kMaxKParts)
        return NVFP4_ERR_RANGE;
    if (K % 16 != 0 || K > kMaxK)
        return NVFP4_ERR_SHAPE;
    if (ks == 0)
        ks = ksplit_for(N, K);
    Geometry geo;
    if (!geometry_for(N, K, 256, ks, &geo))
        return NVFP4_ERR_SHAPE;
    if (!pick_kernel(n, geo.mt, geo.exact, geo.kc > 1, ks > 1))
        return NVFP4_ERR_SHAPE;
    variant[0] = geo.mt;
    variant[1] = (n + 3) / 4;
    variant[2] = geo.exact ? 1 : 0;
    variant[3] = geo.kc;
    variant[4] = ks;
    return NVFP4_OK;
}

const char *nvfp4_strerror(int status)
{
    switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "null pointer argument";
    case NVFP4_ERR_RANGE: return "argument out of range";
    case NVFP4_ERR_ALIGN: return "misaligned pointer";
    case NVFP4_ERR_SHAPE: return "unsupported shape";
    case NVFP4_ERR_SCHEDULE: return "invalid tile schedule";
    case NVFP4_ERR_LAUNCH: return "kernel launch failed";
    case NVFP4_ERR_DEVICE: return "current device is not gfx950";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_SCRATCH: return "call needs more than the library's fixed scratch memory";
    default: return "unknown status";
    }
}

}  // extern "C"
