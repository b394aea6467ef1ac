// LoRA expand kernels for gfx950: y[i][n] <- bf16( fma(s, sum_j bf16(h[i][j]) B[n][j], y[i][n]) )
// (paper Eq. 1, the s (X A^T) B^T term added into Y; h is rounded to bf16 as
// in section 6.2 before it meets B).
//
// The expand moves 4 bytes of y (read + write) per output element and does
// only 2r flops on it, so it is bound by HBM traffic on y.  The layout is
// chosen for y: each lane ends up owning 16 consecutive columns of one token,
// so y is read and written with 16-byte vector accesses straight from the
// matrix-core accumulators, with no LDS round trip.
//
// How: the matrix-core "row" operand is B (a row per output column n) and the
// "column" operand is h (a column per token).  Accumulator register v of lane
// (li, g) holds output row 4g+v of column li, and the kernel chooses which n
// each operand row stands for: in tile t (0..3), operand row m is column
//     n = n_base + 16 (m / 4) + 4 t + (m % 4),
// so lane (li, g) collects columns n_base + 16 g + 4 t + v, t, v in 0..3 - a
// contiguous run of 16 - for token li.  Per element, the arithmetic is one
// matrix-core step over j < 32 (r <= 32) or two (r <= 64) with zero-padded
// reduction slots, then one fma and one rounding; it does not depend on the
// tiling, M or the token's neighbours.
#include "device.h"
#include "kernels.h"

namespace lora {

namespace {

// bf16(h[row][j0 .. j0+7]) with columns >= r read as 0.
__device__ __forceinline__ bf16x8 load_h_as_bf16(const float* hp, int j0, int r)
{
    float f[8];
    if (j0 + 8 <= r) {
        const float4 a = *reinterpret_cast<const float4*>(hp);
        const float4 b = *reinterpret_cast<const float4*>(hp + 4);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            f[e] = (j0 + e < r) ? hp[e] : 0.0f;
    }
    u16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        v[e] = f32_to_bf16_bits(f[e]);
    return __builtin_bit_cast(bf16x8, v);
}

// Tokens row0 .. row0+nrows-1 (nrows <= 16) x columns [256 cb, 256 cb + 256).
// KS = matrix-core steps over the rank: 1 for r <= 32, 2 for r <= 64.
template <int KS>
__device__ __forceinline__ void expand_tile(const ExpandParams& p, int64_t row0, int nrows,
                                            const uint16_t* __restrict__ B, int64_t ld_b, int r,
                                            float scale, int64_t cb)
{
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int g = lane >> 4;
    const int64_t n_base = cb * kExpandCols + wave * 64;
    if (n_base >= p.N)
        return;
    const bool row_ok = li < nrows;
    const int64_t row = row0 + (row_ok ? li : 0);

    bf16x8 hb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int j0 = ks * kKStep + 8 * g;
        hb[ks] = (row_ok && j0 < r) ? load_h_as_bf16(p.h + row * p.ld_h + j0, j0, r) : bf16x8_zero();
    }

    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int64_t n = n_base + (li >> 2) * 16 + t * 4 + (li & 3);
        const bool n_ok = n < p.N;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int j0 = ks * kKStep + 8 * g;
            const bf16x8 bv = (n_ok && j0 < r) ? load_bf16x8_partial(B + n * ld_b + j0, r - j0)
                                               : bf16x8_zero();
            acc[t] = mfma_16x16x32(bv, hb[ks], acc[t]);
        }
    }

    if (!row_ok)
        return;
    const int64_t n0 = n_base + 16 * g;
    uint16_t* yp = p.y + row * p.ld_y + n0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        if (n0 + half * 8 < p.N) {                 // N % 8 == 0: chunks are whole
            u16x8* q = reinterpret_cast<u16x8*>(yp + half * 8);
            const u16x8 yv = *q;
            u16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int idx = half * 8 + e;
                o[e] = f32_to_bf16_bits(__builtin_fmaf(scale, acc[idx >> 2][idx & 3], bf16_bits_to_f32(yv[e])));
            }
            *q = o;
        }
    }
}

// Single adapter: grid (ceil(M/16), ceil(N/256)), 4 waves.
template <int KS>
__global__ __launch_bounds__(256) void k_expand(ExpandParams p)
{
    const int64_t row0 = (int64_t)blockIdx.x * kRowBlock;
    const int64_t left = p.M - row0;
    const int nrows = left < kRowBlock ? (int)left : kRowBlock;
    expand_tile<KS>(p, row0, nrows, p.B, p.ld_b, p.r, p.scale, blockIdx.y);
}

// Multi-adapter: a fixed grid walks the plan's (tile, column block) items.
__global__ __launch_bounds__(256) void k_sgmv_expand(ExpandParams p)
{
    const int ntiles = plan_tiles(p.tiles, p.M, p.n_adapters);
    const int64_t nblocks = (p.N + kExpandCols - 1) / kExpandCols;
    const int64_t items = (int64_t)ntiles * nblocks;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int tile = (int)(it / nblocks);
        const int64_t cb = it - (int64_t)tile * nblocks;
        const int32_t* t = p.tiles + kPlanHeaderInts + 3 * tile;
        if (!tile_ok(t, p.M, p.n_adapters))
            continue;
        const int a = t[2];
        int ra = p.ranks[a];
        ra = ra < 0 ? 0 : (ra > p.r_max ? p.r_max : ra);
        const float scale = p.scales ? p.scales[a] : 1.0f;
        const int64_t ld_b = (ra + 7) & ~7;
        if (ra > 32)
            expand_tile<2>(p, t[0], t[1], p.B_ptrs[a], ld_b, ra, scale, cb);
        else
            expand_tile<1>(p, t[0], t[1], p.B_ptrs[a], ld_b, ra, scale, cb);
    }
}

}  // namespace

hipError_t launch_expand(const ExpandParams& p, hipStream_t st)
{
    dim3 grid((unsigned)((p.M + kRowBlock - 1) / kRowBlock), (unsigned)((p.N + kExpandCols - 1) / kExpandCols));
    dim3 block(256);
    if (p.r > 32)
        hipLaunchKernelGGL(k_expand<2>, grid, block, 0, st, p);
    else
        hipLaunchKernelGGL(k_expand<1>, grid, block, 0, st, p);
    return hipGetLastError();
}

hipError_t launch_sgmv_expand(const ExpandParams& p, int grid, hipStream_t st)
{
    hipLaunchKernelGGL(k_sgmv_expand, dim3((unsigned)grid), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace lora
