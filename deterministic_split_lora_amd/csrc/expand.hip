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

// (row block, column block) of a 1-D grid, column block fastest: consecutive
// workgroups, which land on different XCDs, cover adjacent stretches of the
// same y rows.
struct ExpandItem {
    int64_t row0;
    int64_t cb;
    int nrows;
};

__device__ __forceinline__ ExpandItem expand_item(int64_t M, int64_t N)
{
    ExpandItem q;                                 // 32-bit: the grid is below 2^31
    const uint32_t nblocks = (uint32_t)((N + kExpandCols - 1) / kExpandCols);
    q.cb = blockIdx.x % nblocks;
    q.row0 = (int64_t)(blockIdx.x / nblocks) * kRowBlock;
    const int64_t left = M - q.row0;
    q.nrows = left < kRowBlock ? (int)left : kRowBlock;
    return q;
}

// Single adapter: 4 waves of 64 columns per workgroup.
template <int KS>
__global__ __launch_bounds__(256) void k_expand(ExpandParams p)
{
    const ExpandItem q = expand_item(p.M, p.N);
    const int64_t row0 = q.row0;
    const int nrows = q.nrows;
    ExpandLane L = expand_lane(row0, nrows, q.cb * kExpandCols);
    if (L.n_base >= p.N)
        return;
    u16x8 yv[2];
    bf16x8 bop[4][KS];
    expand_load<KS>(L, p.y, p.ld_y, p.N, p.B, p.ld_b, p.r, yv, bop);
    expand_finish<KS>(L, p.y, p.ld_y, p.N, p.h + row0 * p.ld_h, p.ld_h, p.r, p.scale, yv, bop);
}

// Fused: the fixed pairwise tree over the Split-K workspace for this row block
// (exactly the second pass of the deterministic shrink: tree, then one
// multiply by the shrink scale) is evaluated into an LDS tile, written out as
// h by the first column block, and fed to the expand without a round trip
// through a separate kernel.  Same bits as shrink then expand.
constexpr int kHTileStride = 68;          // floats per LDS row (64 + 4 padding)

template <int KS, int S>
__global__ __launch_bounds__(256) void k_expand_combine(ExpandParams p, TreeParams c)
{
    __shared__ __align__(16) float hs[kRowBlock * kHTileStride];
    const ExpandItem q = expand_item(p.M, p.N);
    const int64_t row0 = q.row0;
    const int nrows = q.nrows;
    const int r = p.r;
    // y and B first: they do not depend on the workspace
    ExpandLane L = expand_lane(row0, nrows, q.cb * kExpandCols);
    const bool active = L.n_base < p.N;
    u16x8 yv[2];
    bf16x8 bop[4][KS];
    if (active)
        expand_load<KS>(L, p.y, p.ld_y, p.N, p.B, p.ld_b, r, yv, bop);
    const bool write_h = c.h != nullptr && q.cb == 0;
    for (int e = threadIdx.x; e < kRowBlock * r; e += 256) {
        const int row = e / r;
        const int col = e - row * r;
        if (row < nrows) {
            float v[S];
            const float* w = c.ws + (row0 + row) * c.ldw + col;
#pragma unroll
            for (int s = 0; s < S; ++s)
                v[s] = w[(int64_t)s * c.split_stride];
            const float hv = __fmul_rn(pairwise_tree<S>(v), c.scale);
            hs[row * kHTileStride + col] = hv;
            if (write_h)
                c.h[(row0 + row) * c.ld_h + col] = hv;
        }
    }
    __syncthreads();
    if (!active)
        return;
    expand_finish<KS>(L, p.y, p.ld_y, p.N, hs, kHTileStride, r, p.scale, yv, bop);
}

// Multi-adapter: a fixed grid walks the plan's (tile, column block) items.
__global__ __launch_bounds__(256) void k_sgmv_expand(ExpandParams p)
{
    const int ntiles = plan_tiles(p.tiles, p.M, p.n_adapters);
    const uint32_t nblocks = (uint32_t)((p.N + kExpandCols - 1) / kExpandCols);
    const uint32_t items = (uint32_t)ntiles * nblocks;
    for (uint32_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int tile = (int)(it / nblocks);
        const int64_t cb = it - (uint32_t)tile * nblocks;
        const int32_t* t = p.tiles + kPlanHeaderInts + 3 * tile;
        if (!tile_ok(t, p.M, p.n_adapters))
            continue;
        const int a = t[2];
        int ra = p.ranks[a];
        ra = ra < 0 ? 0 : (ra > p.r_max ? p.r_max : ra);
        const float scale = p.scales ? p.scales[a] : 1.0f;
        const int64_t ld_b = (ra + 7) & ~7;
        ExpandLane L = expand_lane(t[0], t[1], cb * kExpandCols);
        if (L.n_base >= p.N)
            continue;
        const float* hrows = p.h + (int64_t)t[0] * p.ld_h;
        u16x8 yv[2];
        if (ra > 32) {
            bf16x8 bop[4][2];
            expand_load<2>(L, p.y, p.ld_y, p.N, p.B_ptrs[a], ld_b, ra, yv, bop);
            expand_finish<2>(L, p.y, p.ld_y, p.N, hrows, p.ld_h, ra, scale, yv, bop);
        } else {
            bf16x8 bop[4][1];
            expand_load<1>(L, p.y, p.ld_y, p.N, p.B_ptrs[a], ld_b, ra, yv, bop);
            expand_finish<1>(L, p.y, p.ld_y, p.N, hrows, p.ld_h, ra, scale, yv, bop);
        }
    }
}

}  // namespace

inline dim3 expand_grid(int64_t M, int64_t N)
{
    return dim3((unsigned)(((M + kRowBlock - 1) / kRowBlock) * ((N + kExpandCols - 1) / kExpandCols)));
}

hipError_t launch_expand(const ExpandParams& p, hipStream_t st)
{
    const dim3 grid = expand_grid(p.M, p.N);
    dim3 block(256);
    if (p.r > 32)
        hipLaunchKernelGGL(k_expand<2>, grid, block, 0, st, p);
    else
        hipLaunchKernelGGL(k_expand<1>, grid, block, 0, st, p);
    return hipGetLastError();
}

template <int KS>
hipError_t launch_expand_combine_ks(const ExpandParams& p, const TreeParams& c, int S, dim3 grid, hipStream_t st)
{
    switch (S) {
    case 1: hipLaunchKernelGGL((k_expand_combine<KS, 1>), grid, dim3(256), 0, st, p, c); break;
    case 2: hipLaunchKernelGGL((k_expand_combine<KS, 2>), grid, dim3(256), 0, st, p, c); break;
    case 4: hipLaunchKernelGGL((k_expand_combine<KS, 4>), grid, dim3(256), 0, st, p, c); break;
    case 8: hipLaunchKernelGGL((k_expand_combine<KS, 8>), grid, dim3(256), 0, st, p, c); break;
    default: hipLaunchKernelGGL((k_expand_combine<KS, 16>), grid, dim3(256), 0, st, p, c); break;
    }
    return hipGetLastError();
}

hipError_t launch_expand_combine(const ExpandParams& p, const TreeParams& c, int split_k, hipStream_t st)
{
    const dim3 grid = expand_grid(p.M, p.N);
    return p.r > 32 ? launch_expand_combine_ks<2>(p, c, split_k, grid, st)
                    : launch_expand_combine_ks<1>(p, c, split_k, grid, st);
}

hipError_t launch_sgmv_expand(const ExpandParams& p, int grid, hipStream_t st)
{
    hipLaunchKernelGGL(k_sgmv_expand, dim3((unsigned)grid), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace lora
