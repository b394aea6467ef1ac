// Split-K LoRA shrink kernels for gfx950.
//
// The shrink h = x A^T (paper Eq. 1) is a narrow GEMM: K = hidden size is long,
// r <= 64 is short.  Split-K (section 2.1, Eq. 3) cuts K into S contiguous
// chunks so S workgroups share one output tile.  One workgroup owns one
// (16-token row block, split) pair and W wavefronts; wave w walks
// k_steps * 32 consecutive k of the split's chunk with matrix-core steps, the
// bf16 operands streamed straight from HBM into registers with 16-byte loads
// (x rows and A rows are both k-contiguous, which is exactly the per-lane
// operand layout, so no LDS transpose is needed and every byte is loaded once
// per workgroup).  The W wave results meet in LDS and are added along a fixed
// pairwise tree.  The split's fp32 partial then goes to the workspace
// (deterministic path), straight to h (split_k == 1), or is atomically added
// to h (the nondeterministic contrast of section 4.1).
//
// Every element's arithmetic - which k each matrix-core step covers, the step
// order, the wave tree, the split tree - is fixed by (K, split_k) alone, so a
// token's bits do not depend on M or on its neighbours in the batch.
#include "device.h"
#include "kernels.h"

namespace lora {

namespace {

enum ShrinkMode { kToWorkspace = 0, kToOutputScaled = 1, kAtomicScaled = 2 };

// Output element (row, col) of the tile: write / atomically add.
template <int MODE>
__device__ __forceinline__ void shrink_store(const ShrinkParams& p, int64_t row0, int s, int row,
                                             int col, float v, float scale)
{
    const int64_t rr = row0 + row;
    if (MODE == kToWorkspace) {
        p.out[(int64_t)s * p.split_stride + rr * p.ld_out + col] = v;
    } else if (MODE == kToOutputScaled) {
        p.out[rr * p.ld_out + col] = __fmul_rn(v, scale);
    } else {
        unsafeAtomicAdd(&p.out[rr * p.ld_out + col], __fmul_rn(v, scale));
    }
}

// One (row block, split) work item.  RT = number of 16-wide rank tiles the
// kernel is built for; r <= 16 * RT is the rank actually used.
template <int RT, int W, int MODE>
__device__ __forceinline__ void shrink_tile(const ShrinkParams& p, int64_t row0, int nrows,
                                            const uint16_t* __restrict__ A, int r, int s,
                                            float scale, float* red)
{
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int g = lane >> 4;
    const int steps = p.k_steps;

    // Reduction slots 8g..8g+7 of step t hold k = kbase + 32 t + (0..7).
    const int64_t kbase = (int64_t)s * p.k_chunk + (int64_t)wave * steps * kKStep + g * 8;
    const bool row_ok = li < nrows;
    const uint16_t* xp = p.x + (row0 + (row_ok ? li : 0)) * p.ld_x + kbase;
    const uint16_t* ap[RT];
    bool a_ok[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int j = rt * 16 + li;
        a_ok[rt] = j < r;
        ap[rt] = A + (int64_t)(a_ok[rt] ? j : 0) * p.ld_a + kbase;
    }

    f32x4 acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Groups of up to 4 steps: issue all loads of the group, then the
    // matrix-core steps in ascending k.
    for (int t0 = 0; t0 < steps; t0 += 4) {
        bf16x8 xa[4];
        bf16x8 b[4][RT];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (t0 + u < steps) {
                const int off = (t0 + u) * kKStep;
                xa[u] = row_ok ? load_bf16x8(xp + off) : bf16x8_zero();
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    b[u][rt] = (rt * 16 < r && a_ok[rt]) ? load_bf16x8(ap[rt] + off) : bf16x8_zero();
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (t0 + u < steps) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    if (rt * 16 < r)
                        acc[rt] = mfma_16x16x32(xa[u], b[u][rt], acc[rt]);
            }
        }
    }

    // acc[rt][v] is the wave's sum for token row 4g+v, rank column 16 rt + li.
    if constexpr (W == 1) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 4 * g + v, col = rt * 16 + li;
                if (row < nrows && col < r)
                    shrink_store<MODE>(p, row0, s, row, col, acc[rt][v], scale);
            }
    } else {
        constexpr int RS = 16 * RT + 4;          // padded LDS row stride (floats)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[(wave * 16 + 4 * g + v) * RS + rt * 16 + li] = acc[rt][v];
        __syncthreads();
        const int ncols = r < 16 * RT ? r : 16 * RT;
        for (int e = threadIdx.x; e < 16 * 16 * RT; e += W * kWave) {
            const int row = e / (16 * RT);
            const int col = e - row * (16 * RT);
            if (row < nrows && col < ncols) {
                float v[W];
#pragma unroll
                for (int w = 0; w < W; ++w)
                    v[w] = red[(w * 16 + row) * RS + col];
                shrink_store<MODE>(p, row0, s, row, col, pairwise_tree<W>(v), scale);
            }
        }
        __syncthreads();                          // LDS is reused by the next item
    }
}

template <int RT, int W>
constexpr int red_floats()
{
    return W > 1 ? W * 16 * (16 * RT + 4) : 1;
}

// Single adapter: grid (ceil(M/16), split_k), W waves.
template <int RT, int W, int MODE>
__global__ __launch_bounds__(W * 64) void k_shrink_partial(ShrinkParams p)
{
    __shared__ float red[red_floats<RT, W>()];
    const int64_t row0 = (int64_t)blockIdx.x * kRowBlock;
    const int64_t left = p.M - row0;
    const int nrows = left < kRowBlock ? (int)left : kRowBlock;
    shrink_tile<RT, W, MODE>(p, row0, nrows, p.A, p.r, (int)blockIdx.y, p.scale, red);
}

// Multi-adapter: a fixed grid walks the plan's (tile, split) items with a
// static stride; every wave of a workgroup sees the same item count and
// leaves the loop together.
template <int W>
__global__ __launch_bounds__(W * 64) void k_sgmv_shrink_partial(ShrinkParams p)
{
    __shared__ float red[red_floats<4, W>()];
    const int ntiles = plan_tiles(p.tiles, p.M, p.n_adapters);
    const int S = p.split_k;
    const int64_t items = (int64_t)ntiles * S;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int tile = (int)(it / S);
        const int s = (int)(it - (int64_t)tile * S);
        const int32_t* t = p.tiles + kPlanHeaderInts + 3 * tile;
        if (!tile_ok(t, p.M, p.n_adapters))      // uniform across the workgroup
            continue;
        const int64_t row0 = t[0];
        const int nrows = t[1];
        const int a = t[2];
        int ra = p.ranks[a];
        ra = ra < 0 ? 0 : (ra > p.r_max ? p.r_max : ra);
        shrink_tile<4, W, kToWorkspace>(p, row0, nrows, p.A_ptrs[a], ra, s, 1.0f, red);
    }
}

// h = scale * tree(ws[0..S-1]) elementwise.
template <int S, bool SGMV>
__global__ __launch_bounds__(256) void k_splitk_tree(TreeParams p)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= p.M * p.ncols)
        return;
    const int64_t i = e / p.ncols;
    const int j = (int)(e - i * p.ncols);
    float scale = p.scale;
    float* hp = p.h + i * p.ld_h + j;
    if constexpr (SGMV) {
        const int a = p.ids[i];
        if (a < 0 || a >= p.n_adapters) {
            *hp = 0.0f;
            return;
        }
        int ra = p.ranks[a];
        ra = ra < 0 ? 0 : (ra > p.ncols ? p.ncols : ra);
        if (j >= ra) {
            *hp = 0.0f;
            return;
        }
        scale = p.scales ? p.scales[a] : 1.0f;
    }
    float v[S];
    const float* w = p.ws + i * p.ldw + j;
#pragma unroll
    for (int s = 0; s < S; ++s)
        v[s] = w[(int64_t)s * p.split_stride];
    *hp = __fmul_rn(pairwise_tree<S>(v), scale);
}

__global__ __launch_bounds__(256) void k_fill_zero(float* h, int64_t ld_h, int64_t M, int ncols)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= M * ncols)
        return;
    const int64_t i = e / ncols;
    h[i * ld_h + (e - i * ncols)] = 0.0f;
}

template <int MODE, int W>
hipError_t launch_partial_w(const ShrinkParams& p, int rt, hipStream_t st)
{
    dim3 grid((unsigned)((p.M + kRowBlock - 1) / kRowBlock), (unsigned)p.split_k);
    dim3 block(W * 64);
    switch (rt) {
    case 1: hipLaunchKernelGGL((k_shrink_partial<1, W, MODE>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((k_shrink_partial<2, W, MODE>), grid, block, 0, st, p); break;
    case 3: hipLaunchKernelGGL((k_shrink_partial<3, W, MODE>), grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL((k_shrink_partial<4, W, MODE>), grid, block, 0, st, p); break;
    }
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_partial(const ShrinkParams& p, int waves, int rt, hipStream_t st)
{
    switch (waves) {
    case 1: return launch_partial_w<MODE, 1>(p, rt, st);
    case 2: return launch_partial_w<MODE, 2>(p, rt, st);
    case 4: return launch_partial_w<MODE, 4>(p, rt, st);
    default: return launch_partial_w<MODE, 8>(p, rt, st);
    }
}

template <bool SGMV>
hipError_t launch_tree_t(const TreeParams& p, int S, hipStream_t st)
{
    const int64_t n = p.M * p.ncols;
    dim3 grid((unsigned)((n + 255) / 256)), block(256);
    switch (S) {
    case 1: hipLaunchKernelGGL((k_splitk_tree<1, SGMV>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((k_splitk_tree<2, SGMV>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((k_splitk_tree<4, SGMV>), grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL((k_splitk_tree<8, SGMV>), grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL((k_splitk_tree<16, SGMV>), grid, block, 0, st, p); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_shrink_partial_ws(const ShrinkParams& p, int waves, int rank_tiles, hipStream_t st)
{
    return launch_partial<kToWorkspace>(p, waves, rank_tiles, st);
}

hipError_t launch_shrink_partial_direct(const ShrinkParams& p, int waves, int rank_tiles, hipStream_t st)
{
    return launch_partial<kToOutputScaled>(p, waves, rank_tiles, st);
}

hipError_t launch_shrink_partial_atomic(const ShrinkParams& p, int waves, int rank_tiles, hipStream_t st)
{
    return launch_partial<kAtomicScaled>(p, waves, rank_tiles, st);
}

hipError_t launch_sgmv_shrink_partial(const ShrinkParams& p, int waves, int grid, hipStream_t st)
{
    dim3 g((unsigned)grid), b(waves * 64);
    switch (waves) {
    case 1: hipLaunchKernelGGL((k_sgmv_shrink_partial<1>), g, b, 0, st, p); break;
    case 2: hipLaunchKernelGGL((k_sgmv_shrink_partial<2>), g, b, 0, st, p); break;
    case 4: hipLaunchKernelGGL((k_sgmv_shrink_partial<4>), g, b, 0, st, p); break;
    default: hipLaunchKernelGGL((k_sgmv_shrink_partial<8>), g, b, 0, st, p); break;
    }
    return hipGetLastError();
}

hipError_t launch_splitk_tree(const TreeParams& p, int split_k, bool sgmv, hipStream_t st)
{
    return sgmv ? launch_tree_t<true>(p, split_k, st) : launch_tree_t<false>(p, split_k, st);
}

hipError_t launch_fill_zero(float* h, int64_t ld_h, int64_t M, int ncols, hipStream_t st)
{
    const int64_t n = M * ncols;
    dim3 grid((unsigned)((n + 255) / 256)), block(256);
    hipLaunchKernelGGL(k_fill_zero, grid, block, 0, st, h, ld_h, M, ncols);
    return hipGetLastError();
}

}  // namespace lora
