// Deterministic Split-K shrink and expand in a single launch, for gfx950.
//
// The paper's point (section 2) is that the shrink alone exposes too little
// output parallelism, which Split-K (Eq. 3) restores by cutting K into S
// chunks.  When the shrink is immediately followed by its expand, the expand's
// H_out columns are plenty of parallelism: here each workgroup owns one
// 16-token block and 512 output columns, recomputes that block's shrink itself
// and expands it - so no workgroup ever waits for, or reads the results of,
// another one, and there is a single kernel launch.
//
// The recomputed shrink is the deterministic Split-K shrink of this library
// step for step: the same S contiguous chunks, each cut into the same W
// consecutive sub-chunks of k_steps matrix-core steps (each a fresh fp32 chain
// in ascending k with the same lane/slot assignment), the same pairwise tree
// over the W chains, the same pairwise tree over the S split partials, the same
// single multiply by the shrink scale.  Wave v evaluates the splits v, v+8, ...
// in registers and leaves their partials in LDS; the split tree runs over LDS.
// Every h and y bit therefore equals the two-pass path's (partials kernel,
// tree kernel, expand kernel) - the tests check this - while the 16-byte
// loads of y and B are issued before the shrink so that their latency hides
// behind it.
#include "device.h"
#include "kernels.h"

namespace lora {

namespace {

constexpr int kFusedWaves = 8;
constexpr int kFusedCols = kFusedWaves * 64;   // output columns per workgroup

// The operands one wave needs to run the matrix-core chains of a split.
template <int RTMAX>
struct ChainOperands {
    const uint16_t* xrow;          // token row li of the block, + 8g
    const uint16_t* arow[RTMAX];   // rank row 16 rt + li of A, + 8g
    bool a_ok[RTMAX];
    bool row_ok;
    int r;
    int steps;
    int64_t k0;                    // first k of the split's chunk
};

// Issues the loads of matrix-core steps q0 .. q0+G-1 of the split (those < n).
template <int RTMAX, int G>
__device__ __forceinline__ void load_steps(const ChainOperands<RTMAX>& c, int q0, int n, bf16x8 (&xg)[G],
                                           bf16x8 (&ag)[G][RTMAX])
{
#pragma unroll
    for (int u = 0; u < G; ++u) {
        const int q = q0 + u;
        const int64_t off = c.k0 + (int64_t)(q < n ? q : 0) * kKStep;
        xg[u] = (q < n && c.row_ok) ? load_bf16x8(c.xrow + off) : bf16x8_zero();
#pragma unroll
        for (int rt = 0; rt < RTMAX; ++rt)
            ag[u][rt] = (q < n && rt * 16 < c.r && c.a_ok[rt]) ? load_bf16x8(c.arow[rt] + off) : bf16x8_zero();
    }
}

template <int RTMAX>
__device__ __forceinline__ void add4(f32x4 (&d)[RTMAX], const f32x4 (&a)[RTMAX], const f32x4 (&b)[RTMAX])
{
#pragma unroll
    for (int rt = 0; rt < RTMAX; ++rt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            d[rt][v] = __fadd_rn(a[rt][v], b[rt][v]);
}

// Runs steps q0 .. q0+G-1 (those < n) from the given operand buffers.  A
// chain starts from zero every k_steps steps; a finished chain w joins the
// neighbour-pairwise tree over the W chains held in l0 (single), l1 (pair),
// l2 (quad): chain w pairs with w^1, pairs with pairs, quads with quads -
// ((c0+c1)+(c2+c3)) + ((c4+c5)+(c6+c7)), the additions of the two-pass
// kernel's wave tree in the same order.  `out` is set by the last chain.
template <int RTMAX, int W, int G>
__device__ __forceinline__ void run_steps(const ChainOperands<RTMAX>& c, int q0, int n, const bf16x8 (&xg)[G],
                                          const bf16x8 (&ag)[G][RTMAX], f32x4 (&acc)[RTMAX], int& tin, int& w,
                                          f32x4 (&l0)[RTMAX], f32x4 (&l1)[RTMAX], f32x4 (&l2)[RTMAX],
                                          f32x4 (&out)[RTMAX])
{
#pragma unroll
    for (int u = 0; u < G; ++u) {
        if (q0 + u < n) {
            if (tin == 0) {
#pragma unroll
                for (int rt = 0; rt < RTMAX; ++rt)
                    acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int rt = 0; rt < RTMAX; ++rt)
                if (rt * 16 < c.r)
                    acc[rt] = mfma_16x16x32(xg[u], ag[u][rt], acc[rt]);
            if (++tin == c.steps) {
                tin = 0;
                if (W == 1) {
#pragma unroll
                    for (int rt = 0; rt < RTMAX; ++rt)
                        out[rt] = acc[rt];
                } else if ((w & 1) == 0) {
#pragma unroll
                    for (int rt = 0; rt < RTMAX; ++rt)
                        l0[rt] = acc[rt];
                } else {
                    f32x4 p2[RTMAX];
                    add4<RTMAX>(p2, l0, acc);
                    if (W == 2) {
#pragma unroll
                        for (int rt = 0; rt < RTMAX; ++rt)
                            out[rt] = p2[rt];
                    } else if ((w & 2) == 0) {
#pragma unroll
                        for (int rt = 0; rt < RTMAX; ++rt)
                            l1[rt] = p2[rt];
                    } else {
                        f32x4 p4[RTMAX];
                        add4<RTMAX>(p4, l1, p2);
                        if (W == 4) {
#pragma unroll
                            for (int rt = 0; rt < RTMAX; ++rt)
                                out[rt] = p4[rt];
                        } else if ((w & 4) == 0) {
#pragma unroll
                            for (int rt = 0; rt < RTMAX; ++rt)
                                l2[rt] = p4[rt];
                        } else {
                            add4<RTMAX>(out, l2, p4);
                        }
                    }
                }
                ++w;
            }
        }
    }
}

// One split's partial for the wave's 16 tokens: the W chains of k_steps
// matrix-core steps each over k0 .. k0 + W * k_steps * 32, every chain from a
// zero accumulator in ascending k, then the pairwise tree over the chains.
// The split's W * k_steps steps are walked as one stream in groups of G steps,
// double-buffered, so the loads of later chains overlap the matrix-core work
// of earlier ones.
template <int RTMAX, int W>
__device__ __forceinline__ void split_partial(const ChainOperands<RTMAX>& c, f32x4 (&out)[RTMAX])
{
    constexpr int G = RTMAX > 2 ? 2 : 4;
    const int n = W * c.steps;
    bf16x8 xa[G], xb[G];
    bf16x8 aa[G][RTMAX], ab[G][RTMAX];
    f32x4 acc[RTMAX], l0[RTMAX], l1[RTMAX], l2[RTMAX];
#pragma unroll
    for (int rt = 0; rt < RTMAX; ++rt) {
        acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        l0[rt] = acc[rt];
        l1[rt] = acc[rt];
        l2[rt] = acc[rt];
        out[rt] = acc[rt];
    }
    int tin = 0, w = 0;
    load_steps<RTMAX, G>(c, 0, n, xa, aa);
    for (int q0 = 0; q0 < n; q0 += 2 * G) {
        load_steps<RTMAX, G>(c, q0 + G, n, xb, ab);
        run_steps<RTMAX, W, G>(c, q0, n, xa, aa, acc, tin, w, l0, l1, l2, out);
        load_steps<RTMAX, G>(c, q0 + 2 * G, n, xa, aa);
        run_steps<RTMAX, W, G>(c, q0 + G, n, xb, ab, acc, tin, w, l0, l1, l2, out);
    }
}

// Which (row block, column block) a workgroup owns.  Every workgroup of a row
// block re-reads that block's x rows and all of A, so with at least 8 row
// blocks the 1-D grid keeps all column blocks of a row block on one XCD
// (workgroup ids go round-robin over the 8 XCDs, each with its own L2): XCD x
// takes row blocks x, x + 8, ...; ids past the last row block exit at once.
// With fewer row blocks the column blocks are spread over the XCDs instead.
struct FusedItem {
    int64_t mb;
    int64_t cb;
    bool ok;
};

__device__ __forceinline__ FusedItem fused_item(int64_t M, int64_t N)
{
    FusedItem q;
    const uint32_t nblocks = (uint32_t)((N + kFusedCols - 1) / kFusedCols);
    const uint32_t mbs = (uint32_t)((M + kRowBlock - 1) / kRowBlock);
    const uint32_t b = blockIdx.x;
    if (mbs >= kXcds) {
        const uint32_t slot = b / kXcds;
        q.mb = (b % kXcds) + kXcds * (slot / nblocks);
        q.cb = slot % nblocks;
    } else {
        q.mb = b / nblocks;
        q.cb = b % nblocks;
    }
    q.ok = q.mb < mbs;
    return q;
}

// RTMAX: rank tiles the kernel is built for (1: r <= 16, 2: r <= 32, one
// expand step; 4: r <= 64, two expand steps).  S: split count.  W: chains
// per split.
template <int RTMAX, int S, int W>
__global__ __launch_bounds__(kFusedWaves * 64) void k_shrink_expand_fused(FusedParams p)
{
    constexpr int KS = RTMAX > 2 ? 2 : 1;
    constexpr int PS = 16 * RTMAX + 4;            // LDS row stride of a split partial tile
    constexpr int HS = 68;                        // LDS row stride of the h tile
    __shared__ __align__(16) float ps[S * 16 * PS];
    __shared__ __align__(16) float hs[16 * HS];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int g = lane >> 4;
    const int r = p.r;
    const FusedItem item = fused_item(p.M, p.N);
    if (!item.ok)
        return;                                   // uniform: the whole workgroup leaves
    const int64_t cb = item.cb;
    const int64_t row0 = item.mb * kRowBlock;
    const int64_t left = p.M - row0;
    const int nrows = left < kRowBlock ? (int)left : kRowBlock;
    const bool row_ok = li < nrows;
    const int64_t row = row0 + (row_ok ? li : 0);

    // ---- expand operands first: y and B do not depend on the shrink -------
    ExpandLane L = expand_lane(row0, nrows, cb * kFusedCols);
    const bool cols_ok = L.n_base < p.N;
    u16x8 yv[2];
    bf16x8 bop[4][KS];
    if (cols_ok)
        expand_load<KS>(L, p.y, p.ld_y, p.N, p.B, p.ld_b, r, yv, bop);

    // ---- the block's shrink: splits wave, wave + 8, ... -------------------
    ChainOperands<RTMAX> c;
    c.xrow = p.x + row * p.ld_x + g * 8;
#pragma unroll
    for (int rt = 0; rt < RTMAX; ++rt) {
        const int j = rt * 16 + li;
        c.a_ok[rt] = j < r;
        c.arow[rt] = p.A + (int64_t)(c.a_ok[rt] ? j : 0) * p.ld_a + g * 8;
    }
    c.row_ok = row_ok;
    c.r = r;
    c.steps = p.k_steps;
    for (int s = wave; s < S; s += kFusedWaves) {
        c.k0 = (int64_t)s * p.k_chunk;
        f32x4 part[RTMAX];
        split_partial<RTMAX, W>(c, part);
#pragma unroll
        for (int rt = 0; rt < RTMAX; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                ps[(s * 16 + 4 * g + v) * PS + rt * 16 + li] = part[rt][v];
    }
    __syncthreads();

    // ---- pairwise tree over the S split partials, times the shrink scale --
    const int ncols = r < 16 * RTMAX ? r : 16 * RTMAX;
    const bool write_h = p.h != nullptr && cb == 0;
    for (int e = threadIdx.x; e < 16 * ncols; e += kFusedWaves * 64) {
        const int rr = e / ncols;
        const int cc = e - rr * ncols;
        float v[S];
#pragma unroll
        for (int s = 0; s < S; ++s)
            v[s] = ps[(s * 16 + rr) * PS + cc];
        const float hv = __fmul_rn(pairwise_tree<S>(v), p.shrink_scale);
        hs[rr * HS + cc] = hv;
        if (write_h && rr < nrows)
            p.h[(row0 + rr) * p.ld_h + cc] = hv;
    }
    __syncthreads();

    // ---- expand: the same code as lora_expand's ------------------------------
    if (!cols_ok)
        return;
    expand_finish<KS>(L, p.y, p.ld_y, p.N, hs, HS, r, p.expand_scale, yv, bop);
}

template <int RTMAX, int S>
hipError_t launch_s(const FusedParams& p, int waves, dim3 grid, hipStream_t st)
{
    const dim3 block(kFusedWaves * 64);
    switch (waves) {
    case 1: hipLaunchKernelGGL((k_shrink_expand_fused<RTMAX, S, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((k_shrink_expand_fused<RTMAX, S, 2>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((k_shrink_expand_fused<RTMAX, S, 4>), grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL((k_shrink_expand_fused<RTMAX, S, 8>), grid, block, 0, st, p); break;
    }
    return hipGetLastError();
}

template <int RTMAX>
hipError_t launch_rt(const FusedParams& p, int split_k, int waves, dim3 grid, hipStream_t st)
{
    switch (split_k) {
    case 1: return launch_s<RTMAX, 1>(p, waves, grid, st);
    case 2: return launch_s<RTMAX, 2>(p, waves, grid, st);
    case 4: return launch_s<RTMAX, 4>(p, waves, grid, st);
    case 8: return launch_s<RTMAX, 8>(p, waves, grid, st);
    default: return launch_s<RTMAX, 16>(p, waves, grid, st);
    }
}

}  // namespace

int64_t fused_grid(int64_t M, int64_t N)
{
    const int64_t mbs = (M + kRowBlock - 1) / kRowBlock;
    const int64_t nblocks = (N + kFusedCols - 1) / kFusedCols;
    return (mbs >= kXcds ? (mbs + kXcds - 1) / kXcds * kXcds : mbs) * nblocks;
}

hipError_t launch_shrink_expand_fused(const FusedParams& p, int split_k, int waves, hipStream_t st)
{
    if (p.r > kFusedMaxRank)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)fused_grid(p.M, p.N));
    if (p.r > 32)
        return launch_rt<4>(p, split_k, waves, grid, st);
    if (p.r > 16)
        return launch_rt<2>(p, split_k, waves, grid, st);
    return launch_rt<1>(p, split_k, waves, grid, st);
}

}  // namespace lora
