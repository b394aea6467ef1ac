// The Split-K shrink work item shared by the shrink kernels and the
// single-launch shrink + expand: one (16-token row block, split, group of RT
// 16-wide rank tiles) computed by W wavefronts with matrix-core steps, the
// wave results added along a fixed pairwise tree, the split's fp32 partial
// stored, scaled, or atomically added.
#pragma once

#include "device.h"
#include "kernels.h"

namespace lora {

enum ShrinkMode { kToWorkspace = 0, kToOutputScaled = 1, kAtomicScaled = 2, kToWorkspaceCoherent = 3 };

// Agent-scope atomic store / load: performed at the device-wide coherence
// point, past the per-XCD L2 caches (used for the single-launch combine).
__device__ __forceinline__ void store_coherent(float* p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_coherent(const float* p)
{
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Output element (row, col) of the tile: write / atomically add.
template <int MODE>
__device__ __forceinline__ void shrink_store(const ShrinkParams& p, int64_t row0, int s, int row, int col, float v,
                                             float scale)
{
    const int64_t rr = row0 + row;
    if (MODE == kToWorkspace) {
        p.out[(int64_t)s * p.split_stride + rr * p.ld_out + col] = v;
    } else if (MODE == kToWorkspaceCoherent) {
        store_coherent(&p.out[(int64_t)s * p.split_stride + rr * p.ld_out + col], v);
    } else if (MODE == kToOutputScaled) {
        p.out[rr * p.ld_out + col] = __fmul_rn(v, scale);
    } else {
        unsafeAtomicAdd(&p.out[rr * p.ld_out + col], __fmul_rn(v, scale));
    }
}

template <int RT, int W, int MODE>
__device__ __forceinline__ void wave_tree_store(const ShrinkParams& p, int64_t row0, int nrows, uint32_t mask, int rg,
                                                int col0, int s, float scale, float* red, const f32x4 (&acc)[RT]);

// The matrix-core chains of one wave: T row tiles (x row pointers xp[u]) times
// NRT rank tiles (A row pointers ap[rt]), `steps` steps of 32 k from the
// pointers on, each accumulator in ascending k.  Steps go in groups of G with
// all loads of a group issued before its matrix-core steps, without any guard;
// the steps left over after the last full group form one more, smaller group.
// Lanes whose token row or rank column lies outside the tile load from a
// clamped, valid row: matrix-core output (i, j) depends only on row i of the
// first operand and column j of the second, and outputs of such lanes are
// never stored, so no operand needs to be zeroed.
template <bool MASK>
__device__ __forceinline__ bf16x8 operand_load(const uint16_t* p, bool ok)
{
    if constexpr (MASK)
        return ok ? load_bf16x8(p) : bf16x8_zero();
    else
        return load_bf16x8(p);
}

// One group: the loads of steps t .. t + G - 1, then their matrix-core steps.
// MASK: lanes outside the tile skip their loads (fewer addresses for the
// texture units when a tile has few rows, e.g. one decode token); their
// operands are then zeros instead of a clamped row - again never stored.
template <int NRT, int RT, int T, int G, bool MASK>
__device__ __forceinline__ void mfma_group(const uint16_t* const (&xp)[T], const bool (&x_ok)[T],
                                           const uint16_t* const (&ap)[RT], const bool (&a_ok)[RT], int t,
                                           f32x4 (&acc)[T][RT])
{
    bf16x8 xa[G][T];
    bf16x8 b[G][NRT];
#pragma unroll
    for (int q = 0; q < G; ++q) {
        const int off = (t + q) * kKStep;
#pragma unroll
        for (int u = 0; u < T; ++u)
            xa[q][u] = operand_load<MASK>(xp[u] + off, x_ok[u]);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
            b[q][rt] = operand_load<MASK>(ap[rt] + off, a_ok[rt]);
    }
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
        for (int u = 0; u < T; ++u)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
                acc[u][rt] = mfma_16x16x32(xa[q][u], b[q][rt], acc[u][rt]);
}

// KST > 0: the chain length is known at compile time (it must equal
// `steps`), so only the groups it takes are compiled - the same groups, in the
// same order, as the run-time path; these latency-bound kernels run faster
// with less code.
template <int NRT, int RT, int T, int G, bool MASK, int KST = 0>
__device__ __forceinline__ void mfma_chains(const uint16_t* const (&xp)[T], const bool (&x_ok)[T],
                                            const uint16_t* const (&ap)[RT], const bool (&a_ok)[RT], int steps,
                                            f32x4 (&acc)[T][RT])
{
    if constexpr (KST > 0) {
        constexpr int full = KST / G * G;
#pragma unroll
        for (int t = 0; t < full; t += G)
            mfma_group<NRT, RT, T, G, MASK>(xp, x_ok, ap, a_ok, t, acc);
        if constexpr (KST - full > 0)
            mfma_group<NRT, RT, T, KST - full, MASK>(xp, x_ok, ap, a_ok, full, acc);
        return;
    }
    int t = 0;
    for (; t + G <= steps; t += G)
        mfma_group<NRT, RT, T, G, MASK>(xp, x_ok, ap, a_ok, t, acc);
    const int left = steps - t;                   // 0 .. G - 1, uniform
    if constexpr (G >= 4) {
        if (left == 3) {
            mfma_group<NRT, RT, T, 3, MASK>(xp, x_ok, ap, a_ok, t, acc);
            return;
        }
    }
    if constexpr (G >= 3) {
        if (left == 2) {
            mfma_group<NRT, RT, T, 2, MASK>(xp, x_ok, ap, a_ok, t, acc);
            return;
        }
    }
    if (left == 1)
        mfma_group<NRT, RT, T, 1, MASK>(xp, x_ok, ap, a_ok, t, acc);
}

// The chains for nrt (1 .. RT) active rank tiles.
template <int RT, int T, int G, bool MASK, int KST = 0>
__device__ __forceinline__ void mfma_dispatch(int nrt, const uint16_t* const (&xp)[T], const bool (&x_ok)[T],
                                              const uint16_t* const (&ap)[RT], const bool (&a_ok)[RT], int steps,
                                              f32x4 (&acc)[T][RT])
{
    if (nrt >= RT)
        mfma_chains<RT, RT, T, G, MASK, KST>(xp, x_ok, ap, a_ok, steps, acc);
    else if constexpr (RT >= 2) {
        if (nrt == 1)
            mfma_chains<1, RT, T, G, MASK, KST>(xp, x_ok, ap, a_ok, steps, acc);
        else if constexpr (RT >= 3) {
            if (nrt == 2)
                mfma_chains<2, RT, T, G, MASK, KST>(xp, x_ok, ap, a_ok, steps, acc);
            else if constexpr (RT >= 4)
                mfma_chains<3, RT, T, G, MASK, KST>(xp, x_ok, ap, a_ok, steps, acc);
        }
    }
}

// T row tiles (rows row0[u] + i for i < nrows[u] with bit i of mask[u] set;
// a tile with nrows 0 is skipped) that share one adapter, split s and rank
// columns col0 .. col0 + 16 RT - 1 (those below r): every (tile, rank tile)
// accumulator gets its chain over the wave's k range, the A loads shared by
// the T tiles, then the wave tree and the store of the tile's rows.  Per
// element the arithmetic depends only on (K, split_k): the tiles a workgroup
// holds, the rank tiles grouped with it and the other rows of its tile change
// no bit.
template <int RT, int W, int MODE, int T, int KST = 0>
__device__ __forceinline__ void shrink_tiles(const ShrinkParams& p, const int64_t (&row0)[T], const int (&nrows)[T],
                                             const uint32_t (&mask)[T], const uint16_t* __restrict__ A, int r,
                                             int col0, int s, float scale, float* red)
{
    constexpr int G = T == 1 ? 4 : 2;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int g = lane >> 4;
    const int steps = KST > 0 ? KST : p.k_steps;
    const int rg = r - col0;                 // rank columns left from col0

    // Reduction slots 8g..8g+7 of step t hold k = kbase + 32 t + (0..7).
    const int64_t kbase = (int64_t)s * p.k_chunk + (int64_t)wave * steps * kKStep + g * 8;
    const uint16_t* xp[T];
    bool x_ok[T];
    bool full = true;                        // every tile has 16 rows (uniform)
#pragma unroll
    for (int u = 0; u < T; ++u) {
        x_ok[u] = li < nrows[u] && row_in(mask[u], li);
        full = full && ((nrows[u] == kRowBlock && mask[u] == kFullMask) || nrows[u] == 0);
        xp[u] = p.x + (row0[u] + (x_ok[u] ? li : 0)) * p.ld_x + kbase;
    }
    const uint16_t* ap[RT];
    bool a_ok[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int j = rt * 16 + li;
        a_ok[rt] = j < rg;
        ap[rt] = A + (int64_t)(col0 + (a_ok[rt] ? j : 0)) * p.ld_a + kbase;
    }
    f32x4 acc[T][RT];
#pragma unroll
    for (int u = 0; u < T; ++u)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            acc[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // rank tiles with at least one column below r (uniform); masked loads
    // only for a single tile with padding rows or padding rank columns (the
    // several-tile kernels are register-bound and see full tiles almost only)
    const int nrt = (rg + 15) / 16 < RT ? (rg + 15) / 16 : RT;
    if (T > 1 || (full && rg >= 16 * nrt))
        mfma_dispatch<RT, T, G, false, KST>(nrt, xp, x_ok, ap, a_ok, steps, acc);
    else if constexpr (T == 1)
        mfma_dispatch<RT, T, G, true, KST>(nrt, xp, x_ok, ap, a_ok, steps, acc);
#pragma unroll
    for (int u = 0; u < T; ++u)
        if (nrows[u] > 0)                         // uniform across the workgroup
            wave_tree_store<RT, W, MODE>(p, row0[u], nrows[u], mask[u], rg, col0, s, scale, red, acc[u]);
}

// One work item: rows row0 .. row0+nrows-1 (those in mask), split s, rank
// columns col0 .. col0 + 16 RT - 1 (those below r).  A is the adapter's row 0.
template <int RT, int W, int MODE, int KST = 0>
__device__ __forceinline__ void shrink_tile(const ShrinkParams& p, int64_t row0, int nrows, uint32_t mask,
                                            const uint16_t* __restrict__ A, int r, int col0, int s, float scale,
                                            float* red)
{
    const int64_t rows[1] = {row0};
    const int n[1] = {nrows};
    const uint32_t m[1] = {mask};
    shrink_tiles<RT, W, MODE, 1, KST>(p, rows, n, m, A, r, col0, s, scale, red);
}

// acc[rt][v] is the wave's sum for token row 4g+v, rank column col0 + 16 rt + li:
// with W waves, the W wave sums meet in LDS and are added along the fixed
// pairwise tree; then the split's partial is stored.
template <int RT, int W, int MODE>
__device__ __forceinline__ void wave_tree_store(const ShrinkParams& p, int64_t row0, int nrows, uint32_t mask, int rg,
                                                int col0, int s, float scale, float* red, const f32x4 (&acc)[RT])
{
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int g = lane >> 4;
    if constexpr (W == 1) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 4 * g + v, col = rt * 16 + li;
                if (row < nrows && row_in(mask, row) && col < rg)
                    shrink_store<MODE>(p, row0, s, row, col0 + col, acc[rt][v], scale);
            }
    } else {
        constexpr int RS = 16 * RT + 4;          // padded LDS row stride (floats)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[(wave * 16 + 4 * g + v) * RS + rt * 16 + li] = acc[rt][v];
        __syncthreads();
        const int ncols = rg < 16 * RT ? rg : 16 * RT;
        for (int e = threadIdx.x; e < 16 * 16 * RT; e += W * kWave) {
            const int row = e / (16 * RT);
            const int col = e - row * (16 * RT);
            if (row < nrows && row_in(mask, row) && col < ncols) {
                float v[W];
#pragma unroll
                for (int w = 0; w < W; ++w)
                    v[w] = red[(w * 16 + row) * RS + col];
                shrink_store<MODE>(p, row0, s, row, col0 + col, pairwise_tree<W>(v), scale);
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

// Fixed pairwise tree over the S workspace slices of one element, read with
// agent-scope loads (the slices may have been written by other XCDs during
// the same launch).
template <int S>
__device__ __forceinline__ float tree_of_splits(const float* w, int64_t split_stride)
{
    float v[S];
#pragma unroll
    for (int s = 0; s < S; ++s)
        v[s] = load_coherent(w + (int64_t)s * split_stride);
    return pairwise_tree<S>(v);
}

// The same for a split count known at run time (1, 2, 4, 8 or 16).
__device__ __forceinline__ float split_tree(const float* w, int64_t split_stride, int split_k)
{
    switch (split_k) {
    case 1: return tree_of_splits<1>(w, split_stride);
    case 2: return tree_of_splits<2>(w, split_stride);
    case 4: return tree_of_splits<4>(w, split_stride);
    case 8: return tree_of_splits<8>(w, split_stride);
    default: return tree_of_splits<16>(w, split_stride);
    }
}

}  // namespace lora
