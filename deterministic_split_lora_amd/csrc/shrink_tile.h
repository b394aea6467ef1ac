// The Split-K shrink work item shared by the shrink kernels and the
// single-launch shrink + expand: one (16-token row block, split, group of RT
// 16-wide rank tiles) computed by W wavefronts with matrix-core steps, the
// wave results added along a fixed pairwise tree, the split's fp32 partial
// stored, scaled, or atomically added.
#pragma once

#include "device.h"
#include "kernels.h"

namespace lora {

enum ShrinkMode {
    kToWorkspace = 0,
    kToOutputScaled = 1,
    kAtomicScaled = 2,
    kToWorkspaceCoherent = 3,
    kToLds = 4                              // the split's partial into an LDS tile (single-launch combine)
};

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
                                                int col0, int s, float scale, float* red, const f32x4 (&acc)[RT],
                                                float* own);

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
// MODE kToLds: tile u's partial goes to own[(u * 16 + row) * 16 RT + column -
// col0] instead of memory.
template <int RT, int W, int MODE, int T, int KST = 0>
__device__ __forceinline__ void shrink_tiles(const ShrinkParams& p, const int64_t (&row0)[T], const int (&nrows)[T],
                                             const uint32_t (&mask)[T], const uint16_t* __restrict__ A, int r,
                                             int col0, int s, float scale, float* red, float* own = nullptr)
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
            wave_tree_store<RT, W, MODE>(p, row0[u], nrows[u], mask[u], rg, col0, s, scale, red, acc[u],
                                         MODE == kToLds ? own + u * 16 * 16 * RT : nullptr);
}

// One work item: rows row0 .. row0+nrows-1 (those in mask), split s, rank
// columns col0 .. col0 + 16 RT - 1 (those below r).  A is the adapter's row 0.
template <int RT, int W, int MODE, int KST = 0>
__device__ __forceinline__ void shrink_tile(const ShrinkParams& p, int64_t row0, int nrows, uint32_t mask,
                                            const uint16_t* __restrict__ A, int r, int col0, int s, float scale,
                                            float* red, float* own = nullptr)
{
    const int64_t rows[1] = {row0};
    const int n[1] = {nrows};
    const uint32_t m[1] = {mask};
    shrink_tiles<RT, W, MODE, 1, KST>(p, rows, n, m, A, r, col0, s, scale, red, own);
}

// acc[rt][v] is the wave's sum for token row 4g+v, rank column col0 + 16 rt + li:
// with W waves, the W wave sums meet in LDS and are added along the fixed
// pairwise tree; then the split's partial is stored.
template <int RT, int W, int MODE>
__device__ __forceinline__ void wave_tree_store(const ShrinkParams& p, int64_t row0, int nrows, uint32_t mask, int rg,
                                                int col0, int s, float scale, float* red, const f32x4 (&acc)[RT],
                                                float* own)
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
                if (row < nrows && row_in(mask, row) && col < rg) {
                    if constexpr (MODE == kToLds)
                        own[row * 16 * RT + col] = acc[rt][v];
                    else
                        shrink_store<MODE>(p, row0, s, row, col0 + col, acc[rt][v], scale);
                }
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
                if constexpr (MODE == kToLds)
                    own[e] = pairwise_tree<W>(v);
                else
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

// ---------------------------------------------------------------------------
// Tagged workspace slots of the single-launch shrinks.  A slot is one 64-bit
// word: the fp32 partial in the low half and a tag in the high half (1: this
// call's partial, 0: consumed).  Slots are written and read only with
// agent-scope atomic stores and loads of the whole word, so a reader that
// sees the tag 1 sees the partial stored with it (single-copy atomicity of an
// aligned 64-bit atomic), and by per-location coherence it eventually sees
// the store, whichever XCD made it.  No ordering between different
// locations is needed - no release or acquire, hence no L2 write-back or
// invalidate - because every slot carries its own evidence of being written.
// The combining workgroup clears each slot it consumed; the kernel boundary
// orders those clears before the next call's stores.
// ---------------------------------------------------------------------------
constexpr uint32_t kSlotWritten = 1u;
// Polls per slot before a reader gives up (each a memory round trip: about a
// quarter of a second in all).  A writer that has made its arrival add is
// resident and finishes its item without waiting for anyone, and the reader
// started last, so no correct launch comes near this.
constexpr uint32_t kSlotSpinLimit = 1u << 18;

__device__ __forceinline__ void slot_store(uint64_t* slot, float v)
{
    const uint64_t w = ((uint64_t)kSlotWritten << 32) | (uint64_t)__builtin_bit_cast(uint32_t, v);
    __hip_atomic_store(slot, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t slot_load(uint64_t* slot)
{
    return __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void slot_clear(uint64_t* slot)
{
    __hip_atomic_store(slot, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool slot_written(uint64_t w)
{
    return (uint32_t)(w >> 32) == kSlotWritten;
}

__device__ __forceinline__ float slot_value(uint64_t w)
{
    return __builtin_bit_cast(float, (uint32_t)w);
}

// Fixed pairwise tree over the S partials of one element: split s_own's from
// `own` (the combining workgroup's own partial, never stored), the others
// from their tagged slots w[s * stride], each read until written and then
// cleared.  False (and the slots left as they are) if a slot never showed
// its partial.
// Slots are polled in groups of GMAX (4 or 8): each poll loads the group's
// missing slots at once.  Fewer loads in flight per thread keep the register
// count, and with it the occupancy, close to the two-pass partial kernel's;
// more cut the round trips of the last workgroup.
template <int S, int GMAX>
__device__ __forceinline__ bool tagged_tree(uint64_t* w, int64_t stride, int s_own, float own, float& out)
{
    constexpr int G = S < GMAX ? S : GMAX;
    float v[S];
#pragma unroll
    for (int g0 = 0; g0 < S; g0 += G) {
        const int d = s_own - g0;
        uint32_t pending = ((1u << G) - 1u) & ~((unsigned)d < (unsigned)G ? 1u << d : 0u);
        for (uint32_t n = 0; pending != 0u && n < kSlotSpinLimit; ++n) {
            if (n > 0)
                __builtin_amdgcn_s_sleep(2);
            uint64_t t[G];
#pragma unroll
            for (int q = 0; q < G; ++q)
                t[q] = ((pending >> q) & 1u) ? slot_load(w + (int64_t)(g0 + q) * stride) : 0;
#pragma unroll
            for (int q = 0; q < G; ++q)
                if (((pending >> q) & 1u) && slot_written(t[q])) {
                    v[g0 + q] = slot_value(t[q]);
                    pending &= ~(1u << q);
                }
        }
        if (pending != 0u)
            return false;
    }
    // the own split's slot was not written in this call and still reads 0,
    // so clearing it too changes nothing
#pragma unroll
    for (int s = 0; s < S; ++s) {
        v[s] = s == s_own ? own : v[s];
        slot_clear(w + (int64_t)s * stride);
    }
    out = pairwise_tree<S>(v);
    return true;
}

// Sixteen splits as two trees of eight added at the end - the same sum as
// the 16-way pairwise tree, whose top level is exactly that add - so that no
// thread holds more than eight partials.
template <int GMAX>
__device__ __forceinline__ bool tagged_split_tree(uint64_t* w, int64_t stride, int split_k, int s_own, float own,
                                                  float& out)
{
    switch (split_k) {
    case 1: out = own; return true;
    case 2: return tagged_tree<2, GMAX>(w, stride, s_own, own, out);
    case 4: return tagged_tree<4, GMAX>(w, stride, s_own, own, out);
    case 8: return tagged_tree<8, GMAX>(w, stride, s_own, own, out);
    default: {
        float lo, hi;
        if (!tagged_tree<8, GMAX>(w, stride, s_own, own, lo) ||
            !tagged_tree<8, GMAX>(w + 8 * stride, stride, s_own - 8, own, hi))
            return false;
        out = __fadd_rn(lo, hi);
        return true;
    }
    }
}

// After shrink_tile<kToLds>: the tile's rows row0 + i (i < nrows, in mask) and
// columns [c0, c_data) are in own[i * 16 RT + column - c0].  A workgroup that
// did not arrive last stores them to its split's tagged slots
// (ws[s * split_stride + row * ld_out + column], 64-bit words); the last one
// evaluates h = scale * tree over the S partials for those columns and writes
// zeros for columns [c_data, c_zero).  A slot that never shows its partial
// (no correct launch) gives NaN in h.
template <int RT, int GMAX>
__device__ __forceinline__ void tagged_finish(const ShrinkParams& p, int64_t row0, int nrows, uint32_t mask, int c0,
                                              int c_data, int c_zero, int s, bool last, float scale,
                                              const float* own, float* h, int64_t ld_h)
{
    uint64_t* ws = reinterpret_cast<uint64_t*>(p.out);
    if (!last) {
        const int ncols = c_data - c0;
        for (int e = threadIdx.x; e < nrows * ncols; e += blockDim.x) {
            const int row = e / ncols;
            const int col = e - row * ncols;
            if (row_in(mask, row))
                slot_store(ws + (int64_t)s * p.split_stride + (row0 + row) * p.ld_out + c0 + col,
                           own[row * 16 * RT + col]);
        }
        return;
    }
    const int ncols = c_zero - c0;
    for (int e = threadIdx.x; e < nrows * ncols; e += blockDim.x) {
        const int row = e / ncols;
        if (!row_in(mask, row))
            continue;
        const int col = c0 + (e - row * ncols);
        float val = 0.0f;
        if (col < c_data) {
            float t;
            if (tagged_split_tree<GMAX>(ws + (row0 + row) * p.ld_out + col, p.split_stride, p.split_k, s,
                                  own[row * 16 * RT + col - c0], t))
                val = __fmul_rn(t, scale);
            else
                val = __builtin_nanf("");
        }
        h[(row0 + row) * ld_h + col] = val;
    }
}

}  // namespace lora
