// Split-K LoRA shrink kernels for gfx950.
//
// The shrink h = x A^T (paper Eq. 1) is a narrow GEMM: K = hidden size is long,
// r <= 128 is short.  Split-K (section 2.1, Eq. 3) cuts K into S contiguous
// chunks so S workgroups share one output tile.  A workgroup owns one
// (16-token row block, split, group of RT 16-wide rank tiles) and W
// wavefronts; wave w walks k_steps * 32 consecutive k of the split's chunk
// with matrix-core steps, the bf16 operands streamed straight from HBM into
// registers with 16-byte loads (x rows and A rows are both k-contiguous, which
// is exactly the per-lane operand layout, so no LDS transpose is needed).  The
// W wave results meet in LDS and are added along a fixed pairwise tree.  The
// split's fp32 partial then goes to the workspace (deterministic paths),
// straight to h (split_k == 1), or is atomically added to h (the
// nondeterministic contrast of section 4.1).
//
// Every element's arithmetic - which k each matrix-core step covers, the step
// order, the wave tree, the split tree - is fixed by (K, split_k) alone, and
// each rank column's chain is independent of the others, so neither M, a
// token's neighbours, nor how rank tiles are grouped into workgroups changes a
// single bit.  Small calls spread their rank tiles over more workgroups (more
// memory parallelism); large calls keep them together (x is read once).
#include "device.h"
#include "kernels.h"
#include "shrink_tile.h"

namespace lora {

namespace {

// ---------------------------------------------------------------------------
// Single-launch combine (the completion-counter protocol of the paper's
// section 4.3 / Alg. 1, with the pairwise tree of the two-pass path as the
// fixed order).
//
// The XCDs of an MI355X each have their own L2, so a partial written by one
// workgroup must reach the device-wide coherence point before a workgroup on
// another XCD reads it.  Ordering the partial stores before an arrival
// counter would take a release at agent scope, which on gfx950 writes back
// the XCD's L2 (buffer_wbl2) once per arriving workgroup; those write-backs
// queue per XCD and made the multi-adapter single launch ~4x slower than the
// two passes.  Instead each partial travels in a tagged 64-bit slot
// (tagged_tree): the reader checks every slot's own tag, so nothing but
// per-location coherence is needed.
//
// Every workgroup of a (row block or plan tile, rank group) makes one relaxed
// integer add to its counter when it STARTS the item; the add's result comes
// back while the workgroup streams its operands.  The one whose add returned
// split_k - 1 started last (its add also put the counter back to 0): it keeps
// its own partial in LDS and waits for the other split_k - 1 slots.  Those belong to workgroups
// that already made their add, so they are resident and finish their item
// without waiting for anyone; the wait always ends.  The floating-point sum
// has one fixed order whichever workgroup combines.
// ---------------------------------------------------------------------------
// The arrival is a wrapping increment (old >= split_k - 1 ? 0 : old + 1),
// so the add that returns split_k - 1 also puts the counter back to 0 for the
// next call.  (An integer fetch-add here is rewritten by the compiler into a
// wave-wide add whose result it waits for at once; the increment's result is
// waited for only where it is used, after the partial.)
__device__ __forceinline__ int arrival_add(int32_t* counter, int split_k)
{
    return (int)__builtin_amdgcn_atomic_inc32(reinterpret_cast<uint32_t*>(counter), (uint32_t)(split_k - 1),
                                              __ATOMIC_RELAXED, "agent");
}

// ---------------------------------------------------------------------------
// Single adapter.  A 1-D grid of (row block, rank group, split) items with the
// split index fastest.  Consecutive workgroup ids go to different XCDs, so
// this order makes the XCDs stream adjacent pieces of the same rows at the
// same time; measured on MI355X, it reads the same bytes ~25% faster than
// the row-block-fastest order (which leaves each XCD a strided subset).
// ---------------------------------------------------------------------------
struct SingleItem {
    int64_t row0;
    int nrows;
    int s;
    int grp;
    int64_t mb;
};

__device__ __forceinline__ SingleItem single_item(const ShrinkParams& p, int groups)
{
    SingleItem q;                                 // 32-bit: the grid is below 2^31
    const uint32_t bid = blockIdx.x;
    const uint32_t S = (uint32_t)p.split_k;
    q.s = (int)(bid % S);
    const uint32_t rest = bid / S;
    q.grp = (int)(rest % (uint32_t)groups);
    q.mb = rest / (uint32_t)groups;
    q.row0 = q.mb * kRowBlock;
    const int64_t left = p.M - q.row0;
    q.nrows = left < kRowBlock ? (int)left : kRowBlock;
    return q;
}

// KST: the wave chain length when it is 1, 2 or 4 (0: read from p.k_steps).
template <int RT, int W, int MODE, int KST>
__global__ __launch_bounds__(W * 64) void k_shrink_partial(ShrinkParams p, int groups)
{
    __shared__ float red[red_floats<RT, W>()];
    const SingleItem q = single_item(p, groups);
    shrink_tile<RT, W, MODE, KST>(p, q.row0, q.nrows, kFullMask, p.A, p.r, q.grp * 16 * RT, q.s, p.scale, red);
}

// Large M: T consecutive row blocks per workgroup, all rank tiles together,
// split index fastest in the 1-D grid.  The row blocks share the A loads (see
// shrink_tiles); partials and their bits are those of k_shrink_partial.
// Two 8-wave workgroups per compute unit (4 waves per SIMD, <= 128 VGPRs):
// one workgroup's loads are in flight while the other runs its trees.
template <int RT, int W, int T, int MODE>
__global__ __launch_bounds__(W * 64, 4) void k_shrink_partial_multi(ShrinkParams p)
{
    __shared__ float red[red_floats<RT, W>()];
    const uint32_t S = (uint32_t)p.split_k;
    const int s = (int)(blockIdx.x % S);
    const int64_t first = (int64_t)(blockIdx.x / S) * T * kRowBlock;
    int64_t row0[T];
    int nrows[T];
    uint32_t mask[T];
#pragma unroll
    for (int u = 0; u < T; ++u) {
        const int64_t r0 = first + (int64_t)u * kRowBlock;
        const int64_t left = p.M - r0;
        nrows[u] = left <= 0 ? 0 : (left < kRowBlock ? (int)left : kRowBlock);
        row0[u] = nrows[u] > 0 ? r0 : first;      // empty tiles keep a valid base address
        mask[u] = kFullMask;
    }
    shrink_tiles<RT, W, MODE, T>(p, row0, nrows, mask, p.A, p.r, 0, s, MODE == kAtomicScaled ? p.scale : 1.0f,
                                 red);
}

// Single launch: the split that starts last in each (row block, rank group)
// writes h.  Occupancy hint as for k_sgmv_shrink_counted.
template <int RT, int W, int KST>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(RT == 1 && KST > 0 && W >= 4 ? 8 : 1, 8)))
void k_shrink_counted(ShrinkParams p, CounterParams c, int groups)
{
    __shared__ float red[red_floats<RT, W>()];
    __shared__ float own[16 * 16 * RT];
    __shared__ int flag;
    const SingleItem q = single_item(p, groups);
    const int col0 = q.grp * 16 * RT;
    int32_t* counter = c.counters + q.mb * kMaxRankTiles + q.grp;
    int arrived = 0;
    if (threadIdx.x == 0)
        arrived = arrival_add(counter, p.split_k);
    shrink_tile<RT, W, kToLds, KST>(p, q.row0, q.nrows, kFullMask, p.A, p.r, col0, q.s, 1.0f, red, own);
    if (threadIdx.x == 0)
        flag = arrived;
    __syncthreads();
    const bool last = flag == p.split_k - 1;
    const int cend = col0 + 16 * RT < p.r ? col0 + 16 * RT : p.r;
    tagged_finish<RT, 8>(p, q.row0, q.nrows, kFullMask, col0, cend, cend, q.s, last, p.scale, own, c.h, c.ld_h);
}

// ---------------------------------------------------------------------------
// Multi-adapter.  A fixed grid walks the plan's (tile, split, rank group)
// items with a static stride; every wave of a workgroup sees the same item
// count and leaves the loop together.  Items of rank groups beyond the tile's
// adapter rank are skipped.
// ---------------------------------------------------------------------------
// A plan tile entry (wave-uniform) through the scalar cache (table_load): in
// the single-launch kernels a vector load's wait would also wait for the
// arrival add issued before the first operand load.
__device__ __forceinline__ PlanInts plan_entry(const int32_t* e)
{
    return PlanInts{{table_load(e, 0), table_load(e, 1), table_load(e, 2), table_load(e, 3)}};
}

struct SgmvItem {
    int64_t row0;
    int nrows;
    uint32_t mask;   // the tile's rows among row0 .. row0 + nrows - 1
    int a;           // adapter, -1 for tokens without one
    int s;
    int grp;
    int tile;
    bool ok;         // rows inside [0, M), adapter -1 or valid
};

__device__ __forceinline__ SgmvItem sgmv_item(const ShrinkParams& p, uint32_t it, int groups)
{
    SgmvItem q;                                   // order: tile, rank group, split (fastest)
    const uint32_t S = (uint32_t)p.split_k;
    q.s = (int)(it % S);
    const uint32_t rest = it / S;
    q.grp = (int)(rest % (uint32_t)groups);
    q.tile = (int)(rest / (uint32_t)groups);
    const PlanInts e = plan_entry(p.tiles + kPlanHeaderInts + kPlanTileInts * q.tile);
    const int32_t* t = e.v;
    q.ok = tile_rows_ok(t, p.M) & (t[2] >= -1) & (t[2] < p.n_adapters);
    q.row0 = t[0];
    q.nrows = t[1];
    q.mask = q.ok ? tile_mask(t) : 0u;
    q.a = t[2];
    return q;
}

__device__ __forceinline__ const uint16_t* adapter_weights(const ShrinkParams& p, int a)
{
    return table_load(p.A_ptrs, a);
}

__device__ __forceinline__ int adapter_rank(const ShrinkParams& p, int a)
{
    int ra = table_load(p.ranks, a);
    return ra < 0 ? 0 : (ra > p.r_max ? p.r_max : ra);
}

// The factor a split's partial is multiplied by before it leaves the
// workgroup: 1 into the workspace, the adapter's shrink scale for the atomic
// contrast's direct adds into h.
template <int MODE>
__device__ __forceinline__ float sgmv_item_scale(const ShrinkParams& p, int a)
{
    if constexpr (MODE == kAtomicScaled)
        return p.scales ? table_load(p.scales, a) : 1.0f;
    else
        return 1.0f;
}

template <int RT, int W, int MODE, int KST>
__global__ __launch_bounds__(W * 64) void k_sgmv_shrink_partial(ShrinkParams p)
{
    __shared__ float red[red_floats<RT, W>()];
    const int groups = (p.r_max + 16 * RT - 1) / (16 * RT);
    const uint32_t items = (uint32_t)plan_tiles(p.tiles, p.M, p.n_adapters) * p.split_k * groups;
    for (uint32_t it = blockIdx.x; it < items; it += gridDim.x) {
        const SgmvItem q = sgmv_item(p, it, groups);
        if (!q.ok || q.a < 0)                     // uniform across the workgroup
            continue;
        // the adapter's weight pointer is read together with its rank, not
        // after the rank test (one dependent round trip less per item)
        const uint16_t* Aa = adapter_weights(p, q.a);
        const int ra = adapter_rank(p, q.a);
        const int col0 = q.grp * 16 * RT;
        if (col0 >= ra)
            continue;
        shrink_tile<RT, W, MODE, KST>(p, q.row0, q.nrows, q.mask, Aa, ra, col0, q.s, sgmv_item_scale<MODE>(p, q.a),
                                      red);
    }
}

// Large M: items are (chunk of T consecutive plan tiles, split), split
// fastest; in a chunk, each stretch of consecutive tiles with one adapter
// goes through shrink_tiles together (tiles of one adapter are consecutive
// in the plan, so a chunk is usually one stretch).  All rank tiles of r_max
// in one workgroup.  Same partials, same bits as k_sgmv_shrink_partial.
template <int RT, int W, int T, int MODE>
__global__ __launch_bounds__(W * 64, 4) void k_sgmv_shrink_partial_multi(ShrinkParams p)
{
    __shared__ float red[red_floats<RT, W>()];
    const int ntiles = plan_tiles(p.tiles, p.M, p.n_adapters);
    const uint32_t S = (uint32_t)p.split_k;
    const uint32_t items = (uint32_t)((ntiles + T - 1) / T) * S;
    const int32_t* plan = p.tiles + kPlanHeaderInts;
    for (uint32_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int s = (int)(it % S);
        const int c0 = (int)(it / S) * T;
        const int c1 = c0 + T < ntiles ? c0 + T : ntiles;
        int j = c0;
        while (j < c1) {                          // uniform: plan data only
            const PlanInts et = plan_entry(plan + kPlanTileInts * j);
            const int32_t* t = et.v;
            if (!tile_ok(t, p.M, p.n_adapters)) {
                ++j;
                continue;
            }
            const int a = t[2];
            int64_t row0[T];
            int nrows[T];
            uint32_t mask[T];
            int n = 0;
#pragma unroll
            for (int u = 0; u < T; ++u) {
                PlanInts eu{{0, 0, -1, 0}};
                if (j + u < c1)
                    eu = plan_entry(plan + kPlanTileInts * (j + u));
                const int32_t* tu = eu.v;
                const bool take = n == u && j + u < c1 && tile_ok(tu, p.M, p.n_adapters) && tu[2] == a;
                row0[u] = take ? tu[0] : t[0];
                nrows[u] = take ? tu[1] : 0;
                mask[u] = take ? tile_mask(tu) : 0u;
                n += take ? 1 : 0;
            }
            const uint16_t* Aa = adapter_weights(p, a);  // with the rank, not after its test
            const int ra = adapter_rank(p, a);
                if (ra > 0)
                shrink_tiles<RT, W, MODE, T>(p, row0, nrows, mask, Aa, ra, 0, s, sgmv_item_scale<MODE>(p, a), red);
            j += n;
        }
    }
}

// ---------------------------------------------------------------------------
// Large M with short wave chains (the 16 RT rank rows x k_steps operands of a
// wave's k range fit in 32 registers): a workgroup takes one split and R
// consecutive row blocks (plan tiles for the multi-adapter shrink).  Each wave
// loads its k range of the adapter's A once - again only when the adapter
// changes - and keeps it in registers while it walks the row blocks; the x
// operands of a block are loaded two blocks ahead; the wave sums of a block
// meet in LDS (two buffers, one barrier per block) and are added along the
// fixed pairwise tree while the other waves run the next block's
// matrix-core steps.  Per element this is the arithmetic of shrink_tiles: the
// same chains in the same k order, the same wave tree, the same partial
// stored to the workspace.  What changes is the traffic: A is read once per
// workgroup instead of once per few row blocks.
// ---------------------------------------------------------------------------
template <int RT, int W, int STEPS, bool SGMV, int MODE>
__global__ __launch_bounds__(W * 64, 2) void k_shrink_stream(ShrinkParams p, int R)
{
    // x buffers in rotation: blocks are loaded NB - 1 = 2 ahead (measured on
    // MI355X: loading 3 ahead makes the 4096 x 8192 multi-adapter partials no
    // faster)
    constexpr int NB = 3;
    constexpr int RS = 16 * RT + 4;               // padded LDS row stride (floats)
    __shared__ __align__(16) float red[2][W * 16 * RS];
    __shared__ int32_t tl[kPlanTileInts * kStreamMaxRows];   // the item's plan entries
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int g = lane >> 4;
    const int32_t* plan = p.tiles + kPlanHeaderInts;
    const int64_t ntiles = SGMV ? plan_tiles(p.tiles, p.M, p.n_adapters) : (p.M + kRowBlock - 1) / kRowBlock;
    const uint32_t S = (uint32_t)p.split_k;
    const uint32_t items = (uint32_t)((ntiles + R - 1) / R) * S;
    // tile j (the item's u-th): first row, row span (0: nothing to compute),
    // adapter and row mask; plan entries come from LDS, checked once when the
    // item's entries are staged, so reading them never waits for the x loads
    // in flight and costs no scalar work per block
    auto tile = [&](int64_t j, int u, int64_t& row0, int& nrows, int& a, uint32_t& msk) {
        if constexpr (SGMV) {
            // uniform by construction: scalar registers
            row0 = __builtin_amdgcn_readfirstlane(tl[kPlanTileInts * u]);
            nrows = __builtin_amdgcn_readfirstlane(tl[kPlanTileInts * u + 1]);
            a = __builtin_amdgcn_readfirstlane(tl[kPlanTileInts * u + 2]);
            msk = (uint32_t)__builtin_amdgcn_readfirstlane(tl[kPlanTileInts * u + 3]);
        } else {
            row0 = j * kRowBlock;
            nrows = p.M - row0 < kRowBlock ? (int)(p.M - row0) : kRowBlock;
            a = 0;
            msk = kFullMask;
        }
    };
    // this thread's elements of a block's 16 x 16 RT partial tile: row, column
    // and byte offset inside the block's workspace rows (erow = 16 for the
    // threads left over: never stored).  The offsets are computed once and the
    // block's base goes into scalar registers, so the per-block stores need no
    // fresh address registers (with addresses recomputed each block, the
    // compiled loop waited for all loads in flight more often).
    constexpr int EPT = (16 * 16 * RT + W * kWave - 1) / (W * kWave);
    int erow[EPT], ecol[EPT];
    uint32_t voff[EPT];
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = (int)threadIdx.x + q * W * kWave;
        erow[q] = e < 16 * 16 * RT ? e / (16 * RT) : 16;
        ecol[q] = e % (16 * RT);
        voff[q] = (uint32_t)((erow[q] * p.ld_out + ecol[q]) * 4);
    }
    // registers of the values stored by the NB unrolled blocks (see block)
    float kept[NB][EPT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < EPT; ++q)
            kept[b][q] = 0.0f;
    uint32_t k = 0;                               // blocks walked: selects the LDS buffer
    for (uint32_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int s = (int)(it % S);
        const int64_t c0 = (int64_t)(it / S) * R;
        const int cnt = ntiles - c0 < R ? (int)(ntiles - c0) : R;
        if constexpr (SGMV) {
            __syncthreads();                      // the previous item's entries are no longer read
            if ((int)threadIdx.x < cnt) {         // one tile per thread, checked and normalised
                const PlanInts e = load_plan_ints(plan + kPlanTileInts * (c0 + threadIdx.x));
                const int32_t* t = e.v;
                const bool ok = tile_ok(t, p.M, p.n_adapters);
                int32_t* d = tl + kPlanTileInts * threadIdx.x;
                d[0] = ok ? t[0] : 0;
                d[1] = ok ? t[1] : 0;
                d[2] = ok ? t[2] : -1;
                d[3] = ok ? (int32_t)tile_mask(t) : 0;
            }
            __syncthreads();
        }
        // reduction slots 8g..8g+7 of step t hold k = kbase + 32 t + (0..7)
        const int64_t kbase = (int64_t)s * p.k_chunk + (int64_t)wave * STEPS * kKStep + g * 8;
        auto xload = [&](int u, u32x4 (&dst)[STEPS]) {
            int64_t row0;
            int nrows, a;
            uint32_t msk;
            tile(c0 + u, u, row0, nrows, a, msk);
            const uint16_t* xp = p.x + (row0 + (li < nrows ? li : 0)) * p.ld_x + kbase;
#pragma unroll
            for (int t = 0; t < STEPS; ++t)
                dst[t] = *(const global_u32x4*)(xp + t * kKStep);
        };
        // x operands held as raw 32-bit words until the matrix-core step: moves
        // of 8 x bf16 vectors between registers compiled to per-half shuffles
        u32x4 xb[NB][STEPS];
        bf16x8 aop[STEPS][RT];
        // runs of blocks with one adapter: the run's first two x blocks and
        // its A chunk are loaded at the start of the run and waited for there,
        // so the loop over the run's blocks waits only for the x operands it
        // is about to use
        int u = 0;
        while (u < cnt) {
            int64_t row0;
            int nrows, a;
            uint32_t msk;
            tile(c0 + u, u, row0, nrows, a, msk); // uniform: plan data only
            int u1 = u + 1;
            if constexpr (SGMV) {
                while (u1 < cnt) {
                    int64_t r1;
                    int n1, a1;
                    uint32_t m1;
                    tile(c0 + u1, u1, r1, n1, a1, m1);
                    if (a1 != a)
                        break;
                    ++u1;
                }
            } else {
                u1 = cnt;
            }
            // the weight pointer with the rank, not after the rank test
            const uint16_t* A = SGMV ? (a < 0 ? nullptr : adapter_weights(p, a)) : p.A;
            const int ra = a < 0 ? 0 : (SGMV ? adapter_rank(p, a) : p.r);
            const int nrt = (ra + 15) / 16 < RT ? (ra + 15) / 16 : RT;
            // the atomic contrast's factor for the run (loaded once per run)
            const float run_sc = MODE != kAtomicScaled || ra == 0 ? 1.0f
                                 : (SGMV ? sgmv_item_scale<MODE>(p, a) : p.scale);
#pragma unroll
            for (int q = 0; q + 1 < NB; ++q)
                xload(u + q < u1 ? u + q : u1 - 1, xb[q]);
            if (ra > 0) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    if (rt < nrt) {
                        const int j = rt * 16 + li;
                        const uint16_t* ap = A + (int64_t)(j < ra ? j : 0) * p.ld_a + kbase;
#pragma unroll
                        for (int t = 0; t < STEPS; ++t)
                            aop[t][rt] = load_bf16x8(ap + t * kKStep);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            // the run's i-th block uses buffer i % NB and loads block
            // i + NB - 1 into buffer (i + NB - 1) % NB (loop unrolled by NB:
            // no register is copied while its load is in flight).  The matrix-core steps run
            // on every path - also for rank tiles past the adapter's rank and
            // for blocks without rows, whose results are never stored - so
            // that every buffer is known to have landed once its block is
            // done and its registers can be reused without draining the
            // loads in flight.
            auto block = [&](const u32x4 (&xc)[STEPS], u32x4 (&xn)[STEPS], float (&kept)[EPT]) {
                xload(u + NB - 1 < u1 ? u + NB - 1 : u1 - 1, xn);   // unconditional: no branch-dependent buffer
                tile(c0 + u, u, row0, nrows, a, msk);
                const bool on = nrows > 0 && ra > 0;
                float* rb = red[k & 1];
                f32x4 acc[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 0; t < STEPS; ++t)
                        acc[rt] = mfma_16x16x32(__builtin_bit_cast(bf16x8, xc[t]), aop[t][rt], acc[rt]);
                }
                if (on) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            rb[(wave * 16 + 4 * g + v) * RS + rt * 16 + li] = acc[rt][v];
                }
                __syncthreads();
                if (on) {
                    const int ncols = ra < 16 * RT ? ra : 16 * RT;
                    // the block's 16 workspace rows, addressed from scalar
                    // registers; the per-lane offsets never change
                    const BufferRsrc ws = buffer_rsrc(p.out + (int64_t)s * p.split_stride + row0 * p.ld_out,
                                                      (uint32_t)(16 * p.ld_out * 4));
#pragma unroll
                    for (int q = 0; q < EPT; ++q) {
                        const bool mine = erow[q] < nrows && row_in(msk, erow[q]) && ecol[q] < ncols;
                        float val = 0.0f;
                        if (mine) {
                            float v[W];
#pragma unroll
                            for (int w = 0; w < W; ++w)
                                v[w] = rb[(w * 16 + erow[q]) * RS + ecol[q]];
                            val = pairwise_tree<W>(v);
                            if constexpr (MODE == kAtomicScaled)
                                val = __fmul_rn(val, run_sc);
                        }
                        // the value this slot stored NB blocks ago stays
                        // in its register until here, so no later
                        // instruction of the loop overwrites a register a
                        // recent store still reads; the new one is stored
                        // from the register it then keeps (the empty asm
                        // statements pin both)
                        asm volatile("" : "+v"(kept[q]));
                        kept[q] = val;
                        asm volatile("" : "+v"(kept[q]));
                        if (mine) {
                            if constexpr (MODE == kAtomicScaled)
                                buffer_atomic_add_f32(kept[q], ws, voff[q]);
                            else
                                buffer_store_f32(kept[q], ws, voff[q]);
                        }
                    }
                }
            };
            // whole rounds of NB blocks, then the run's last blocks: the loop
            // is entered again only after all NB blocks of a round, so the
            // compiled waits at its head know which loads are in flight (a
            // round that may stop after any block merged those paths there,
            // and the head then waited for the loads of the next two blocks)
            for (; u + NB <= u1;) {
#pragma unroll
                for (int q = 0; q < NB; ++q) {
                    block(xb[q], xb[(q + NB - 1) % NB], kept[q]);
                    ++k;
                    ++u;
                }
            }
#pragma unroll
            for (int q = 0; q + 1 < NB; ++q) {
                if (u < u1) {                     // uniform
                    block(xb[q], xb[(q + NB - 1) % NB], kept[q]);
                    ++k;
                    ++u;
                }
            }
        }
    }
}

// Single launch: the split that starts last in each (tile, rank group)
// writes its h columns; the group holding the adapter's last rank column
// also zeroes the columns from the rank up to r_max; tiles of tokens without
// an adapter are zeroed by their (split 0, group 0) workgroup.
// Eight waves per SIMD for the one-rank-tile kernels with compile-time
// chains, as the two-pass partial kernel gets: the poll loops would otherwise
// raise the scalar register count past that occupancy (the compiler keeps the
// excess in vector-register lanes; the other variants would spill to memory).
// Measured on MI355X, 32 decode tokens with one rank-64 adapter each: 15.9 ->
// 13.2 us.
template <int RT, int W, int KST>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(RT == 1 && KST > 0 && W >= 4 ? 8 : 1, 8)))
void k_sgmv_shrink_counted(ShrinkParams p, CounterParams c)
{
    __shared__ float red[red_floats<RT, W>()];
    __shared__ float own[16 * 16 * RT];
    __shared__ int flag;
    const int groups = (p.r_max + 16 * RT - 1) / (16 * RT);
    const uint32_t items = (uint32_t)plan_tiles(p.tiles, p.M, p.n_adapters) * p.split_k * groups;
    for (uint32_t it = blockIdx.x; it < items; it += gridDim.x) {
        const SgmvItem q = sgmv_item(p, it, groups);
        if (!q.ok)
            continue;
        if (q.a < 0) {
            if (q.s == 0 && q.grp == 0)
                for (int e = threadIdx.x; e < q.nrows * p.r_max; e += blockDim.x)
                    if (row_in(q.mask, e / p.r_max))
                        c.h[(q.row0 + e / p.r_max) * c.ld_h + e % p.r_max] = 0.0f;
            continue;
        }
        const uint16_t* Aa = adapter_weights(p, q.a);
        const int ra = adapter_rank(p, q.a);
        const int col0 = q.grp * 16 * RT;
        if (col0 >= ra)
            continue;
        int32_t* counter = c.counters + (int64_t)q.tile * kMaxRankTiles + q.grp;
        int arrived = 0;
        if (threadIdx.x == 0)
            arrived = arrival_add(counter, p.split_k);
        shrink_tile<RT, W, kToLds, KST>(p, q.row0, q.nrows, q.mask, Aa, ra, col0, q.s, 1.0f, red, own);
        if (threadIdx.x == 0)
            flag = arrived;
        __syncthreads();
        const bool last = flag == p.split_k - 1;
        const float scale = last && c.scales ? table_load(c.scales, q.a) : 1.0f;
        const int cend = col0 + 16 * RT < ra ? col0 + 16 * RT : ra;
        const int czero = cend == ra ? p.r_max : cend;
        tagged_finish<RT, 4>(p, q.row0, q.nrows, q.mask, col0, cend, czero, q.s, last, scale, own, c.h, c.ld_h);
        __syncthreads();                          // own and flag are reused by the next item
    }
}

// Large M, single launch: the items of k_sgmv_shrink_partial_multi (up to T
// consecutive plan tiles of one adapter share the A loads; every rank tile
// of r_max <= 64 in one workgroup) with the arrival-counter combine of
// k_sgmv_shrink_counted per tile: one counter add per tile when the item
// starts, partials kept in LDS, then stored to tagged slots; the split that
// started last evaluates the tile's h (fixed tree, the adapter's shrink
// scale).  Tiles of tokens without
// an adapter get zero h rows from their split-0 item.  Same bits as the
// two-pass multi-adapter shrink.
template <int RT, int W, int T>
__global__ __launch_bounds__(W * 64, 4) void k_sgmv_shrink_counted_multi(ShrinkParams p, CounterParams c)
{
    __shared__ float red[red_floats<RT, W>()];
    __shared__ float own[T * 16 * 16 * RT];
    __shared__ int flag[T];
    const int ntiles = plan_tiles(p.tiles, p.M, p.n_adapters);
    const uint32_t S = (uint32_t)p.split_k;
    const uint32_t items = (uint32_t)((ntiles + T - 1) / T) * S;
    const int32_t* plan = p.tiles + kPlanHeaderInts;
    for (uint32_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int s = (int)(it % S);
        const int c0 = (int)(it / S) * T;
        const int c1 = c0 + T < ntiles ? c0 + T : ntiles;
        int j = c0;
        while (j < c1) {                          // uniform: plan data only
            const PlanInts et = plan_entry(plan + kPlanTileInts * j);
            const int32_t* t = et.v;
            if (!tile_rows_ok(t, p.M)) {
                ++j;
                continue;
            }
            if (t[2] < 0 || t[2] >= p.n_adapters) {
                if (s == 0) {
                    const uint32_t m = tile_mask(t);
                    for (int e = threadIdx.x; e < t[1] * p.r_max; e += blockDim.x)
                        if (row_in(m, e / p.r_max))
                            c.h[(t[0] + e / p.r_max) * c.ld_h + e % p.r_max] = 0.0f;
                }
                ++j;
                continue;
            }
            const int a = t[2];
            int64_t row0[T];
            int nrows[T];
            uint32_t mask[T];
            int n = 0;
#pragma unroll
            for (int u = 0; u < T; ++u) {
                PlanInts eu{{0, 0, -1, 0}};
                if (j + u < c1)
                    eu = plan_entry(plan + kPlanTileInts * (j + u));
                const int32_t* tu = eu.v;
                const bool take = n == u && j + u < c1 && tile_ok(tu, p.M, p.n_adapters) && tu[2] == a;
                row0[u] = take ? tu[0] : t[0];
                nrows[u] = take ? tu[1] : 0;
                mask[u] = take ? tile_mask(tu) : 0u;
                n += take ? 1 : 0;
            }
            const int ra = adapter_rank(p, a);
            if (ra > 0) {
                int arrived = 0;
                if ((int)threadIdx.x < n)
                    arrived = arrival_add(c.counters + (int64_t)(j + (int)threadIdx.x) * kMaxRankTiles, p.split_k);
                shrink_tiles<RT, W, kToLds, T>(p, row0, nrows, mask, adapter_weights(p, a), ra, 0, s, 1.0f, red,
                                               own);
                if ((int)threadIdx.x < n)
                    flag[threadIdx.x] = arrived;
                __syncthreads();
#pragma unroll
                for (int u = 0; u < T; ++u) {
                    if (u < n) {                  // uniform
                        const bool last = flag[u] == p.split_k - 1;
                        const float scale = last && c.scales ? table_load(c.scales, a) : 1.0f;
                        tagged_finish<RT, 4>(p, row0[u], nrows[u], mask[u], 0, ra < 16 * RT ? ra : 16 * RT, p.r_max,
                                          s, last, scale, own + u * 16 * 16 * RT, c.h, c.ld_h);
                    }
                }
                __syncthreads();                  // own and flag are reused
            }
            j += n;
        }
    }
}

// ---------------------------------------------------------------------------
// Second pass of the two-pass shrink: h = scale * tree(ws[0..S-1]).
// ---------------------------------------------------------------------------
// Multi-adapter, TABLE: the token's id, the workspace slices (read for every
// element; those of tokens without an adapter and of columns past the rank
// are discarded) and the rank and scale tables are loaded at once, instead of
// the id, then the rank and scale, then the slices.  Used for grids of at most
// one workgroup per compute unit, where each dependent load is latency that
// no other workgroup hides.  Measured on MI355X after the multi-adapter
// partials (HIP graphs, cold inputs; 32 and 128 decode tokens, one rank-64
// adapter each): the tree adds 2.1 and 1.9 us instead of 2.7 and 2.5 us.
// Same arithmetic either way.
//
// Each workgroup takes rows_per_wg = 256 / ncols whole rows, thread t
// column t % ncols of row t / ncols (the quotient from the hardware
// reciprocal, exact in this range): no 64-bit division ahead of the loads.
template <int S, bool SGMV, bool TABLE>
__global__ __launch_bounds__(256) void k_splitk_tree(TreeParams p, int rows_per_wg)
{
    const int tr = div_small((int)threadIdx.x, __builtin_amdgcn_rcpf((float)p.ncols));
    const int j = (int)threadIdx.x - tr * p.ncols;
    const int64_t i0 = (int64_t)blockIdx.x * rows_per_wg + tr;
    const bool live = tr < rows_per_wg && i0 < p.M;
    if (!TABLE && !live)
        return;
    const int64_t i = live ? i0 : 0;
    float scale = p.scale;
    bool zero = false;
    float v[S];
    if constexpr (TABLE) {
        const int a = live ? p.ids[i] : -1;
        if (live) {
            const float* w = p.ws + i * p.ldw + j;
#pragma unroll
            for (int s = 0; s < S; ++s)
                v[s] = w[(int64_t)s * p.split_stride];
        }
        __shared__ int32_t trank[kAdapterTable];
        __shared__ float tscale[kAdapterTable];
        table_fill(trank, p.ranks, p.n_adapters);
        table_fill(tscale, p.scales, p.n_adapters);
        __syncthreads();
        if (!live)
            return;
        if (a < 0 || a >= p.n_adapters) {
            zero = true;
        } else {
            int ra = table_get(trank, p.ranks, a, 0);
            ra = ra < 0 ? 0 : (ra > p.ncols ? p.ncols : ra);
            zero = j >= ra;
            scale = table_get(tscale, p.scales, a, 1.0f);
        }
    } else {
        if constexpr (SGMV) {
            const int a = p.ids[i];
            if (a < 0 || a >= p.n_adapters) {
                zero = true;
            } else {
                int ra = p.ranks[a];
                ra = ra < 0 ? 0 : (ra > p.ncols ? p.ncols : ra);
                zero = j >= ra;
                scale = p.scales ? p.scales[a] : 1.0f;
            }
        }
        if (!zero) {
            const float* w = p.ws + i * p.ldw + j;
#pragma unroll
            for (int s = 0; s < S; ++s)
                v[s] = w[(int64_t)s * p.split_stride];
        }
    }
    p.h[i * p.ld_h + j] = zero ? 0.0f : __fmul_rn(pairwise_tree<S>(v), scale);
}

__global__ __launch_bounds__(256) void k_fill_zero(float* h, int64_t ld_h, int64_t M, int ncols)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= M * ncols)
        return;
    const int64_t i = e / ncols;
    h[i * ld_h + (e - i * ncols)] = 0.0f;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
inline dim3 single_grid(const ShrinkParams& p, int groups)
{
    return dim3((unsigned)(((p.M + kRowBlock - 1) / kRowBlock) * p.split_k * groups));
}

template <int MODE, int RT, int W>
void launch_partial_rw(const ShrinkParams& p, int groups, hipStream_t st)
{
    const dim3 g = single_grid(p, groups);
    switch (p.k_steps) {
    case 1: hipLaunchKernelGGL((k_shrink_partial<RT, W, MODE, 1>), g, dim3(W * 64), 0, st, p, groups); break;
    case 2: hipLaunchKernelGGL((k_shrink_partial<RT, W, MODE, 2>), g, dim3(W * 64), 0, st, p, groups); break;
    case 4: hipLaunchKernelGGL((k_shrink_partial<RT, W, MODE, 4>), g, dim3(W * 64), 0, st, p, groups); break;
    default: hipLaunchKernelGGL((k_shrink_partial<RT, W, MODE, 0>), g, dim3(W * 64), 0, st, p, groups); break;
    }
}

template <int MODE, int RT>
void launch_partial_r(const ShrinkParams& p, int waves, int groups, hipStream_t st)
{
    switch (waves) {
    case 1: launch_partial_rw<MODE, RT, 1>(p, groups, st); break;
    case 2: launch_partial_rw<MODE, RT, 2>(p, groups, st); break;
    case 4: launch_partial_rw<MODE, RT, 4>(p, groups, st); break;
    default: launch_partial_rw<MODE, RT, 8>(p, groups, st); break;
    }
}

// group_tiles: rank tiles per workgroup (1 .. rank_tiles).
template <int MODE>
hipError_t launch_partial(const ShrinkParams& p, int waves, int rank_tiles, int group_tiles, hipStream_t st)
{
    if (group_tiles < 1 || group_tiles > kGroupTiles)
        return hipErrorInvalidValue;
    const int groups = (rank_tiles + group_tiles - 1) / group_tiles;
    switch (group_tiles) {
    case 1: launch_partial_r<MODE, 1>(p, waves, groups, st); break;
    case 2: launch_partial_r<MODE, 2>(p, waves, groups, st); break;
    case 3: launch_partial_r<MODE, 3>(p, waves, groups, st); break;
    default: launch_partial_r<MODE, 4>(p, waves, groups, st); break;
    }
    return hipGetLastError();
}

template <int RT, int W>
void launch_counted_rw(const ShrinkParams& p, const CounterParams& c, int groups, hipStream_t st)
{
    const dim3 g = single_grid(p, groups);
    switch (p.k_steps) {
    case 1: hipLaunchKernelGGL((k_shrink_counted<RT, W, 1>), g, dim3(W * 64), 0, st, p, c, groups); break;
    case 2: hipLaunchKernelGGL((k_shrink_counted<RT, W, 2>), g, dim3(W * 64), 0, st, p, c, groups); break;
    case 4: hipLaunchKernelGGL((k_shrink_counted<RT, W, 4>), g, dim3(W * 64), 0, st, p, c, groups); break;
    default: hipLaunchKernelGGL((k_shrink_counted<RT, W, 0>), g, dim3(W * 64), 0, st, p, c, groups); break;
    }
}

template <int RT>
void launch_counted_r(const ShrinkParams& p, const CounterParams& c, int waves, int groups, hipStream_t st)
{
    switch (waves) {
    case 1: launch_counted_rw<RT, 1>(p, c, groups, st); break;
    case 2: launch_counted_rw<RT, 2>(p, c, groups, st); break;
    case 4: launch_counted_rw<RT, 4>(p, c, groups, st); break;
    default: launch_counted_rw<RT, 8>(p, c, groups, st); break;
    }
}

template <int RT, bool COUNTED, int MODE = kToWorkspace>
void launch_sgmv_r(const ShrinkParams& p, const CounterParams& c, int waves, int grid, hipStream_t st)
{
    dim3 g((unsigned)grid);
#define LORA_SGMV_LAUNCH(W_)                                                                          \
    do {                                                                                              \
        if (COUNTED && p.k_steps == 2)                                                                \
            hipLaunchKernelGGL((k_sgmv_shrink_counted<RT, W_, 2>), g, dim3(W_ * 64), 0, st, p, c);     \
        else if (COUNTED && p.k_steps == 4)                                                           \
            hipLaunchKernelGGL((k_sgmv_shrink_counted<RT, W_, 4>), g, dim3(W_ * 64), 0, st, p, c);     \
        else if (COUNTED)                                                                             \
            hipLaunchKernelGGL((k_sgmv_shrink_counted<RT, W_, 0>), g, dim3(W_ * 64), 0, st, p, c);     \
        else if (p.k_steps == 2)                                                                      \
            hipLaunchKernelGGL((k_sgmv_shrink_partial<RT, W_, MODE, 2>), g, dim3(W_ * 64), 0, st, p);  \
        else if (p.k_steps == 4)                                                                      \
            hipLaunchKernelGGL((k_sgmv_shrink_partial<RT, W_, MODE, 4>), g, dim3(W_ * 64), 0, st, p);  \
        else                                                                                          \
            hipLaunchKernelGGL((k_sgmv_shrink_partial<RT, W_, MODE, 0>), g, dim3(W_ * 64), 0, st, p);  \
    } while (0)
    switch (waves) {
    case 1: LORA_SGMV_LAUNCH(1); break;
    case 2: LORA_SGMV_LAUNCH(2); break;
    case 4: LORA_SGMV_LAUNCH(4); break;
    default: LORA_SGMV_LAUNCH(8); break;
    }
#undef LORA_SGMV_LAUNCH
}

// Whole rows of the tree kernel per 256-thread workgroup (ncols <= kMaxRank).
inline int tree_rows_per_wg(int ncols)
{
    return 256 / ncols;
}

template <bool SGMV, bool TABLE>
hipError_t launch_tree_t(const TreeParams& p, int S, hipStream_t st)
{
    const int rows = tree_rows_per_wg(p.ncols);
    dim3 grid((unsigned)((p.M + rows - 1) / rows)), block(256);
    switch (S) {
    case 1: hipLaunchKernelGGL((k_splitk_tree<1, SGMV, TABLE>), grid, block, 0, st, p, rows); break;
    case 2: hipLaunchKernelGGL((k_splitk_tree<2, SGMV, TABLE>), grid, block, 0, st, p, rows); break;
    case 4: hipLaunchKernelGGL((k_splitk_tree<4, SGMV, TABLE>), grid, block, 0, st, p, rows); break;
    case 8: hipLaunchKernelGGL((k_splitk_tree<8, SGMV, TABLE>), grid, block, 0, st, p, rows); break;
    default: hipLaunchKernelGGL((k_splitk_tree<16, SGMV, TABLE>), grid, block, 0, st, p, rows); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_shrink_partial_ws(const ShrinkParams& p, int waves, int rank_tiles, int group_tiles,
                                    hipStream_t st)
{
    return launch_partial<kToWorkspace>(p, waves, rank_tiles, group_tiles, st);
}

namespace {

template <int RT, int T, int MODE>
void launch_multi_rt(const ShrinkParams& p, int waves, dim3 grid, bool sgmv, hipStream_t st)
{
    // the multi-adapter kernel takes at most two tiles with 3-4 rank tiles
    // (four do not fit in 128 registers), so that variant is not built
    constexpr int TS = (RT > 2 && T > 2) ? 2 : T;
#define LORA_MULTI(W_)                                                                                    \
    do {                                                                                                  \
        if (sgmv)                                                                                         \
            hipLaunchKernelGGL((k_sgmv_shrink_partial_multi<RT, W_, TS, MODE>), grid, dim3(W_ * 64), 0, st, p); \
        else                                                                                              \
            hipLaunchKernelGGL((k_shrink_partial_multi<RT, W_, T, MODE>), grid, dim3(W_ * 64), 0, st, p);       \
    } while (0)
    switch (waves) {
    case 1: LORA_MULTI(1); break;
    case 2: LORA_MULTI(2); break;
    case 4: LORA_MULTI(4); break;
    default: LORA_MULTI(8); break;
    }
#undef LORA_MULTI
}

template <int T, int MODE>
void launch_multi_tm(const ShrinkParams& p, int waves, int rank_tiles, dim3 grid, bool sgmv, hipStream_t st)
{
    if (rank_tiles == 1)
        launch_multi_rt<1, T, MODE>(p, waves, grid, sgmv, st);
    else if (rank_tiles == 2)
        launch_multi_rt<2, T, MODE>(p, waves, grid, sgmv, st);
    else
        launch_multi_rt<4, T, MODE>(p, waves, grid, sgmv, st);
}

template <int T>
void launch_multi_t(const ShrinkParams& p, int waves, int rank_tiles, dim3 grid, bool sgmv, bool atomic,
                    hipStream_t st)
{
    if (atomic)
        launch_multi_tm<T, kAtomicScaled>(p, waves, rank_tiles, grid, sgmv, st);
    else
        launch_multi_tm<T, kToWorkspace>(p, waves, rank_tiles, grid, sgmv, st);
}

}  // namespace

hipError_t launch_shrink_partial_multi(const ShrinkParams& p, int waves, int rank_tiles, int tiles_per_wg,
                                       hipStream_t st, bool atomic)
{
    if (rank_tiles < 1 || rank_tiles > kGroupTiles)
        return hipErrorInvalidValue;
    const int64_t mbs = (p.M + kRowBlock - 1) / kRowBlock;
    const dim3 grid((unsigned)(((mbs + tiles_per_wg - 1) / tiles_per_wg) * p.split_k));
    if (tiles_per_wg == 2)
        launch_multi_t<2>(p, waves, rank_tiles, grid, false, atomic, st);
    else
        launch_multi_t<4>(p, waves, rank_tiles, grid, false, atomic, st);
    return hipGetLastError();
}

hipError_t launch_sgmv_shrink_partial_multi(const ShrinkParams& p, int waves, int tiles_per_wg, int grid,
                                            hipStream_t st, bool atomic)
{
    const int rank_tiles = (p.r_max + 15) / 16;
    if (rank_tiles > kGroupTiles)
        return hipErrorInvalidValue;
    // with 3-4 rank tiles, four plan tiles per workgroup do not fit in the
    // 128 registers of two workgroups per compute unit: take two
    if (tiles_per_wg == 2 || rank_tiles > 2)
        launch_multi_t<2>(p, waves, rank_tiles, dim3((unsigned)grid), true, atomic, st);
    else
        launch_multi_t<4>(p, waves, rank_tiles, dim3((unsigned)grid), true, atomic, st);
    return hipGetLastError();
}

namespace {

template <int RT, int T>
void launch_counted_multi_rt(const ShrinkParams& p, const CounterParams& c, int waves, dim3 grid, hipStream_t st)
{
    constexpr int TS = (RT > 2 && T > 2) ? 2 : T;   // as for the two-pass kernel: registers
    switch (waves) {
    case 1: hipLaunchKernelGGL((k_sgmv_shrink_counted_multi<RT, 1, TS>), grid, dim3(64), 0, st, p, c); break;
    case 2: hipLaunchKernelGGL((k_sgmv_shrink_counted_multi<RT, 2, TS>), grid, dim3(128), 0, st, p, c); break;
    case 4: hipLaunchKernelGGL((k_sgmv_shrink_counted_multi<RT, 4, TS>), grid, dim3(256), 0, st, p, c); break;
    default: hipLaunchKernelGGL((k_sgmv_shrink_counted_multi<RT, 8, TS>), grid, dim3(512), 0, st, p, c); break;
    }
}

}  // namespace

hipError_t launch_sgmv_shrink_counted_multi(const ShrinkParams& p, const CounterParams& c, int waves,
                                            int tiles_per_wg, int grid, hipStream_t st)
{
    const int rank_tiles = (p.r_max + 15) / 16;
    if (rank_tiles > kGroupTiles || grid < 1)
        return hipErrorInvalidValue;
    const dim3 g((unsigned)grid);
    if (rank_tiles == 1)
        tiles_per_wg == 2 ? launch_counted_multi_rt<1, 2>(p, c, waves, g, st)
                          : launch_counted_multi_rt<1, 4>(p, c, waves, g, st);
    else if (rank_tiles == 2)
        tiles_per_wg == 2 ? launch_counted_multi_rt<2, 2>(p, c, waves, g, st)
                          : launch_counted_multi_rt<2, 4>(p, c, waves, g, st);
    else
        launch_counted_multi_rt<4, 2>(p, c, waves, g, st);
    return hipGetLastError();
}

namespace {

template <int RT, int W, bool SGMV, int MODE>
hipError_t launch_stream_rws(const ShrinkParams& p, int steps, int R, dim3 grid, hipStream_t st)
{
    switch (steps) {
    case 1: hipLaunchKernelGGL((k_shrink_stream<RT, W, 1, SGMV, MODE>), grid, dim3(W * 64), 0, st, p, R); break;
    case 2: hipLaunchKernelGGL((k_shrink_stream<RT, W, 2, SGMV, MODE>), grid, dim3(W * 64), 0, st, p, R); break;
    default:
        if constexpr (RT <= 2)
            hipLaunchKernelGGL((k_shrink_stream<RT, W, 4, SGMV, MODE>), grid, dim3(W * 64), 0, st, p, R);
        else
            return hipErrorInvalidValue;
        break;
    }
    return hipGetLastError();
}

template <int RT, bool SGMV, int MODE>
hipError_t launch_stream_rm(const ShrinkParams& p, int waves, int steps, int R, dim3 grid, hipStream_t st)
{
    return waves == 8 ? launch_stream_rws<RT, 8, SGMV, MODE>(p, steps, R, grid, st)
                      : launch_stream_rws<RT, 4, SGMV, MODE>(p, steps, R, grid, st);
}

template <int RT, bool SGMV>
hipError_t launch_stream_r(const ShrinkParams& p, int waves, int steps, int R, dim3 grid, bool atomic,
                           hipStream_t st)
{
    return atomic ? launch_stream_rm<RT, SGMV, kAtomicScaled>(p, waves, steps, R, grid, st)
                  : launch_stream_rm<RT, SGMV, kToWorkspace>(p, waves, steps, R, grid, st);
}

}  // namespace

bool shrink_stream_fits(int waves, int k_steps, int rank_tiles)
{
    if (rank_tiles < 1 || rank_tiles > kGroupTiles)
        return false;
    const int rt = rank_tiles <= 1 ? 1 : (rank_tiles == 2 ? 2 : 4);
    return (waves == 4 || waves == 8) && (k_steps == 1 || k_steps == 2 || k_steps == 4) && rt * k_steps <= 8;
}

hipError_t launch_shrink_stream(const ShrinkParams& p, int waves, int k_steps, int rank_tiles, int R, int grid,
                                bool sgmv, hipStream_t st, bool atomic)
{
    if (!shrink_stream_fits(waves, k_steps, rank_tiles) || R < 1 || R > kStreamMaxRows || grid < 1)
        return hipErrorInvalidValue;
    const dim3 g((unsigned)grid);
    if (rank_tiles <= 1)
        return sgmv ? launch_stream_r<1, true>(p, waves, k_steps, R, g, atomic, st)
                    : launch_stream_r<1, false>(p, waves, k_steps, R, g, atomic, st);
    if (rank_tiles == 2)
        return sgmv ? launch_stream_r<2, true>(p, waves, k_steps, R, g, atomic, st)
                    : launch_stream_r<2, false>(p, waves, k_steps, R, g, atomic, st);
    return sgmv ? launch_stream_r<4, true>(p, waves, k_steps, R, g, atomic, st)
                : launch_stream_r<4, false>(p, waves, k_steps, R, g, atomic, st);
}

hipError_t launch_shrink_partial_direct(const ShrinkParams& p, int waves, int rank_tiles, int group_tiles,
                                        hipStream_t st)
{
    return launch_partial<kToOutputScaled>(p, waves, rank_tiles, group_tiles, st);
}

hipError_t launch_shrink_partial_atomic(const ShrinkParams& p, int waves, int rank_tiles, int group_tiles,
                                        hipStream_t st)
{
    return launch_partial<kAtomicScaled>(p, waves, rank_tiles, group_tiles, st);
}

hipError_t launch_shrink_counted(const ShrinkParams& p, const CounterParams& c, int waves, int rank_tiles,
                                 int group_tiles, hipStream_t st)
{
    if (group_tiles < 1 || group_tiles > kGroupTiles)
        return hipErrorInvalidValue;
    const int groups = (rank_tiles + group_tiles - 1) / group_tiles;
    switch (group_tiles) {
    case 1: launch_counted_r<1>(p, c, waves, groups, st); break;
    case 2: launch_counted_r<2>(p, c, waves, groups, st); break;
    case 3: launch_counted_r<3>(p, c, waves, groups, st); break;
    default: launch_counted_r<4>(p, c, waves, groups, st); break;
    }
    return hipGetLastError();
}

hipError_t launch_sgmv_shrink_partial(const ShrinkParams& p, int waves, int group_tiles, int grid, hipStream_t st,
                                      bool atomic)
{
    const CounterParams none{};
    if (atomic) {
        if (group_tiles == 1)
            launch_sgmv_r<1, false, kAtomicScaled>(p, none, waves, grid, st);
        else if (group_tiles == 2)
            launch_sgmv_r<2, false, kAtomicScaled>(p, none, waves, grid, st);
        else
            launch_sgmv_r<4, false, kAtomicScaled>(p, none, waves, grid, st);
    } else {
        if (group_tiles == 1)
            launch_sgmv_r<1, false>(p, none, waves, grid, st);
        else if (group_tiles == 2)
            launch_sgmv_r<2, false>(p, none, waves, grid, st);
        else
            launch_sgmv_r<4, false>(p, none, waves, grid, st);
    }
    return hipGetLastError();
}

hipError_t launch_sgmv_shrink_counted(const ShrinkParams& p, const CounterParams& c, int waves, int group_tiles,
                                      int grid, hipStream_t st)
{
    if (group_tiles == 1)
        launch_sgmv_r<1, true>(p, c, waves, grid, st);
    else if (group_tiles == 2)
        launch_sgmv_r<2, true>(p, c, waves, grid, st);
    else
        launch_sgmv_r<4, true>(p, c, waves, grid, st);
    return hipGetLastError();
}

hipError_t launch_splitk_tree(const TreeParams& p, int split_k, bool sgmv, hipStream_t st)
{
    if (!sgmv)
        return launch_tree_t<false, false>(p, split_k, st);
    // adapter tables for grids of at most one workgroup per compute unit
    const int64_t wgs = (p.M + tree_rows_per_wg(p.ncols) - 1) / tree_rows_per_wg(p.ncols);
    return wgs <= 256 ? launch_tree_t<true, true>(p, split_k, st) : launch_tree_t<true, false>(p, split_k, st);
}

hipError_t launch_fill_zero(float* h, int64_t ld_h, int64_t M, int ncols, hipStream_t st)
{
    const int64_t n = M * ncols;
    dim3 grid((unsigned)((n + 255) / 256)), block(256);
    hipLaunchKernelGGL(k_fill_zero, grid, block, 0, st, h, ld_h, M, ncols);
    return hipGetLastError();
}

}  // namespace lora
