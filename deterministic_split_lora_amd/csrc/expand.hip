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
// matrix-core step over j < 32 (r <= 32), two (r <= 64) or four (r <= 128)
// with zero-padded reduction slots, then one fma and one rounding; it does not
// depend on the tiling, M or the token's neighbours.
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

__device__ __forceinline__ ExpandItem expand_item_at(uint32_t item, int64_t M, int64_t N, int cols = kExpandCols)
{
    ExpandItem q;                                 // 32-bit: the grid is below 2^31
    const uint32_t nblocks = (uint32_t)((N + cols - 1) / cols);
    q.cb = item % nblocks;
    q.row0 = (int64_t)(item / nblocks) * kRowBlock;
    const int64_t left = M - q.row0;
    q.nrows = left < kRowBlock ? (int)left : kRowBlock;
    return q;
}

__device__ __forceinline__ ExpandItem expand_item(int64_t M, int64_t N)
{
    return expand_item_at(blockIdx.x, M, N);
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

// Compensated single-adapter expand: the grid and loads of k_expand, the
// arithmetic of expand_finish_comp (two matrix-core passes, hi and lo of h).
template <int KS>
__global__ __launch_bounds__(256) void k_expand_comp(ExpandParams p)
{
    const ExpandItem q = expand_item(p.M, p.N);
    ExpandLane L = expand_lane(q.row0, q.nrows, q.cb * kExpandCols);
    if (L.n_base >= p.N)
        return;
    u16x8 yv[2];
    bf16x8 bop[4][KS];
    expand_load<KS>(L, p.y, p.ld_y, p.N, p.B, p.ld_b, p.r, yv, bop);
    expand_finish_comp<KS>(L, p.y, p.ld_y, p.N, p.h + q.row0 * p.ld_h, p.ld_h, p.r, p.scale, yv, bop);
}

// Single adapter, large M: a workgroup walks R consecutive 16-token tiles of
// one 256-column block.  Its B operands are loaded once and stay in
// registers; each tile's h rows are converted to bf16 once into LDS instead
// of once per wave.  y moves through LDS: it is read and written row by row
// (thread t moves the 16-byte chunk t % 32 of rows t / 32 and t / 32 + 8, so
// a wave covers two whole 512-byte row segments per access) and each lane
// takes its 16 matrix-core-layout values from the LDS tile and puts its
// results back in their place.  Loads run one tile ahead, stores one tile
// behind: while tile i is computed, tile i + 1's y and h are in flight and
// tile i - 1 is being written out, with one barrier per tile (y and h tiles
// double buffered).  Per element this is the arithmetic of k_expand (same
// operands, steps and epilogue code); only the data movement differs.
__device__ __forceinline__ int tile_rows(int64_t M, int64_t row0)
{
    const int64_t left = M - row0;
    return left < kRowBlock ? (int)left : kRowBlock;
}

constexpr int kYStride = kExpandCols + 8;     // bf16 per LDS row of a y tile (528 bytes)

struct YChunk {
    int row;                                  // first of the thread's rows; the other is row + 8
    int col;                                  // first of its 8 columns
};

__device__ __forceinline__ YChunk y_chunk()
{
    return YChunk{(int)threadIdx.x >> 5, ((int)threadIdx.x & 31) * 8};
}

// ok bit e: the thread's row e (row + 8 e) is read / written.  y is read
// once and written once per call, so both go with the nontemporal hint: y
// streams past the caches instead of leaving hundreds of MB of dirty lines
// for the next kernel to compete with (measured on MI355X at 4096 x 28672,
// 32 adapters: multi-adapter shrink + expand 137.5 -> 125.5 us, the expand
// alone 106.6 -> 101.1 us; the shrink that follows an expand had been 4 us
// slower than one that follows a small kernel).
__device__ __forceinline__ void y_chunk_load(const YChunk& c, const uint16_t* y, int64_t ld_y, int64_t row0,
                                             int64_t col0, unsigned ok, u16x8 (&g)[2])
{
#pragma unroll
    for (int e = 0; e < 2; ++e)
        g[e] = (ok >> e & 1u) ? __builtin_nontemporal_load(
                                    reinterpret_cast<const u16x8*>(y + (row0 + c.row + 8 * e) * ld_y + col0 + c.col))
                              : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
}

__device__ __forceinline__ void y_chunk_put(const YChunk& c, const u16x8 (&g)[2], uint16_t* tile)
{
#pragma unroll
    for (int e = 0; e < 2; ++e)
        *reinterpret_cast<u16x8*>(tile + (c.row + 8 * e) * kYStride + c.col) = g[e];
}

__device__ __forceinline__ void y_chunk_store(const YChunk& c, const uint16_t* tile, uint16_t* y, int64_t ld_y,
                                              int64_t row0, int64_t col0, unsigned ok)
{
#pragma unroll
    for (int e = 0; e < 2; ++e)
        if (ok >> e & 1u)
            __builtin_nontemporal_store(*reinterpret_cast<const u16x8*>(tile + (c.row + 8 * e) * kYStride + c.col),
                                        reinterpret_cast<u16x8*>(y + (row0 + c.row + 8 * e) * ld_y + col0 + c.col));
}

// Rows of the thread's chunk inside a tile of nrows rows (and N, when the
// chunk's columns are inside N).
__device__ __forceinline__ unsigned y_chunk_rows(const YChunk& c, int nrows, bool col_ok)
{
    return col_ok ? (unsigned)(c.row < nrows) | (unsigned)(c.row + 8 < nrows) << 1 : 0u;
}

// This lane's 16 values in the LDS y tile: row li, columns 64 wave + 16 g ..
__device__ __forceinline__ uint16_t* y_lane(const ExpandLane& L, uint16_t* tile)
{
    return tile + L.li * kYStride + (int)(threadIdx.x >> 6) * 64 + 16 * L.g;
}

// The expand of one lane's 16 values held in the LDS y tile, written back in place.
template <int KS>
__device__ __forceinline__ void expand_in_tile(uint16_t* yl, const bf16x8 (&hb)[KS], float scale,
                                               const bf16x8 (&bop)[4][KS])
{
    u16x8 yv[2], o[2];
    yv[0] = *reinterpret_cast<const u16x8*>(yl);
    yv[1] = *reinterpret_cast<const u16x8*>(yl + 8);
    expand_mma<KS>(hb, scale, yv, bop, o);
    *reinterpret_cast<u16x8*>(yl) = o[0];
    *reinterpret_cast<u16x8*>(yl + 8) = o[1];
}

template <int KS>
__global__ __launch_bounds__(256) void k_expand_rows(ExpandParams p, int R)
{
    __shared__ __align__(16) uint16_t hs[2][kRowBlock * kHbStride];
    __shared__ __align__(16) uint16_t ys[2][kRowBlock * kYStride];
    const uint32_t nblocks = (uint32_t)((p.N + kExpandCols - 1) / kExpandCols);
    const int64_t col0 = (int64_t)(blockIdx.x % nblocks) * kExpandCols;
    const int64_t row_base = (int64_t)(blockIdx.x / nblocks) * kRowBlock * R;
    const int64_t left = (p.M - row_base + kRowBlock - 1) / kRowBlock;
    const int tiles = left < R ? (int)left : R;
    constexpr int HC = KS == 4 ? 8 : 4;          // h columns each staging thread converts
    const HStageSlot slot = h_stage_slot<HC>(p.r);
    const YChunk yc = y_chunk();
    const bool col_ok = col0 + yc.col < p.N;
    const unsigned full = y_chunk_rows(yc, kRowBlock, col_ok);
    ExpandLane L = expand_lane(row_base, kRowBlock, col0);
    const bool active = L.n_base < p.N;
    bf16x8 bop[4][KS];
    expand_load_b<KS>(L, p.N, p.B, p.ld_b, p.r, bop);
    u16x8 g[2];
    float f[HC];
    int nr = tile_rows(p.M, row_base);
    unsigned ok = y_chunk_rows(yc, nr, col_ok);
    y_chunk_load(yc, p.y, p.ld_y, row_base, col0, ok, g);
    h_load(slot, p.h, p.ld_h, row_base, nr, p.r, f);
    y_chunk_put(yc, g, ys[0]);
    h_put(slot, f, p.r, hs[0]);
    __syncthreads();
    for (int i = 0; i < tiles; ++i) {
        const int64_t row0 = row_base + (int64_t)kRowBlock * i;
        const bool next = i + 1 < tiles;
        const int nr1 = next ? tile_rows(p.M, row0 + kRowBlock) : 0;
        const unsigned ok1 = y_chunk_rows(yc, nr1, col_ok);
        if (next) {
            y_chunk_load(yc, p.y, p.ld_y, row0 + kRowBlock, col0, ok1, g);
            h_load(slot, p.h, p.ld_h, row0 + kRowBlock, nr1, p.r, f);
        }
        if (i > 0)                                   // tile i - 1 is whole
            y_chunk_store(yc, ys[(i - 1) & 1], p.y, p.ld_y, row0 - kRowBlock, col0, full);
        if (active) {
            L.row_ok = L.li < nr;
            bf16x8 hb[KS];
            hb_from_tile<KS>(L, hs[i & 1], p.r, hb);
            expand_in_tile<KS>(y_lane(L, ys[i & 1]), hb, p.scale, bop);
        }
        if (next) {
            y_chunk_put(yc, g, ys[(i + 1) & 1]);
            h_put(slot, f, p.r, hs[(i + 1) & 1]);
        }
        __syncthreads();
        if (next) {
            nr = nr1;
            ok = ok1;
        }
    }
    y_chunk_store(yc, ys[(tiles - 1) & 1], p.y, p.ld_y, row_base + (int64_t)kRowBlock * (tiles - 1), col0, ok);
}

// Compensated expand, large M: the data movement of k_expand_rows with the
// arithmetic of k_expand_comp - each tile's h is staged as its bf16 hi and lo
// halves in two LDS tiles and both pass through expand_mma_comp.
template <int KS>
__global__ __launch_bounds__(256) void k_expand_comp_rows(ExpandParams p, int R)
{
    __shared__ __align__(16) uint16_t hs[2][kRowBlock * kHbStride];
    __shared__ __align__(16) uint16_t hl[2][kRowBlock * kHbStride];
    __shared__ __align__(16) uint16_t ys[2][kRowBlock * kYStride];
    const uint32_t nblocks = (uint32_t)((p.N + kExpandCols - 1) / kExpandCols);
    const int64_t col0 = (int64_t)(blockIdx.x % nblocks) * kExpandCols;
    const int64_t row_base = (int64_t)(blockIdx.x / nblocks) * kRowBlock * R;
    const int64_t left = (p.M - row_base + kRowBlock - 1) / kRowBlock;
    const int tiles = left < R ? (int)left : R;
    constexpr int HC = KS == 4 ? 8 : 4;          // h columns each staging thread converts
    const HStageSlot slot = h_stage_slot<HC>(p.r);
    const YChunk yc = y_chunk();
    const bool col_ok = col0 + yc.col < p.N;
    const unsigned full = y_chunk_rows(yc, kRowBlock, col_ok);
    ExpandLane L = expand_lane(row_base, kRowBlock, col0);
    const bool active = L.n_base < p.N;
    bf16x8 bop[4][KS];
    expand_load_b<KS>(L, p.N, p.B, p.ld_b, p.r, bop);
    u16x8 g[2];
    float f[HC];
    int nr = tile_rows(p.M, row_base);
    unsigned ok = y_chunk_rows(yc, nr, col_ok);
    y_chunk_load(yc, p.y, p.ld_y, row_base, col0, ok, g);
    h_load(slot, p.h, p.ld_h, row_base, nr, p.r, f);
    y_chunk_put(yc, g, ys[0]);
    h_put_comp(slot, f, p.r, hs[0], hl[0]);
    __syncthreads();
    for (int i = 0; i < tiles; ++i) {
        const int64_t row0 = row_base + (int64_t)kRowBlock * i;
        const bool next = i + 1 < tiles;
        const int nr1 = next ? tile_rows(p.M, row0 + kRowBlock) : 0;
        const unsigned ok1 = y_chunk_rows(yc, nr1, col_ok);
        if (next) {
            y_chunk_load(yc, p.y, p.ld_y, row0 + kRowBlock, col0, ok1, g);
            h_load(slot, p.h, p.ld_h, row0 + kRowBlock, nr1, p.r, f);
        }
        if (i > 0)                                   // tile i - 1 is whole
            y_chunk_store(yc, ys[(i - 1) & 1], p.y, p.ld_y, row0 - kRowBlock, col0, full);
        if (active) {
            L.row_ok = L.li < nr;
            bf16x8 hi[KS], lo[KS];
            hb_from_tile<KS>(L, hs[i & 1], p.r, hi);
            hb_from_tile<KS>(L, hl[i & 1], p.r, lo);
            uint16_t* yl = y_lane(L, ys[i & 1]);
            u16x8 yv[2], o[2];
            yv[0] = *reinterpret_cast<const u16x8*>(yl);
            yv[1] = *reinterpret_cast<const u16x8*>(yl + 8);
            expand_mma_comp<KS>(hi, lo, p.scale, yv, bop, o);
            *reinterpret_cast<u16x8*>(yl) = o[0];
            *reinterpret_cast<u16x8*>(yl + 8) = o[1];
        }
        if (next) {
            y_chunk_put(yc, g, ys[(i + 1) & 1]);
            h_put_comp(slot, f, p.r, hs[(i + 1) & 1], hl[(i + 1) & 1]);
        }
        __syncthreads();
        if (next) {
            nr = nr1;
            ok = ok1;
        }
    }
    y_chunk_store(yc, ys[(tiles - 1) & 1], p.y, p.ld_y, row_base + (int64_t)kRowBlock * (tiles - 1), col0, ok);
}

// Fused: the fixed pairwise tree over the Split-K workspace for this row block
// (exactly the second pass of the deterministic shrink: tree, then one
// multiply by the shrink scale) is evaluated into an LDS tile, written out as
// h by the first column block, and fed to the expand without a round trip
// through a separate kernel.  Same bits as shrink then expand.
constexpr int kHTileStride = 132;         // floats per LDS row (128 + 4 padding)

// XR: how the (row block, column block) items meet the XCDs - workgroup w
// runs on XCD w % 8, consecutive workgroups on different XCDs.
//   XR = 1: column block fastest, so an XCD takes every eighth column block
//           of every row block (B is fetched once; every row block's
//           workspace slices by every XCD);
//   XR = 8: the workgroups of XCD x take row blocks x, x + 8, ... with their
//           column blocks one after another (a row block's workspace in one
//           L2; B by every XCD);
//   XR = 2: two row groups x four column groups (XCD x takes row blocks
//           x / 4, x / 4 + 2, ... and column blocks x % 4, x % 4 + 4, ...;
//           the number of column blocks is a multiple of 4): each workspace
//           slice and each B column reaches 4 and 2 L2s.
// Workgroups past the last row block exit at once.
template <int XR>
__device__ __forceinline__ bool combine_item(const ExpandParams& p, int cols, ExpandItem& q)
{
    const uint32_t nblocks = (uint32_t)((p.N + cols - 1) / cols);
    if constexpr (XR == 1) {
        q = expand_item_at(blockIdx.x, p.M, p.N, cols);
    } else {
        const uint32_t x = blockIdx.x % kXcds;
        const uint32_t j = blockIdx.x / kXcds;
        int64_t rb;
        if constexpr (XR == 8) {
            q.cb = j % nblocks;
            rb = (int64_t)(j / nblocks) * kXcds + x;
        } else {
            constexpr uint32_t XC = kXcds / XR;   // column groups
            const uint32_t per = nblocks / XC;    // column blocks of one group
            q.cb = (x % XC) + XC * (j % per);
            rb = (int64_t)(j / per) * XR + x / XC;
        }
        q.row0 = rb * kRowBlock;
        if (q.row0 >= p.M)
            return false;
        const int64_t left = p.M - q.row0;
        q.nrows = left < kRowBlock ? (int)left : kRowBlock;
    }
    return true;
}

template <int KS, int S, int WAVES, int XR>
__global__ __launch_bounds__(WAVES * 64) void k_expand_combine(ExpandParams p, TreeParams c)
{
    constexpr int kCols = WAVES * 64;
    __shared__ __align__(16) float hs[kRowBlock * kHTileStride];
    ExpandItem q;
    if (!combine_item<XR>(p, kCols, q))            // uniform
        return;
    const int64_t row0 = q.row0;
    const int nrows = q.nrows;
    const int r = p.r;
    // y and B first: they do not depend on the workspace
    ExpandLane L = expand_lane(row0, nrows, q.cb * kCols);
    const bool active = L.n_base < p.N;
    u16x8 yv[2];
    bf16x8 bop[4][KS];
    if (active)
        expand_load<KS>(L, p.y, p.ld_y, p.N, p.B, p.ld_b, r, yv, bop);
    const bool write_h = c.h != nullptr && q.cb == 0;
    // nrows x r tile elements over the workgroup's threads, the passes
    // unrolled to their compile-time bound so that every pass's workspace
    // loads are in flight together; (row, col) advance by kCols elements
    // per pass without a division
    constexpr int kPasses = (kRowBlock * 32 * KS + kCols - 1) / kCols;
    const float rcp_r = __builtin_amdgcn_rcpf((float)r);
    const int drow = div_small(kCols, rcp_r);
    const int dcol = kCols - drow * r;
    int row = div_small((int)threadIdx.x, rcp_r);
    int col = (int)threadIdx.x - row * r;
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass, row += drow, col += dcol) {
        if (col >= r) {
            col -= r;
            ++row;
        }
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

// Multi-adapter: the single-adapter expand's grid, one workgroup per
// (16-token row block, 256 columns), every wave on its own.  Each lane reads
// its token's adapter id; tokens without one (id outside [0, n_adapters))
// are neither read nor written.  A matrix-core step shares its B operand
// across the 16 tokens, so the wave makes one pass per distinct adapter among
// its tokens (in the order of their first token; one pass when the block lies
// inside one run of equal ids): the pass loads that adapter's B rows and
// feeds only its own tokens' h rows (the others read as zeros and are not
// stored).  A token's output column depends only on its own h row, so each
// token gets exactly the single-adapter expand's arithmetic with its
// adapter's rank and scale.  The grid is exact (no persistent loop), so the
// hardware keeps as many y tiles in flight as occupancy allows.
template <int KS>
__device__ __forceinline__ void sgmv_pass(const ExpandParams& p, const ExpandLane& L, const float* hrows,
                                          int64_t ld_hr, int a, const u16x8 (&yv)[2])
{
    int ra = table_load(p.ranks, a);
    ra = ra < 0 ? 0 : (ra > p.r_max ? p.r_max : ra);
    const float scale = p.scales ? table_load(p.scales, a) : 1.0f;
    const int64_t ld_b = (ra + 7) & ~7;
    u16x8 unused[2];
    ExpandLane Lb = L;
    Lb.row_ok = false;                               // B rows only
    // the steps the single-adapter expand takes at this rank
    auto pass = [&](auto steps) {
        constexpr int K2 = decltype(steps)::value;
        bf16x8 bop[4][K2];
        expand_load<K2>(Lb, p.y, p.ld_y, p.N, table_load(p.B_ptrs, a), ld_b, ra, unused, bop);
        expand_finish<K2>(L, p.y, p.ld_y, p.N, hrows, ld_hr, ra, scale, yv, bop);
    };
    const int need = expand_steps(ra);
    if constexpr (KS >= 4) {
        if (need == 4) {
            pass(Steps<4>{});
            return;
        }
    }
    if constexpr (KS >= 2) {
        if (need == 2) {
            pass(Steps<2>{});
            return;
        }
    }
    pass(Steps<1>{});
}

// ---------------------------------------------------------------------------
// Multi-adapter combine: h of one token and rank column evaluated from the
// Split-K workspace exactly as the second pass of lora_sgmv_shrink does it
// (zero for tokens without an adapter and for columns from the adapter's rank
// on; otherwise the fixed pairwise tree over the S slices, then one multiply
// by the adapter's shrink scale).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float splits_tree(const float* w, int64_t stride, int split_k)
{
    float v[16];
    switch (split_k) {
    case 1: return w[0];
    case 2:
#pragma unroll
        for (int s = 0; s < 2; ++s)
            v[s] = w[s * stride];
        return pairwise_tree<2>(v);
    case 4:
#pragma unroll
        for (int s = 0; s < 4; ++s)
            v[s] = w[s * stride];
        return pairwise_tree<4>(v);
    case 8:
#pragma unroll
        for (int s = 0; s < 8; ++s)
            v[s] = w[s * stride];
        return pairwise_tree<8>(v);
    default:
#pragma unroll
        for (int s = 0; s < 16; ++s)
            v[s] = w[s * stride];
        return pairwise_tree<16>(v);
    }
}

__device__ __forceinline__ float sgmv_h_value(const TreeParams& c, int64_t row, int col, int split_k)
{
    const int a = c.ids[row];
    if (a < 0 || a >= c.n_adapters)
        return 0.0f;
    int ra = c.ranks[a];
    ra = ra < 0 ? 0 : (ra > c.ncols ? c.ncols : ra);
    if (col >= ra)
        return 0.0f;
    const float scale = c.scales ? c.scales[a] : 1.0f;
    return __fmul_rn(splits_tree(c.ws + row * c.ldw + col, c.split_stride, split_k), scale);
}

// The slot's 4 h values computed from the workspace (and written to c.h when
// write_h), for h_put.
template <int HC>
__device__ __forceinline__ void h_tree(const HStageSlot& s, const TreeParams& c, int64_t row0, int nrows, int r,
                                       int split_k, bool write_h, float (&f)[HC])
{
#pragma unroll
    for (int e = 0; e < HC; ++e)
        f[e] = 0.f;
    if (!s.on || s.row >= nrows)
        return;
#pragma unroll
    for (int e = 0; e < HC; ++e) {
        if (s.col + e < r) {
            f[e] = sgmv_h_value(c, row0 + s.row, s.col + e, split_k);
            if (write_h)
                c.h[(row0 + s.row) * c.ld_h + s.col + e] = f[e];
        }
    }
}

// Multi-adapter, large M: k_expand_rows' tile walk and y movement, with
// k_sgmv_expand's passes per distinct adapter.  Each wave keeps the B
// operands of the last adapter it used and reloads them only when a pass
// needs another one (tokens of one adapter are usually contiguous); the
// staged h tile holds r_max columns and every pass masks it to its adapter's
// rank.  A lane's result goes back into the LDS y tile only in the pass of its
// token's adapter; y rows are read for every token of a tile but written only
// for tokens with an adapter.
// COMBINE: h comes from the Split-K workspace (sgmv_h_value), the first
// column block also writes it out.
// (at most 128 VGPRs below rank 64: four workgroups per CU)
template <int KS, bool COMBINE>
__global__ __launch_bounds__(256, KS == 4 ? 2 : 4) void k_sgmv_expand_rows(ExpandParams p, TreeParams c, int R, int split_k)
{
    __shared__ __align__(16) uint16_t hs[2][kRowBlock * kHbStride];
    __shared__ __align__(16) uint16_t ys[2][kRowBlock * kYStride];
    const uint32_t nblocks = (uint32_t)((p.N + kExpandCols - 1) / kExpandCols);
    const int64_t col0 = (int64_t)(blockIdx.x % nblocks) * kExpandCols;
    const int64_t row_base = (int64_t)(blockIdx.x / nblocks) * kRowBlock * R;
    const int64_t left = (p.M - row_base + kRowBlock - 1) / kRowBlock;
    const int tiles = left < R ? (int)left : R;
    constexpr int HC = KS == 4 ? 8 : 4;          // h columns each staging thread converts
    const HStageSlot slot = h_stage_slot<HC>(p.r_max);
    const YChunk yc = y_chunk();
    const bool col_ok = col0 + yc.col < p.N;
    ExpandLane L = expand_lane(row_base, kRowBlock, col0);
    const bool active = L.n_base < p.N;
    const bool write_h = COMBINE && c.h != nullptr && col0 == 0;
    // raw adapter id of a row of the tile at r0 (-1 outside the tile)
    auto raw_id = [&](int64_t r0, int nrows, int row) { return row < nrows ? p.ids[r0 + row] : -1; };
    auto valid = [&](int a) { return a >= 0 && a < p.n_adapters; };
    // the tile at r0: its y chunk rows, h slot and this lane's token id in flight
    u16x8 g[2];
    float f[HC];
    int ca[2];                                   // adapter ids of the chunk's rows
    auto fetch = [&](int64_t r0, int nrows, int& lane_id) {
#pragma unroll
        for (int e = 0; e < 2; ++e)
            ca[e] = col_ok ? raw_id(r0, nrows, yc.row + 8 * e) : -1;
        lane_id = raw_id(r0, nrows, L.li);
        y_chunk_load(yc, p.y, p.ld_y, r0, col0, y_chunk_rows(yc, nrows, col_ok), g);
        if constexpr (!COMBINE)
            h_load(slot, p.h, p.ld_h, r0, nrows, p.r_max, f);
    };
    // ... put into LDS buffer b; returns the chunk rows to be written back
    auto put = [&](int64_t r0, int nrows, int b) {
        if constexpr (COMBINE)
            h_tree(slot, c, r0, nrows, p.r_max, split_k, write_h, f);
        y_chunk_put(yc, g, ys[b]);
        h_put(slot, f, p.r_max, hs[b]);
        return (unsigned)valid(ca[0]) | (unsigned)valid(ca[1]) << 1;
    };
    int id;
    int nr = tile_rows(p.M, row_base);
    fetch(row_base, nr, id);
    unsigned w_prev = 0;
    unsigned w_cur = put(row_base, nr, 0);
    __syncthreads();
    int cur = -1;                                // adapter whose B operands this wave holds
    int ra = 0;
    float scale = 1.0f;
    bf16x8 bop[4][KS];
    for (int i = 0; i < tiles; ++i) {
        const int64_t row0 = row_base + (int64_t)kRowBlock * i;
        const bool next = i + 1 < tiles;
        const int nr1 = next ? tile_rows(p.M, row0 + kRowBlock) : 0;
        int idn = -1;
        if (next)
            fetch(row0 + kRowBlock, nr1, idn);
        if (i > 0)
            y_chunk_store(yc, ys[(i - 1) & 1], p.y, p.ld_y, row0 - kRowBlock, col0, w_prev);
        if (active) {
            const int lid = valid(id) ? id : -1;
            uint16_t* yl = y_lane(L, ys[i & 1]);
            u16x8 yv[2];
            yv[0] = *reinterpret_cast<const u16x8*>(yl);
            yv[1] = *reinterpret_cast<const u16x8*>(yl + 8);
            bool done = lid < 0;
            for (;;) {
                const uint64_t pending = __ballot(!done);
                if (pending == 0)
                    break;
                const int a = __builtin_amdgcn_readfirstlane(__shfl(lid, __builtin_ctzll(pending)));
                if (a != cur) {
                    cur = a;
                    ra = table_load(p.ranks, a);
                    ra = ra < 0 ? 0 : (ra > p.r_max ? p.r_max : ra);
                    scale = p.scales ? table_load(p.scales, a) : 1.0f;
                    expand_load_b<KS>(L, p.N, table_load(p.B_ptrs, a), (ra + 7) & ~7, ra, bop);
                }
                const bool mine = !done && lid == a;
                ExpandLane La = L;
                La.row_ok = mine;
                u16x8 o[2];
                // the steps the single-adapter expand takes at this rank
                auto mma = [&](auto steps) {
                    constexpr int K2 = decltype(steps)::value;
                    bf16x8 hb[K2];
                    hb_from_tile<K2>(La, hs[i & 1], ra, hb);
                    if constexpr (K2 == KS) {
                        expand_mma<KS>(hb, scale, yv, bop, o);
                    } else {
                        bf16x8 b2[4][K2];
#pragma unroll
                        for (int t = 0; t < 4; ++t)
#pragma unroll
                            for (int ks = 0; ks < K2; ++ks)
                                b2[t][ks] = bop[t][ks];
                        expand_mma<K2>(hb, scale, yv, b2, o);
                    }
                };
                if constexpr (KS == 4) {
                    const int need = expand_steps(ra);
                    if (need == 4)
                        mma(Steps<4>{});
                    else if (need == 2)
                        mma(Steps<2>{});
                    else
                        mma(Steps<1>{});
                } else if (KS == 2 && ra > 32) {            // KS 2: ra <= r_max <= 64
                    bf16x8 hb[KS];
                    hb_from_tile<KS>(La, hs[i & 1], ra, hb);
                    expand_mma<KS>(hb, scale, yv, bop, o);
                } else {
                    bf16x8 hb[1];
                    bf16x8 b1[4][1];
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        b1[t][0] = bop[t][0];
                    hb_from_tile<1>(La, hs[i & 1], ra, hb);
                    expand_mma<1>(hb, scale, yv, b1, o);
                }
                if (mine) {
                    *reinterpret_cast<u16x8*>(yl) = o[0];
                    *reinterpret_cast<u16x8*>(yl + 8) = o[1];
                }
                done = done || mine;
            }
        }
        unsigned w_next = 0;
        if (next)
            w_next = put(row0 + kRowBlock, nr1, (i + 1) & 1);
        __syncthreads();
        w_prev = w_cur;
        w_cur = w_next;
        id = idn;
    }
    y_chunk_store(yc, ys[(tiles - 1) & 1], p.y, p.ld_y, row_base + (int64_t)kRowBlock * (tiles - 1), col0, w_prev);
}

// The 16-row h tile of a block, rows of `rows` only, from the Split-K
// workspace into LDS (and out to c.h when write_h): the row's shrink scale
// times the tree over the S slices below its rank, zeros from there to
// r_max.  Lane li of each wave holds row li's rank and scale.  Every column
// below r_max of a row below M lies in the workspace, so the loads are
// issued without waiting for the rank, and the passes over the tile are
// unrolled to their compile-time bound (r_max <= 32 KS) so that all of a
// thread's loads are in flight together.
template <int S, int KS>
__device__ __forceinline__ void sgmv_h_tile(const TreeParams& c, int64_t row0, uint32_t rows, int ra_l, float sc_l,
                                            bool write_h, float* hs)
{
    constexpr int kPasses = kRowBlock * 32 * KS / 256;
    const int r_max = c.ncols;
    const float rcp_r = __builtin_amdgcn_rcpf((float)r_max);
    const int drow = div_small(256, rcp_r);
    const int dcol = 256 - drow * r_max;
    int row = div_small((int)threadIdx.x, rcp_r);
    int col = (int)threadIdx.x - row * r_max;
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass, row += drow, col += dcol) {
        if (col >= r_max) {
            col -= r_max;
            ++row;
        }
        const int ra = __shfl(ra_l, row & 15);
        const float sc = __shfl(sc_l, row & 15);
        if (row < kRowBlock && ((rows >> row) & 1u)) {
            const float* w = c.ws + (row0 + row) * c.ldw + col;
            float v[S];
#pragma unroll
            for (int s = 0; s < S; ++s)
                v[s] = w[(int64_t)s * c.split_stride];
            const float t = pairwise_tree<S>(v);
            const float hv = col < ra ? __fmul_rn(t, sc) : 0.0f;
            hs[row * kHTileStride + col] = hv;
            if (write_h)
                c.h[(row0 + row) * c.ld_h + col] = hv;
        }
    }
}

// KS: matrix-core steps the kernel is built for (1: r_max <= 32, 2: r_max <= 64,
// 4: r_max <= 128).  COMBINE: the block's h rows are evaluated from the
// Split-K workspace into LDS first (the first column block also writes them
// out).  slots: workgroups per (16-token block, column block).  The block's
// distinct adapters, in order of first appearance, are dealt out to them -
// workgroup j takes the j-th, (j + slots)-th, ... - so the passes of a block
// whose tokens carry many adapters (one adapter per decode token) run on
// different compute units at once instead of one after another; workgroup 0
// also writes the zero h rows of tokens without an adapter.  Every token
// still gets exactly one pass of the single-adapter arithmetic.
template <int KS, bool COMBINE>
__global__ __launch_bounds__(256) void k_sgmv_expand(ExpandParams p, TreeParams c, int split_k, int slots)
{
    __shared__ __align__(16) float hs[COMBINE ? kRowBlock * kHTileStride : 1];
    // slot slowest: the slot-0 workgroups (the only busy ones where a block
    // holds one adapter) come first and spread over all XCDs
    const uint32_t items = gridDim.x / (uint32_t)slots;
    const int slot = (int)(blockIdx.x / items);
    const uint32_t item = blockIdx.x - (uint32_t)slot * items;
    const ExpandItem q = expand_item_at(item, p.M, p.N);
    ExpandLane L = expand_lane(q.row0, q.nrows, q.cb * kExpandCols);
    const bool active = L.n_base < p.N;              // per wave
    int id = -1;
    if (L.row_ok) {
        id = p.ids[L.row];
        id = (id < 0 || id >= p.n_adapters) ? -1 : id;
    }
    // rows (bit li) of this workgroup's adapters, and of tokens without one;
    // lanes li and li + 16 g hold the same token, so lanes 0..15 tell all
    uint32_t mine = 0;
    if (slots == 1) {
        mine = (uint32_t)(__ballot(id >= 0) & 0xFFFFull);
    } else {
        bool done = id < 0;
        for (int k = 0;; ++k) {
            const uint64_t pending = __ballot(!done);
            if (pending == 0)
                break;
            const int a = __shfl(id, __builtin_ctzll(pending));
            const bool same = !done && id == a;
            const uint32_t rows = (uint32_t)(__ballot(same) & 0xFFFFull);
            if (k % slots == slot)
                mine |= rows;
            done = done || same;
        }
    }
    const uint32_t none = (uint32_t)(__ballot(L.row_ok && id < 0) & 0xFFFFull);
    // the h tile's per-row rank and shrink scale, lane li for row li
    int ra_l = 0;
    float sc_l = 0.0f;
    if (COMBINE && id >= 0) {
        ra_l = c.ranks[id];
        ra_l = ra_l < 0 ? 0 : (ra_l > c.ncols ? c.ncols : ra_l);
        sc_l = c.scales ? c.scales[id] : 1.0f;
    }
    ExpandLane Ly = L;
    Ly.row_ok = ((mine >> L.li) & 1u) != 0;
    u16x8 yv[2] = {u16x8{0, 0, 0, 0, 0, 0, 0, 0}, u16x8{0, 0, 0, 0, 0, 0, 0, 0}};
    if (active)
        expand_load_y(Ly, p.y, p.ld_y, p.N, yv);
    const float* hrows = p.h + q.row0 * p.ld_h;
    int64_t ld_hr = p.ld_h;
    if constexpr (COMBINE) {
        const bool write_h = c.h != nullptr && q.cb == 0;
        const uint32_t rows = mine | (slot == 0 ? none : 0u);
        switch (split_k) {
        case 1: sgmv_h_tile<1, KS>(c, q.row0, rows, ra_l, sc_l, write_h, hs); break;
        case 2: sgmv_h_tile<2, KS>(c, q.row0, rows, ra_l, sc_l, write_h, hs); break;
        case 4: sgmv_h_tile<4, KS>(c, q.row0, rows, ra_l, sc_l, write_h, hs); break;
        case 8: sgmv_h_tile<8, KS>(c, q.row0, rows, ra_l, sc_l, write_h, hs); break;
        default: sgmv_h_tile<16, KS>(c, q.row0, rows, ra_l, sc_l, write_h, hs); break;
        }
        __syncthreads();
        hrows = hs;
        ld_hr = kHTileStride;
    }
    if (!active)
        return;
    bool done = !Ly.row_ok;
    for (;;) {
        const uint64_t pending = __ballot(!done);
        if (pending == 0)
            break;
        const int a = __builtin_amdgcn_readfirstlane(__shfl(id, __builtin_ctzll(pending)));
        const bool mine = !done && id == a;
        ExpandLane La = L;
        La.row_ok = mine;
        sgmv_pass<KS>(p, La, hrows, ld_hr, a, yv);
        done = done || mine;
    }
}

}  // namespace

inline dim3 expand_grid(int64_t M, int64_t N)
{
    return dim3((unsigned)(((M + kRowBlock - 1) / kRowBlock) * ((N + kExpandCols - 1) / kExpandCols)));
}

// Tiles per workgroup for the expands, from the one-tile grid size and the
// rank (any choice gives the same bits).  One tile per workgroup keeps small
// grids parallel; walking tiles saves the per-workgroup B loads (16 r bytes
// per column) and moves y row-contiguously through LDS.  The more B a
// workgroup holds, the more tiles pay: measured on MI355X (cold inputs),
// ranks <= 32 are fastest with 2 tiles once the grid exceeds ~1024
// workgroups (4096 x 28672 at rank 16: 88.9 us against 115 us for one tile
// and 106 us for 16), ranks <= 64 with 2 from ~512 workgroups, 3 from ~1536
// and 6 from ~3072 (rank 64, 4096 x 4096: 19.0 us against 34.1 us for one
// tile), ranks <= 128 with up to 8.
int expand_tiles_per_wg(int64_t M, int64_t N, int r)
{
    const int64_t wgs = ((M + kRowBlock - 1) / kRowBlock) * ((N + kExpandCols - 1) / kExpandCols);
    const int steps = expand_steps(r);
    if (steps == 1)
        return wgs <= 1024 ? 1 : 2;
    if (wgs < 512)
        return 1;
    if (wgs < 1536)
        return 2;
    if (wgs < 3072)
        return steps == 2 ? 3 : 4;
    return steps == 2 ? 6 : 8;
}

inline dim3 expand_rows_grid(int64_t M, int64_t N, int R)
{
    const int64_t tiles = (M + kRowBlock - 1) / kRowBlock;
    return dim3((unsigned)(((tiles + R - 1) / R) * ((N + kExpandCols - 1) / kExpandCols)));
}

hipError_t launch_expand_compensated(const ExpandParams& p, hipStream_t st, int tiles_per_wg)
{
    const int R = tiles_per_wg > 0 ? tiles_per_wg : expand_tiles_per_wg(p.M, p.N, p.r);
    if (R > 1) {
        const dim3 grid = expand_rows_grid(p.M, p.N, R);
        switch (expand_steps(p.r)) {
        case 4: hipLaunchKernelGGL(k_expand_comp_rows<4>, grid, dim3(256), 0, st, p, R); break;
        case 2: hipLaunchKernelGGL(k_expand_comp_rows<2>, grid, dim3(256), 0, st, p, R); break;
        default: hipLaunchKernelGGL(k_expand_comp_rows<1>, grid, dim3(256), 0, st, p, R); break;
        }
        return hipGetLastError();
    }
    const dim3 grid = expand_grid(p.M, p.N);
    switch (expand_steps(p.r)) {
    case 4: hipLaunchKernelGGL(k_expand_comp<4>, grid, dim3(256), 0, st, p); break;
    case 2: hipLaunchKernelGGL(k_expand_comp<2>, grid, dim3(256), 0, st, p); break;
    default: hipLaunchKernelGGL(k_expand_comp<1>, grid, dim3(256), 0, st, p); break;
    }
    return hipGetLastError();
}

hipError_t launch_expand(const ExpandParams& p, hipStream_t st, int tiles_per_wg)
{
    dim3 block(256);
    const int R = tiles_per_wg > 0 ? tiles_per_wg : expand_tiles_per_wg(p.M, p.N, p.r);
    if (R > 1) {
        const dim3 grid = expand_rows_grid(p.M, p.N, R);
        switch (expand_steps(p.r)) {
        case 4: hipLaunchKernelGGL(k_expand_rows<4>, grid, block, 0, st, p, R); break;
        case 2: hipLaunchKernelGGL(k_expand_rows<2>, grid, block, 0, st, p, R); break;
        default: hipLaunchKernelGGL(k_expand_rows<1>, grid, block, 0, st, p, R); break;
        }
        return hipGetLastError();
    }
    const dim3 grid = expand_grid(p.M, p.N);
    switch (expand_steps(p.r)) {
    case 4: hipLaunchKernelGGL(k_expand<4>, grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL(k_expand<2>, grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL(k_expand<1>, grid, block, 0, st, p); break;
    }
    return hipGetLastError();
}

template <int KS, int WAVES, int XR>
hipError_t launch_expand_combine_ks(const ExpandParams& p, const TreeParams& c, int S, hipStream_t st)
{
    int64_t rbs = (p.M + kRowBlock - 1) / kRowBlock;
    if (XR > 1)
        rbs = (rbs + XR - 1) / XR * XR;
    const dim3 grid((unsigned)(rbs * ((p.N + WAVES * 64 - 1) / (WAVES * 64))));
    const dim3 block(WAVES * 64);
    switch (S) {
    case 1: hipLaunchKernelGGL((k_expand_combine<KS, 1, WAVES, XR>), grid, block, 0, st, p, c); break;
    case 2: hipLaunchKernelGGL((k_expand_combine<KS, 2, WAVES, XR>), grid, block, 0, st, p, c); break;
    case 4: hipLaunchKernelGGL((k_expand_combine<KS, 4, WAVES, XR>), grid, block, 0, st, p, c); break;
    case 8: hipLaunchKernelGGL((k_expand_combine<KS, 8, WAVES, XR>), grid, block, 0, st, p, c); break;
    default: hipLaunchKernelGGL((k_expand_combine<KS, 16, WAVES, XR>), grid, block, 0, st, p, c); break;
    }
    return hipGetLastError();
}

template <int KS>
hipError_t launch_expand_combine_w(const ExpandParams& p, const TreeParams& c, int S, int waves, int xr,
                                   hipStream_t st)
{
    if (waves == 2)
        return launch_expand_combine_ks<KS, 2, 1>(p, c, S, st);
    if (waves == 8)
        return xr == 8 ? launch_expand_combine_ks<KS, 8, 8>(p, c, S, st)
                       : (xr == 2 ? launch_expand_combine_ks<KS, 8, 2>(p, c, S, st)
                                  : launch_expand_combine_ks<KS, 8, 1>(p, c, S, st));
    return xr == 8 ? launch_expand_combine_ks<KS, 4, 8>(p, c, S, st)
                   : (xr == 2 ? launch_expand_combine_ks<KS, 4, 2>(p, c, S, st)
                              : launch_expand_combine_ks<KS, 4, 1>(p, c, S, st));
}

// Waves per workgroup of the tree + expand kernel.  Every column block
// evaluates its row block's tree again, so narrow blocks pay only where the
// tree is tiny and wide ones where the grid is large.  Measured on MI355X
// (cold inputs, N = 4096, Split-K 8, rank 16 unless noted; 2 / 4 / 8 waves):
// M = 1: 4.55 / 4.70 / 4.74 us; M = 16: 5.02 / 4.85 / 5.14; M = 256: 5.60 /
// 5.10 / 5.41; M = 1024: 8.78 / 8.31 / 8.18, rank 32: 10.5 / 9.26 / 8.71;
// M = 4096: 23.3 / 21.2 / 20.8.  The bits do not depend on it.
static int combine_waves(int64_t M, int64_t N)
{
    if (M <= 4)
        return 2;
    const int64_t wgs = ((M + kRowBlock - 1) / kRowBlock) * ((N + kExpandCols - 1) / kExpandCols);
    return wgs >= 1024 ? 8 : 4;
}

hipError_t launch_expand_combine(const ExpandParams& p, const TreeParams& c, int split_k, hipStream_t st, int waves,
                                 int xcd)
{
    if (waves == 0)
        waves = combine_waves(p.M, p.N);
    // Row blocks kept on one XCD from 64 row blocks on.  Measured on MI355X
    // (cold inputs, N = 4096, Split-K 8; spread over the XCDs / on one):
    // M = 1024, rank 16: 8.25 / 8.07 us, rank 32: 8.74 / 8.58 us; M = 2048,
    // rank 16: 12.3 / 11.9 us; below, no gain (M = 256, rank 64: 7.89 / 8.12).
    // Between, two row groups x four column groups (XR = 2) where the column
    // blocks split evenly.
    const int64_t rbs = (p.M + kRowBlock - 1) / kRowBlock;
    const int64_t nblocks = (p.N + waves * 64 - 1) / (waves * 64);
    int xr = 1;
    if (waves != 2) {
        if (xcd == 8 || (xcd < 0 && rbs >= 64))
            xr = 8;
        else if ((xcd == 2 || (xcd < 0 && rbs >= 8)) && nblocks % (kXcds / 2) == 0)
            xr = 2;
    }
    switch (expand_steps(p.r)) {
    case 4: return launch_expand_combine_w<4>(p, c, split_k, waves, xr, st);
    case 2: return launch_expand_combine_w<2>(p, c, split_k, waves, xr, st);
    default: return launch_expand_combine_w<1>(p, c, split_k, waves, xr, st);
    }
}

// Tiles per workgroup for the multi-adapter expands.  Measured on MI355X:
// the plain expand takes the single-adapter choice up to ~4096 one-tile
// workgroups and up to 16 tiles beyond (4096 x 28672, 32 adapters of ranks 8
// to 64: 16 tiles 106 us, 6 tiles 108 us, 2 tiles 119 us); the expand that
// also evaluates each row's Split-K tree keeps one tile per workgroup below
// ~4096 workgroups, where the staging threads' tree over the workspace would
// serialise more of it (512 x 6144, rank 64, Split-K 8: 2 tiles 28.3 us per
// shrink + expand against 23.5 us).
static int sgmv_tiles_per_wg(int64_t M, int64_t N, int r_max, bool combine)
{
    const int64_t wgs = ((M + kRowBlock - 1) / kRowBlock) * ((N + kExpandCols - 1) / kExpandCols);
    const int wide = wgs < 4096 ? 1 : (int)(wgs / 2048 > 16 ? 16 : wgs / 2048);
    if (combine)
        return wide;
    const int single = expand_tiles_per_wg(M, N, r_max);
    return single > wide ? single : wide;
}

// Workgroups per (16-token block, column block) of the one-tile multi-adapter
// expand.  Small grids (decode: at most 512 one-tile workgroups) take enough
// to bring the grid towards 2048 workgroups, at most 16 (the distinct
// adapters a block can hold) and at most n_adapters; larger grids keep one,
// where blocks hold few adapters and extra workgroups cost more than they
// save.  Measured on MI355X: 32 tokens with 32 rank-64 adapters, N = 4096:
// 31.8 -> 8.2 us; 512 tokens in runs of 1-64 over 4 adapters, N = 6144, two
// workgroups per block: 22.9 -> 25.0 us per shrink + expand, so one there.
static int sgmv_expand_slots(int64_t M, int64_t N, int n_adapters)
{
    const int64_t wgs = ((M + kRowBlock - 1) / kRowBlock) * ((N + kExpandCols - 1) / kExpandCols);
    if (wgs < 1 || wgs > 512 || n_adapters < 2)
        return 1;
    const int64_t s = 2048 / wgs > 16 ? 16 : 2048 / wgs;
    return (int)(s < n_adapters ? s : n_adapters);
}

template <bool COMBINE>
void launch_sgmv_expand_t(const ExpandParams& p, const TreeParams& c, int split_k, hipStream_t st, int R = 0)
{
    if (R <= 0)
        R = sgmv_tiles_per_wg(p.M, p.N, p.r_max, COMBINE);
    if (R > 1) {
        const dim3 grid = expand_rows_grid(p.M, p.N, R);
        switch (expand_steps(p.r_max)) {
        case 4: hipLaunchKernelGGL((k_sgmv_expand_rows<4, COMBINE>), grid, dim3(256), 0, st, p, c, R, split_k); break;
        case 2: hipLaunchKernelGGL((k_sgmv_expand_rows<2, COMBINE>), grid, dim3(256), 0, st, p, c, R, split_k); break;
        default: hipLaunchKernelGGL((k_sgmv_expand_rows<1, COMBINE>), grid, dim3(256), 0, st, p, c, R, split_k); break;
        }
        return;
    }
    const int slots = sgmv_expand_slots(p.M, p.N, p.n_adapters);
    const dim3 grid(expand_grid(p.M, p.N).x * (unsigned)slots);
    switch (expand_steps(p.r_max)) {
    case 4: hipLaunchKernelGGL((k_sgmv_expand<4, COMBINE>), grid, dim3(256), 0, st, p, c, split_k, slots); break;
    case 2: hipLaunchKernelGGL((k_sgmv_expand<2, COMBINE>), grid, dim3(256), 0, st, p, c, split_k, slots); break;
    default: hipLaunchKernelGGL((k_sgmv_expand<1, COMBINE>), grid, dim3(256), 0, st, p, c, split_k, slots); break;
    }
}

hipError_t launch_sgmv_expand(const ExpandParams& p, hipStream_t st, int tiles_per_wg)
{
    launch_sgmv_expand_t<false>(p, TreeParams{}, 1, st, tiles_per_wg);
    return hipGetLastError();
}

hipError_t launch_sgmv_expand_combine(const ExpandParams& p, const TreeParams& c, int split_k, hipStream_t st)
{
    launch_sgmv_expand_t<true>(p, c, split_k, st);
    return hipGetLastError();
}

}  // namespace lora
