// Internal interface between the C entry points (abi.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

constexpr int kRowBlock = 16;                // tokens per matrix-core tile
constexpr int kMaxRank = 128;                // largest adapter rank
constexpr int kMaxRankTiles = 8;             // 16-wide rank tiles of a rank <= kMaxRank
constexpr int kGroupTiles = 4;               // rank tiles one shrink workgroup computes, at most
constexpr int kFusedMaxRank = 64;            // rank bound of the single-launch recompute kernel

// Plan buffer: int32 header [ntiles, M, n_adapters, magic], then ntiles
// entries of kPlanTileInts: first token row0, span 1..16, adapter id (-1 for
// tokens without an adapter), row mask.  The tile's tokens are the rows
// row0 + i (i < span) whose mask bit i is set; the other rows of the span
// belong to other tiles (a 16-token block holding several adapters gives one
// tile per adapter).
constexpr int kPlanHeaderInts = 4;
constexpr int kPlanTileInts = 4;
constexpr int32_t kPlanMagic = 0x4C6F5242;   // "LoRB"
constexpr uint32_t kFullMask = 0xFFFFu;

struct ShrinkParams {
    const uint16_t* x;
    int64_t ld_x;
    const uint16_t* A;              // single adapter: [r][ld_a]
    int64_t ld_a;                   // row stride of A (every adapter for sgmv)
    const uint16_t* const* A_ptrs;  // sgmv: device array of adapter pointers
    const int32_t* ranks;           // sgmv: device ranks
    const int32_t* tiles;           // sgmv: plan buffer
    float* out;                     // workspace or h
    int64_t ld_out;                 // row stride of out
    int64_t split_stride;           // floats between workspace slices
    int64_t M;
    int32_t r;                      // single adapter rank
    int32_t r_max;                  // sgmv rank bound
    int32_t k_chunk;                // K / split_k
    int32_t k_steps;                // matrix-core steps per wave
    int32_t split_k;
    int32_t n_adapters;             // sgmv
    float scale;
    const float* scales;            // sgmv atomic contrast: per-adapter scale (may be null: 1)
};

struct TreeParams {
    const float* ws;
    int64_t split_stride;
    int64_t ldw;
    float* h;
    int64_t ld_h;
    int64_t M;
    int32_t ncols;                  // r (single) or r_max (sgmv)
    float scale;                    // single adapter
    const int32_t* ids;             // sgmv
    const int32_t* ranks;           // sgmv
    const float* scales;            // sgmv (may be null: 1)
    int32_t n_adapters;
};

struct ExpandParams {
    const float* h;
    int64_t ld_h;
    const uint16_t* B;              // single adapter: [N][ld_b]
    int64_t ld_b;
    const uint16_t* const* B_ptrs;  // sgmv
    const int32_t* ranks;           // sgmv
    const float* scales;            // sgmv (may be null: 1)
    const int32_t* ids;             // sgmv: per-token adapter ids
    uint16_t* y;
    int64_t ld_y;
    int64_t M;
    int64_t N;
    int32_t r;
    int32_t r_max;
    int32_t n_adapters;             // sgmv
    float scale;
};

// The four ints of the plan header or of a tile entry, read together and
// tested without short-circuit branches: tested one by one with && and ||,
// they were loaded one after another, each a scalar round trip ahead of the
// work; read at once, the four loads merge into one.
struct PlanInts {
    int32_t v[4];
};

__device__ __forceinline__ PlanInts load_plan_ints(const int32_t* p)
{
    return PlanInts{{p[0], p[1], p[2], p[3]}};
}

// Number of tiles of a plan buffer, or 0 when the buffer was not built by
// lora_sgmv_plan for these M and n_adapters (the kernels then do nothing
// rather than follow stale entries).
__device__ __forceinline__ int plan_tiles(const int32_t* plan, int64_t M, int32_t n_adapters)
{
    const PlanInts h = load_plan_ints(plan);
    const bool ok = (h.v[3] == kPlanMagic) & (h.v[1] == (int32_t)M) & (h.v[2] == n_adapters);
    const int n = h.v[0];
    return !ok || n < 0 ? 0 : (n > M ? (int)M : n);
}

// A tile entry spans 1..16 rows inside [0, M) ...
__device__ __forceinline__ bool tile_rows_ok(const int32_t* t, int64_t M)
{
    return (t[0] >= 0) & (t[1] >= 1) & (t[1] <= kRowBlock) & ((int64_t)t[0] + t[1] <= M);
}

// ... of which the rows whose mask bit is set are the tile's
__device__ __forceinline__ uint32_t tile_mask(const int32_t* t)
{
    return (uint32_t)t[3] & ((1u << t[1]) - 1u);
}

__device__ __forceinline__ bool row_in(uint32_t mask, int row)
{
    return (mask >> row) & 1u;
}

// ... and is computed on only if it also names a valid adapter (tiles of
// tokens without an adapter carry -1).
__device__ __forceinline__ bool tile_ok(const int32_t* t, int64_t M, int32_t n_adapters)
{
    return tile_rows_ok(t, M) & (t[2] >= 0) & (t[2] < n_adapters);
}

// floor(a / r) for 0 <= a < 4096 and 1 <= r <= 128 from the hardware
// reciprocal of r: with a = q r + m, (a + 1/2) / r lies at least 1/(2r)
// >= 1/256 from both q and q + 1, and the product's error (a few ulp of a
// value below 4096, under 1e-3) cannot carry it across either
__device__ __forceinline__ int div_small(int a, float rcp_r)
{
    return (int)(((float)a + 0.5f) * rcp_r);
}

// Per-adapter values (rank, scale) looked up per element by the
// multi-adapter tree come from an LDS copy of the first kAdapterTable entries
// of their device arrays, loaded by all threads at kernel start together
// with the token ids and the workspace slices, instead of one dependent
// global load after the id; ids from kAdapterTable on read the device array.
// Callers put a __syncthreads() between table_fill and table_get.
constexpr int kAdapterTable = 256;

template <typename T>
__device__ __forceinline__ void table_fill(T* lds, const T* src, int32_t n)
{
    if (src == nullptr)
        return;
    const int m = n < kAdapterTable ? n : kAdapterTable;
    for (int t = (int)threadIdx.x; t < m; t += (int)blockDim.x)
        lds[t] = src[t];
}

// Entry a (0 <= a < n of table_fill) of src; `none` when src is null.
template <typename T>
__device__ __forceinline__ T table_get(const T* lds, const T* src, int a, T none)
{
    if (src == nullptr)
        return none;
    return a < kAdapterTable ? lds[a] : src[a];
}

// Single-launch shrink: the per-tile arrival counters and the h it writes.
struct CounterParams {
    int32_t* counters;              // kMaxRankTiles per row block / plan tile, 0 between calls
    float* h;
    int64_t ld_h;
    const float* scales;            // sgmv (may be null: 1)
};

// Single-launch shrink + expand: per 16-token block, `producers` shrink
// workgroups (split_k x rank groups) then `consumers` expand workgroups.
struct StreamParams {
    int32_t* counters;              // (arrivals, departures) per row block, 0 between calls
    int32_t* status;                // set to 1 when an expand workgroup stops waiting
    int32_t producers;
    int32_t consumers;
};

struct FusedParams {
    const uint16_t* x;
    int64_t ld_x;
    const uint16_t* A;
    int64_t ld_a;
    const uint16_t* B;
    int64_t ld_b;
    float* h;                       // may be null
    int64_t ld_h;
    uint16_t* y;
    int64_t ld_y;
    int64_t M;
    int64_t N;
    int32_t r;
    int32_t k_chunk;
    int32_t k_steps;
    float shrink_scale;
    float expand_scale;
};

// group_tiles: rank tiles per workgroup (1 .. rank_tiles; the sgmv kernels take 1, 2 or 4).
hipError_t launch_shrink_partial_ws(const ShrinkParams& p, int waves, int rank_tiles, int group_tiles,
                                    hipStream_t st);
hipError_t launch_shrink_partial_direct(const ShrinkParams& p, int waves, int rank_tiles, int group_tiles,
                                        hipStream_t st);
hipError_t launch_shrink_partial_atomic(const ShrinkParams& p, int waves, int rank_tiles, int group_tiles,
                                        hipStream_t st);
// atomic: the nondeterministic contrast - the same work items, each split's
// partial times the scale (single adapter: p.scale; sgmv: p.scales[adapter])
// added to h = p.out (row stride p.ld_out) with fp32 atomics instead of being
// stored to the workspace.
hipError_t launch_sgmv_shrink_partial(const ShrinkParams& p, int waves, int group_tiles, int grid, hipStream_t st,
                                      bool atomic = false);
// tiles_per_wg 2 or 4: row blocks (plan tiles) per workgroup, all rank tiles together
hipError_t launch_shrink_partial_multi(const ShrinkParams& p, int waves, int rank_tiles, int tiles_per_wg,
                                       hipStream_t st, bool atomic = false);
hipError_t launch_sgmv_shrink_partial_multi(const ShrinkParams& p, int waves, int tiles_per_wg, int grid,
                                            hipStream_t st, bool atomic = false);
// A-in-registers partial kernel for large M: R row blocks (plan tiles) per
// workgroup item; usable when shrink_stream_fits (waves 4 or 8, k_steps 1, 2
// or 4, at most 32 registers of A operands per wave).
constexpr int kStreamMaxRows = 16;             // row blocks per item, at most
bool shrink_stream_fits(int waves, int k_steps, int rank_tiles);
hipError_t launch_shrink_stream(const ShrinkParams& p, int waves, int k_steps, int rank_tiles, int R, int grid,
                                bool sgmv, hipStream_t st, bool atomic = false);
hipError_t launch_shrink_counted(const ShrinkParams& p, const CounterParams& c, int waves, int rank_tiles,
                                 int group_tiles, hipStream_t st);
hipError_t launch_sgmv_shrink_counted(const ShrinkParams& p, const CounterParams& c, int waves, int group_tiles,
                                      int grid, hipStream_t st);
// tiles_per_wg 2 or 4 plan tiles of one adapter per workgroup item, r_max <= 64
hipError_t launch_sgmv_shrink_counted_multi(const ShrinkParams& p, const CounterParams& c, int waves,
                                            int tiles_per_wg, int grid, hipStream_t st);
hipError_t launch_splitk_tree(const TreeParams& p, int split_k, bool sgmv, hipStream_t st);
hipError_t launch_fill_zero(float* h, int64_t ld_h, int64_t M, int ncols, hipStream_t st);

// tiles_per_wg: 16-token tiles per expand workgroup, 0 = expand_tiles_per_wg(M, N)
// (any value gives the same bits).
hipError_t launch_expand(const ExpandParams& p, hipStream_t st, int tiles_per_wg = 0);
hipError_t launch_expand_compensated(const ExpandParams& p, hipStream_t st, int tiles_per_wg = 0);
// waves: 2, 4 or 8 waves (128, 256 or 512 columns) per workgroup, 0 = the
// default rule; xcd: how items meet the XCDs - 8 keeps each row block's
// workgroups on one XCD, 2 splits the XCDs into two row groups x four column
// groups, 1 spreads a row block's column blocks over all XCDs, -1 = the
// default rule (any choice gives the same bits).
hipError_t launch_expand_combine(const ExpandParams& p, const TreeParams& c, int split_k, hipStream_t st,
                                 int waves = 0, int xcd = -1);
hipError_t launch_sgmv_expand(const ExpandParams& p, hipStream_t st, int tiles_per_wg = 0);
hipError_t launch_sgmv_expand_combine(const ExpandParams& p, const TreeParams& c, int split_k, hipStream_t st);
hipError_t launch_shrink_expand_fused(const FusedParams& p, int split_k, int waves, hipStream_t st);
hipError_t launch_shrink_expand_counted(const ShrinkParams& p, const ExpandParams& e, const TreeParams& c,
                                        const StreamParams& q, int waves, int group_tiles, hipStream_t st);

hipError_t launch_sgmv_plan(const int32_t* ids, int64_t M, int32_t n_adapters, int32_t* plan,
                            hipStream_t st);

// Columns of y one expand workgroup covers (4 waves x 64).
constexpr int kExpandCols = 256;

// 16-token tiles one expand workgroup walks (1: one tile per workgroup) for
// rank (bound) r.
int expand_tiles_per_wg(int64_t M, int64_t N, int r);

// XCDs of an MI355X; consecutive workgroup ids of a launch go to different ones.
constexpr int kXcds = 8;

// Workgroups of the single-launch recompute kernel for M tokens, N columns.
int64_t fused_grid(int64_t M, int64_t N);

}  // namespace lora
