// C entry points of liblora_det.so (declared in include/lora_det.h).
//
// Each entry point checks every scalar and pointer on the host first and
// returns a status before touching HIP when anything is off; only then does it
// fill a parameter block and enqueue kernels on the caller's stream.  Nothing
// here allocates, frees or synchronises.
#include "../../include/lora_det.h"
#include "kernels.h"

#include <atomic>
#include <mutex>

using namespace lora;

// Fixed Split-K workspace of lora_shrink_expand_noalloc, for callers that
// cannot allocate: one copy per device, created with the code object and held
// until the process ends.  In host code the name stands for a host-side
// handle, never a device address: the device address comes from
// hipGetSymbolAddress (scratch_for_device) and only that address is passed
// to kernels.
static __device__ __align__(256) float scratch[LORA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;
constexpr int64_t kMaxGrid = (int64_t{1} << 31) - 1;     // workgroups of a 1-D launch

bool aligned16(const void* p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

bool split_ok(int32_t s)
{
    return s == 1 || s == 2 || s == 4 || s == 8 || s == 16;
}

// The static plan: a function of (K, split_k, r) only.
//   k_chunk = K / S;  n = k_chunk / 32 matrix-core steps per split;
//   waves   = the largest power of two <= 8 that divides n;
//   k_steps = n / waves.
int make_plan(int64_t K, int32_t r, int32_t split_k, lora_shrink_plan_t* pl)
{
    if (!split_ok(split_k))
        return LORA_ERR_UNSUPPORTED;
    if (r < 1 || r > kMaxRank)
        return LORA_ERR_UNSUPPORTED;
    if (K <= 0 || K > kMaxDim)
        return LORA_ERR_SHAPE;
    if (K % (32 * (int64_t)split_k) != 0)
        return LORA_ERR_UNSUPPORTED;
    const int64_t kc = K / split_k;
    const int64_t n = kc / 32;
    int w = 8;
    while (n % w != 0)
        w >>= 1;
    pl->split_k = split_k;
    pl->k_chunk = (int32_t)kc;
    pl->waves = w;
    pl->k_steps = (int32_t)(n / w);
    pl->rank_tiles = (r + 15) / 16;
    pl->row_block = kRowBlock;
    return LORA_OK;
}

// Rank tiles per shrink workgroup.  Per-element arithmetic does not depend on
// it; small calls give every 16-wide rank tile its own workgroup (more loads in
// flight across the chip), larger ones keep up to kGroupTiles of a row block's
// rank tiles together so its x rows are read once (twice above rank 64).
// Measured on MI355X (cold inputs): together from 256 (row block, split)
// pairs on (512 x 14336, rank 32: 9.4 against 10.7 us; 512 x 4096, rank 64:
// 6.3 against 7.0 us), apart below (256 x 4096, rank 64: 5.2 against 6.0 us).
int group_tiles_for(int64_t M, int32_t split_k, int rank_tiles)
{
    const int64_t pairs = ((M + kRowBlock - 1) / kRowBlock) * split_k;
    return pairs < 256 ? 1 : (rank_tiles < kGroupTiles ? rank_tiles : kGroupTiles);
}

// Row blocks per shrink workgroup in the two-pass paths (all rank tiles
// together when above 1).  A workgroup reads its rows' x and the split's
// chunk of A; sharing the A loads between 2 or 4 row blocks cuts the
// traffic through the compute units once the grid is large, while small
// grids keep one row block (and one rank tile) per workgroup for memory
// parallelism.  Per-element arithmetic does not depend on it.
int shrink_tiles_per_wg(int64_t M, int32_t split_k)
{
    const int64_t wgs = ((M + kRowBlock - 1) / kRowBlock) * split_k;
    return wgs >= 2048 ? 4 : (wgs >= 512 ? 2 : 1);
}

// Multi-adapter: 1, 2 or 4 rank tiles per workgroup, with M standing in for
// the (device-side) tile count.  Up to 512 work items every rank tile has its
// own workgroup (memory parallelism: 32 decode tokens with one rank-64 adapter
// each are 1024 items once the plan has one tile per token); up to 2048, two
// rank tiles share their x loads, so that the grid fits in one round of
// residency (4 eight-wave workgroups per compute unit); beyond that four.
// Measured on MI355X, 512 tokens x 4096, 4 adapters of rank 64 (~1440 items
// with one rank tile per workgroup): two-pass shrink 10.8 -> 10.6 us,
// single-launch shrink 15.1 -> 12.4 us; with ids drawn per token 16.8 -> 15.4
// and 30.1 -> 22.9 us; four rank tiles per workgroup were slower (11.1 us).
int sgmv_group_tiles(int64_t M, int32_t split_k, int32_t r_max)
{
    const int64_t items = ((M + kRowBlock - 1) / kRowBlock) * split_k * ((r_max + 15) / 16);
    return items <= 512 ? 1 : (items <= 2048 ? 2 : kGroupTiles);
}

// Work items of the multi-adapter shrinks (at most M tiles x split_k x
// kMaxRankTiles) are counted in 32 bits.
bool sgmv_items_fit(int64_t M, int32_t split_k)
{
    return M * split_k * kMaxRankTiles <= kMaxGrid;
}

int sgmv_grid(int64_t M, int32_t split_k, int32_t r_max, int group_tiles)
{
    const int64_t groups = ((r_max + 15) / 16 + group_tiles - 1) / group_tiles;
    const int64_t bound = M * split_k * groups;
    return (int)(bound < 4096 ? bound : 4096);
}

int launch_status(hipError_t e)
{
    return e == hipSuccess ? LORA_OK : LORA_ERR_LAUNCH;
}

// Row blocks per item of the A-in-registers partial kernel, or 0 when it is
// not used: it needs short wave chains (shrink_stream_fits) and at least 1024
// (row block, split) pairs, and takes one row block per 256 pairs, 4 to 16.
// Measured on MI355X (cold inputs): 1024 x 8192, rank 64, Split-K 16: 10.0 us
// against 11.4 us for two row blocks per workgroup; 4096 x 4096, rank 64: 8
// row blocks 15.0 us, 4 16.1 us; 4096 x 8192, rank 16, Split-K 16: 16 row
// blocks 18.9 us, 8 20.4 us.  Per-element arithmetic does not depend on it.
int stream_rows_per_item(int64_t tiles, const lora_shrink_plan_t& pl)
{
    if (!shrink_stream_fits(pl.waves, pl.k_steps, pl.rank_tiles) || tiles * pl.split_k < 1024)
        return 0;
    const int64_t R = tiles * pl.split_k / 256;
    return R < 4 ? 4 : (R > 16 ? 16 : (int)R);
}

// The Split-K partial kernel of the deterministic two-pass paths; with
// `atomic`, the same kernel and work items for the nondeterministic contrast,
// each split's scaled partial atomically added into p.out = h.
hipError_t launch_partials(const ShrinkParams& p, const lora_shrink_plan_t& pl, int64_t M, int32_t split_k,
                           hipStream_t st, bool atomic = false)
{
    const int64_t tiles = (M + kRowBlock - 1) / kRowBlock;
    const int R = stream_rows_per_item(tiles, pl);
    if (R > 0)
        return launch_shrink_stream(p, pl.waves, pl.k_steps, pl.rank_tiles, R,
                                    (int)((tiles + R - 1) / R * split_k), false, st, atomic);
    // several row blocks per workgroup hold all rank tiles at once: ranks <= 64
    const int T = pl.rank_tiles <= kGroupTiles ? shrink_tiles_per_wg(M, split_k) : 1;
    if (T > 1)
        return launch_shrink_partial_multi(p, pl.waves, pl.rank_tiles, T, st, atomic);
    const int gt = group_tiles_for(M, split_k, pl.rank_tiles);
    return atomic ? launch_shrink_partial_atomic(p, pl.waves, pl.rank_tiles, gt, st)
                  : launch_shrink_partial_ws(p, pl.waves, pl.rank_tiles, gt, st);
}

// Checks shared by the single-adapter shrinks.
int check_shrink(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a, const float* h,
                 int64_t ld_h, int64_t M, int64_t K, int32_t r, int32_t split_k, lora_shrink_plan_t* pl)
{
    if (M < 0 || M > kMaxDim)
        return LORA_ERR_SHAPE;
    int st = make_plan(K, r, split_k, pl);
    if (st != LORA_OK)
        return st;
    if (((M + kRowBlock - 1) / kRowBlock) * split_k * pl->rank_tiles > kMaxGrid)
        return LORA_ERR_SHAPE;
    if (M == 0)
        return LORA_OK;
    if (!x || !A || !h)
        return LORA_ERR_NULL;
    if (ld_x < K || ld_a < K || ld_h < r)
        return LORA_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(A) || (reinterpret_cast<uintptr_t>(h) & 3u) || ld_x % 8 || ld_a % 8)
        return LORA_ERR_ALIGN;
    return LORA_OK;
}

ShrinkParams shrink_params(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a, int64_t M,
                           int32_t r, const lora_shrink_plan_t& pl, float scale)
{
    ShrinkParams p{};
    p.x = x;
    p.ld_x = ld_x;
    p.A = A;
    p.ld_a = ld_a;
    p.M = M;
    p.r = r;
    p.r_max = r;
    p.k_chunk = pl.k_chunk;
    p.k_steps = pl.k_steps;
    p.split_k = pl.split_k;
    p.scale = scale;
    return p;
}

size_t workspace_bytes(int64_t M, int32_t cols, int32_t split_k)
{
    if (M < 0 || M > kMaxDim || cols < 1 || cols > kMaxRank || !split_ok(split_k))
        return 0;
    return (size_t)split_k * (size_t)M * (size_t)cols * sizeof(float);
}

// Checks shared by the single-adapter shrink + expand entry points.
int check_shrink_expand(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a, const uint16_t* B,
                        int64_t ld_b, const float* h, int64_t ld_h, const uint16_t* y, int64_t ld_y, int64_t M,
                        int64_t K, int32_t r, int64_t N, int32_t split_k, lora_shrink_plan_t* pl)
{
    if (M < 0 || M > kMaxDim || N < 0 || N > kMaxDim)
        return LORA_ERR_SHAPE;
    int st = make_plan(K, r, split_k, pl);
    if (st != LORA_OK)
        return st;
    if (N % 8 != 0)
        return LORA_ERR_UNSUPPORTED;
    if (((M + kRowBlock - 1) / kRowBlock) * ((N + kExpandCols - 1) / kExpandCols) > kMaxGrid ||
        ((M + kRowBlock - 1) / kRowBlock) * split_k * pl->rank_tiles > kMaxGrid)
        return LORA_ERR_SHAPE;
    if (M == 0 || N == 0)
        return LORA_OK;
    if (!x || !A || !B || !y)
        return LORA_ERR_NULL;
    if (ld_x < K || ld_a < K || ld_b < r || ld_y < N || (h && ld_h < r))
        return LORA_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(y) ||
        (reinterpret_cast<uintptr_t>(h) & 3u) || ld_x % 8 || ld_a % 8 || ld_b % 8 || ld_y % 8)
        return LORA_ERR_ALIGN;
    return LORA_OK;
}

// Which schedule lora_shrink_expand runs.  Both give the same bits (same
// chunks, chains, trees and expand arithmetic).  The single launch makes every
// workgroup (16 tokens x 512 columns) re-read the whole of A, K * r * 2 bytes,
// through one compute unit; that beats a second dependent launch only while A
// is small (measured on MI355X: at K = 4096, r = 16, i.e. 128 KiB, the two
// launches are faster at every M).
bool use_single_launch(int64_t M, int64_t K, int32_t r, int64_t N)
{
    (void)N;
    return M <= 64 && r <= kFusedMaxRank && K * r * 2 <= 32 * 1024;
}

// Whether lora_shrink_expand's two-launch schedule evaluates the Split-K tree
// inside the expand.  Every column block evaluates its rows' tree again, so
// this holds only while column blocks x splits stays small and the h values
// those re-evaluations produce, M r per column block, stay below 2^19;
// otherwise the tree kernel writes h once and the tile-walking expand reads
// it.  Measured on MI355X (N = 4096, Split-K 8, cold inputs; tree in the
// expand / tree kernel + expand): M = 1024, r = 32, K = 14336: 20.3 / 21.8
// us; M = 2048: 33.9 / 33.4 us; M = 4096: 59.0 / 56.1 us; M = 2048, r = 64,
// K = 4096: 29.6 / 24.4 us.  Same bits either way.
bool tree_in_expand(int64_t M, int32_t r, int64_t N, int32_t split_k)
{
    const int64_t nblocks = (N + kExpandCols - 1) / kExpandCols;
    return nblocks * split_k <= 256 && M * r * nblocks <= (int64_t{1} << 19);
}

int launch_fused(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a, const uint16_t* B,
                 int64_t ld_b, float* h, int64_t ld_h, uint16_t* y, int64_t ld_y, int64_t M, int32_t r, int64_t N,
                 const lora_shrink_plan_t& pl, float shrink_scale, float expand_scale, void* stream)
{
    if (fused_grid(M, N) > kMaxGrid)
        return LORA_ERR_SHAPE;
    FusedParams p{};
    p.x = x;
    p.ld_x = ld_x;
    p.A = A;
    p.ld_a = ld_a;
    p.B = B;
    p.ld_b = ld_b;
    p.h = h;
    p.ld_h = ld_h;
    p.y = y;
    p.ld_y = ld_y;
    p.M = M;
    p.N = N;
    p.r = r;
    p.k_chunk = pl.k_chunk;
    p.k_steps = pl.k_steps;
    p.shrink_scale = shrink_scale;
    p.expand_scale = expand_scale;
    return launch_status(launch_shrink_expand_fused(p, pl.split_k, pl.waves, static_cast<hipStream_t>(stream)));
}

// The partial kernel of the multi-adapter two-pass shrink (arguments checked).
// With `atomic` (the nondeterministic contrast) the same kernel and work items
// add each split's partial times the adapter's scale into h (`workspace` is
// then h, with row stride ld_h) instead of storing it.
int launch_sgmv_partials(const uint16_t* x, int64_t ld_x, const uint16_t* const* A_ptrs, int64_t ld_a,
                         const int32_t* ranks, int32_t n_adapters, const void* plan, int64_t M, int32_t r_max,
                         const lora_shrink_plan_t& pl, void* workspace, hipStream_t s, bool atomic = false,
                         const float* scales = nullptr, int64_t ld_h = 0)
{
    ShrinkParams p{};
    p.x = x;
    p.ld_x = ld_x;
    p.ld_a = ld_a;
    p.A_ptrs = A_ptrs;
    p.ranks = ranks;
    p.tiles = static_cast<const int32_t*>(plan);
    p.out = static_cast<float*>(workspace);
    p.ld_out = atomic ? ld_h : r_max;
    p.split_stride = atomic ? 0 : M * r_max;
    p.scales = scales;
    p.M = M;
    p.r = r_max;
    p.r_max = r_max;
    p.k_chunk = pl.k_chunk;
    p.k_steps = pl.k_steps;
    p.split_k = pl.split_k;
    p.n_adapters = n_adapters;
    p.scale = 1.0f;
    // Tiles never exceed M; the grid is a fixed bound, idle workgroups exit.
    // The A-in-registers kernel is sized for about M / 16 + n_adapters tiles
    // (runs of one adapter); its workgroups take further items when the plan
    // has more.
    const int64_t est = (M + kRowBlock - 1) / kRowBlock + n_adapters;
    lora_shrink_plan_t ps = pl;
    ps.rank_tiles = (r_max + 15) / 16;
    const int R = stream_rows_per_item(est, ps);
    if (R > 0) {
        const int64_t grid = (est + R - 1) / R * pl.split_k;
        return launch_status(launch_shrink_stream(p, pl.waves, pl.k_steps, ps.rank_tiles, R,
                                                  (int)(grid < 65536 ? grid : 65536 / pl.split_k * pl.split_k),
                                                  true, s, atomic));
    }
    const int T = r_max <= 16 * kGroupTiles ? shrink_tiles_per_wg(M, pl.split_k) : 1;
    if (T > 1) {
        const int64_t bound = (M + T - 1) / T * pl.split_k;
        return launch_status(
            launch_sgmv_shrink_partial_multi(p, pl.waves, T, (int)(bound < 2048 ? bound : 2048), s, atomic));
    }
    const int gt = sgmv_group_tiles(M, pl.split_k, r_max);
    const int grid = sgmv_grid(M, pl.split_k, r_max, gt);
    return launch_status(launch_sgmv_shrink_partial(p, pl.waves, gt, grid, s, atomic));
}

// Second pass of the multi-adapter shrink over a [split_k][M][r_max] workspace.
TreeParams sgmv_tree_params(void* workspace, int64_t M, int32_t r_max, float* h, int64_t ld_h,
                            const int32_t* token_adapter, const int32_t* ranks, const float* scales,
                            int32_t n_adapters)
{
    TreeParams t{};
    t.ws = static_cast<const float*>(workspace);
    t.split_stride = M * r_max;
    t.ldw = r_max;
    t.h = h;
    t.ld_h = ld_h;
    t.M = M;
    t.ncols = r_max;
    t.scale = 1.0f;
    t.ids = token_adapter;
    t.ranks = ranks;
    t.scales = scales;
    t.n_adapters = n_adapters;
    return t;
}

int expand_entry(const float* h, int64_t ld_h, const uint16_t* B, int64_t ld_b, uint16_t* y, int64_t ld_y,
                 int64_t M, int32_t r, int64_t N, float scale, bool compensated, void* stream)
{
    if (M < 0 || M > kMaxDim || N < 0 || N > kMaxDim)
        return LORA_ERR_SHAPE;
    if (r < 1 || r > kMaxRank)
        return LORA_ERR_UNSUPPORTED;
    if (N % 8 != 0)
        return LORA_ERR_UNSUPPORTED;
    if (((M + kRowBlock - 1) / kRowBlock) * ((N + kExpandCols - 1) / kExpandCols) > kMaxGrid)
        return LORA_ERR_SHAPE;
    if (M == 0 || N == 0)
        return LORA_OK;
    if (!h || !B || !y)
        return LORA_ERR_NULL;
    if (ld_h < r || ld_b < r || ld_y < N)
        return LORA_ERR_SHAPE;
    if (!aligned16(h) || !aligned16(B) || !aligned16(y) || ld_h % 4 || ld_b % 8 || ld_y % 8)
        return LORA_ERR_ALIGN;
    ExpandParams p{};
    p.h = h;
    p.ld_h = ld_h;
    p.B = B;
    p.ld_b = ld_b;
    p.y = y;
    p.ld_y = ld_y;
    p.M = M;
    p.N = N;
    p.r = r;
    p.r_max = r;
    p.scale = scale;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    return launch_status(compensated ? launch_expand_compensated(p, st) : launch_expand(p, st));
}


// Device address of `scratch` on `dev`, looked up once per device with that
// device current (hipGetSymbolAddress) and cached; later calls read the cache
// without a lock.
constexpr int kScratchMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kScratchMaxDevices];
std::mutex g_scratch_lock;

int scratch_for_device(int dev, void** out)
{
    if (dev < 0 || dev >= kScratchMaxDevices)
        return LORA_ERR_LAUNCH;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> guard(g_scratch_lock);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            int prev = -1;
            if (hipGetDevice(&prev) != hipSuccess)
                return LORA_ERR_LAUNCH;
            if (prev != dev && hipSetDevice(dev) != hipSuccess)
                return LORA_ERR_LAUNCH;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (prev != dev)
                (void)hipSetDevice(prev);
            if (e != hipSuccess || p == nullptr)
                return LORA_ERR_LAUNCH;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return LORA_OK;
}

}  // namespace

extern "C" {
// The library is built with hidden visibility; the entry points below are
// its exported interface.
#pragma GCC visibility push(default)

int lora_abi_version(void)
{
    return LORA_DET_ABI_VERSION;
}

const char* lora_status_str(int status)
{
    switch (status) {
    case LORA_OK: return "ok";
    case LORA_ERR_NULL: return "null pointer";
    case LORA_ERR_SHAPE: return "bad shape or leading dimension";
    case LORA_ERR_UNSUPPORTED: return "unsupported rank, split count or K";
    case LORA_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case LORA_ERR_WORKSPACE: return "workspace or plan buffer too small";
    case LORA_ERR_LAUNCH: return "kernel launch failed";
    case LORA_ERR_SCRATCH: return "needs more than the library's fixed scratch buffer";
    default: return "unknown status";
    }
}

int lora_shrink_plan(int64_t K, int32_t r, int32_t split_k, lora_shrink_plan_t* plan)
{
    if (!plan)
        return LORA_ERR_NULL;
    lora_shrink_plan_t pl;
    const int st = make_plan(K, r, split_k, &pl);
    if (st == LORA_OK)
        *plan = pl;
    return st;
}

size_t lora_shrink_workspace_bytes(int64_t M, int32_t r, int32_t split_k)
{
    if (split_k == 1)
        return 0;
    return workspace_bytes(M, r, split_k);
}

int lora_shrink_splitk(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a, float* h,
                       int64_t ld_h, int64_t M, int64_t K, int32_t r, int32_t split_k, float scale,
                       void* workspace, size_t ws_bytes, void* stream)
{
    lora_shrink_plan_t pl;
    int st = check_shrink(x, ld_x, A, ld_a, h, ld_h, M, K, r, split_k, &pl);
    if (st != LORA_OK || M == 0)
        return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    ShrinkParams p = shrink_params(x, ld_x, A, ld_a, M, r, pl, scale);
    if (split_k == 1) {
        p.out = h;
        p.ld_out = ld_h;
        return launch_status(launch_shrink_partial_direct(p, pl.waves, pl.rank_tiles,
                                                          group_tiles_for(M, split_k, pl.rank_tiles), s));
    }
    const size_t need = lora_shrink_workspace_bytes(M, r, split_k);
    if (!workspace)
        return LORA_ERR_NULL;
    if (!aligned16(workspace))
        return LORA_ERR_ALIGN;
    if (ws_bytes < need)
        return LORA_ERR_WORKSPACE;
    p.out = static_cast<float*>(workspace);
    p.ld_out = r;
    p.split_stride = M * r;
    st = launch_status(launch_partials(p, pl, M, split_k, s));
    if (st != LORA_OK)
        return st;
    TreeParams t{};
    t.ws = static_cast<const float*>(workspace);
    t.split_stride = M * r;
    t.ldw = r;
    t.h = h;
    t.ld_h = ld_h;
    t.M = M;
    t.ncols = r;
    t.scale = scale;
    return launch_status(launch_splitk_tree(t, split_k, false, s));
}

int lora_shrink_splitk_atomic(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a, float* h,
                              int64_t ld_h, int64_t M, int64_t K, int32_t r, int32_t split_k, float scale,
                              void* stream)
{
    lora_shrink_plan_t pl;
    int st = check_shrink(x, ld_x, A, ld_a, h, ld_h, M, K, r, split_k, &pl);
    if (st != LORA_OK || M == 0)
        return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = launch_status(launch_fill_zero(h, ld_h, M, r, s));
    if (st != LORA_OK)
        return st;
    ShrinkParams p = shrink_params(x, ld_x, A, ld_a, M, r, pl, scale);
    p.out = h;
    p.ld_out = ld_h;
    p.split_stride = 0;
    return launch_status(launch_partials(p, pl, M, split_k, s, true));
}


int lora_expand(const float* h, int64_t ld_h, const uint16_t* B, int64_t ld_b, uint16_t* y, int64_t ld_y,
                int64_t M, int32_t r, int64_t N, float scale, void* stream)
{
    return expand_entry(h, ld_h, B, ld_b, y, ld_y, M, r, N, scale, false, stream);
}

int lora_expand_compensated(const float* h, int64_t ld_h, const uint16_t* B, int64_t ld_b, uint16_t* y,
                            int64_t ld_y, int64_t M, int32_t r, int64_t N, float scale, void* stream)
{
    return expand_entry(h, ld_h, B, ld_b, y, ld_y, M, r, N, scale, true, stream);
}

size_t lora_shrink_expand_workspace_bytes(int64_t M, int32_t r, int32_t split_k)
{
    return workspace_bytes(M, r, split_k);
}

int lora_shrink_partials(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a, int64_t M, int64_t K,
                         int32_t r, int32_t split_k, void* workspace, size_t ws_bytes, void* stream)
{
    if (M < 0 || M > kMaxDim)
        return LORA_ERR_SHAPE;
    lora_shrink_plan_t pl;
    int st = make_plan(K, r, split_k, &pl);
    if (st != LORA_OK)
        return st;
    if (((M + kRowBlock - 1) / kRowBlock) * split_k * pl.rank_tiles > kMaxGrid)
        return LORA_ERR_SHAPE;
    if (M == 0)
        return LORA_OK;
    if (!x || !A || !workspace)
        return LORA_ERR_NULL;
    if (ld_x < K || ld_a < K)
        return LORA_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(A) || !aligned16(workspace) || ld_x % 8 || ld_a % 8)
        return LORA_ERR_ALIGN;
    if (ws_bytes < workspace_bytes(M, r, split_k))
        return LORA_ERR_WORKSPACE;
    ShrinkParams sp = shrink_params(x, ld_x, A, ld_a, M, r, pl, 1.0f);
    sp.out = static_cast<float*>(workspace);
    sp.ld_out = r;
    sp.split_stride = M * r;
    return launch_status(launch_partials(sp, pl, M, split_k, static_cast<hipStream_t>(stream)));
}

int lora_expand_combine(const void* workspace, size_t ws_bytes, int32_t split_k, float shrink_scale,
                        const uint16_t* B, int64_t ld_b, float* h, int64_t ld_h, uint16_t* y, int64_t ld_y,
                        int64_t M, int32_t r, int64_t N, float expand_scale, void* stream)
{
    if (M < 0 || M > kMaxDim || N < 0 || N > kMaxDim)
        return LORA_ERR_SHAPE;
    if (!split_ok(split_k) || r < 1 || r > kMaxRank || N % 8 != 0)
        return LORA_ERR_UNSUPPORTED;
    if (((M + kRowBlock - 1) / kRowBlock) * ((N + kExpandCols - 1) / kExpandCols) > kMaxGrid)
        return LORA_ERR_SHAPE;
    if (M == 0 || N == 0)
        return LORA_OK;
    if (!workspace || !B || !y)
        return LORA_ERR_NULL;
    if (ld_b < r || ld_y < N || (h && ld_h < r))
        return LORA_ERR_SHAPE;
    if (!aligned16(workspace) || !aligned16(B) || !aligned16(y) || (reinterpret_cast<uintptr_t>(h) & 3u) ||
        ld_b % 8 || ld_y % 8)
        return LORA_ERR_ALIGN;
    if (ws_bytes < workspace_bytes(M, r, split_k))
        return LORA_ERR_WORKSPACE;
    TreeParams t{};
    t.ws = static_cast<const float*>(workspace);
    t.split_stride = M * r;
    t.ldw = r;
    t.h = h;
    t.ld_h = ld_h;
    t.M = M;
    t.ncols = r;
    t.scale = shrink_scale;
    ExpandParams ep{};
    ep.B = B;
    ep.ld_b = ld_b;
    ep.y = y;
    ep.ld_y = ld_y;
    ep.M = M;
    ep.N = N;
    ep.r = r;
    ep.r_max = r;
    ep.scale = expand_scale;
    return launch_status(launch_expand_combine(ep, t, split_k, static_cast<hipStream_t>(stream)));
}

int lora_shrink_expand_launches(int64_t M, int64_t K, int32_t r, int64_t N, int32_t split_k)
{
    lora_shrink_plan_t pl;
    if (M < 0 || N < 0 || make_plan(K, r, split_k, &pl) != LORA_OK)
        return -LORA_ERR_UNSUPPORTED;
    if (M == 0 || N == 0)
        return 0;
    return use_single_launch(M, K, r, N) ? 1 : (tree_in_expand(M, r, N, split_k) ? 2 : 3);
}

int lora_shrink_expand_fused(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a, const uint16_t* B,
                             int64_t ld_b, float* h, int64_t ld_h, uint16_t* y, int64_t ld_y, int64_t M, int64_t K,
                             int32_t r, int64_t N, int32_t split_k, float shrink_scale, float expand_scale,
                             void* stream)
{
    if (r > kFusedMaxRank)
        return LORA_ERR_UNSUPPORTED;
    lora_shrink_plan_t pl;
    const int st = check_shrink_expand(x, ld_x, A, ld_a, B, ld_b, h, ld_h, y, ld_y, M, K, r, N, split_k, &pl);
    if (st != LORA_OK || M == 0 || N == 0)
        return st;
    return launch_fused(x, ld_x, A, ld_a, B, ld_b, h, ld_h, y, ld_y, M, r, N, pl, shrink_scale, expand_scale,
                        stream);
}

int lora_shrink_expand(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a, const uint16_t* B,
                       int64_t ld_b, float* h, int64_t ld_h, uint16_t* y, int64_t ld_y, int64_t M, int64_t K,
                       int32_t r, int64_t N, int32_t split_k, float shrink_scale, float expand_scale,
                       void* workspace, size_t ws_bytes, void* stream)
{
    // all checks of both halves before the first launch
    if (M < 0 || M > kMaxDim || N < 0 || N > kMaxDim)
        return LORA_ERR_SHAPE;
    lora_shrink_plan_t pl;
    int st = make_plan(K, r, split_k, &pl);
    if (st != LORA_OK)
        return st;
    if (N % 8 != 0)
        return LORA_ERR_UNSUPPORTED;
    if (((M + kRowBlock - 1) / kRowBlock) * ((N + kExpandCols - 1) / kExpandCols) > kMaxGrid)
        return LORA_ERR_SHAPE;
    if (M == 0 || N == 0)
        return LORA_OK;
    if (!x || !A || !B || !y || !workspace)
        return LORA_ERR_NULL;
    if (ld_x < K || ld_a < K || ld_b < r || ld_y < N || (h && ld_h < r))
        return LORA_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(y) || !aligned16(workspace) ||
        (reinterpret_cast<uintptr_t>(h) & 3u) || ld_x % 8 || ld_a % 8 || ld_b % 8 || ld_y % 8)
        return LORA_ERR_ALIGN;
    if (ws_bytes < workspace_bytes(M, r, split_k))
        return LORA_ERR_WORKSPACE;
    if (use_single_launch(M, K, r, N)) {
        return launch_fused(x, ld_x, A, ld_a, B, ld_b, h, ld_h, y, ld_y, M, r, N, pl, shrink_scale, expand_scale,
                            stream);
    }
    st = lora_shrink_partials(x, ld_x, A, ld_a, M, K, r, split_k, workspace, ws_bytes, stream);
    if (st != LORA_OK)
        return st;
    // Tree in the expand (tree_in_expand), or the tree kernel writing h once -
    // into the caller's h, or in place into workspace slice 0 - and the expand
    // reading it (which needs 16-byte h rows).
    float* hh = h ? h : static_cast<float*>(workspace);
    const int64_t ldh = h ? ld_h : r;
    if (tree_in_expand(M, r, N, split_k) || !aligned16(hh) || ldh % 4 != 0)
        return lora_expand_combine(workspace, ws_bytes, split_k, shrink_scale, B, ld_b, h, ld_h, y, ld_y, M, r, N,
                                   expand_scale, stream);
    TreeParams t{};
    t.ws = static_cast<const float*>(workspace);
    t.split_stride = M * r;
    t.ldw = r;
    t.h = hh;
    t.ld_h = ldh;
    t.M = M;
    t.ncols = r;
    t.scale = shrink_scale;
    st = launch_status(launch_splitk_tree(t, split_k, false, static_cast<hipStream_t>(stream)));
    if (st != LORA_OK)
        return st;
    return lora_expand(hh, ldh, B, ld_b, y, ld_y, M, r, N, expand_scale, stream);
}

int lora_shrink_expand_noalloc(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a,
                               const uint16_t* B, int64_t ld_b, float* h, int64_t ld_h, uint16_t* y,
                               int64_t ld_y, int64_t M, int64_t K, int32_t r, int64_t N, int32_t split_k,
                               float shrink_scale, float expand_scale, void* stream)
{
    // sizes first: a call the fixed buffer cannot hold is refused before any
    // HIP call, whatever the pointers
    if (M < 0 || M > kMaxDim || N < 0 || N > kMaxDim)
        return LORA_ERR_SHAPE;
    lora_shrink_plan_t pl;
    const int st = make_plan(K, r, split_k, &pl);
    if (st != LORA_OK)
        return st;
    const size_t need = workspace_bytes(M, r, split_k);
    if (need > LORA_NOALLOC_SCRATCH_BYTES)
        return LORA_ERR_SCRATCH;
    if (M == 0 || N == 0)
        return LORA_OK;
    if (!x || !A || !B || !y)
        return LORA_ERR_NULL;
    int dev = -1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((s != nullptr ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess)
        return LORA_ERR_LAUNCH;
    void* ws = nullptr;
    const int sc = scratch_for_device(dev, &ws);
    if (sc != LORA_OK)
        return sc;
    // the two-pass schedules write every workspace element they read, so the
    // buffer needs no clearing between calls
    return lora_shrink_expand(x, ld_x, A, ld_a, B, ld_b, h, ld_h, y, ld_y, M, K, r, N, split_k, shrink_scale,
                              expand_scale, ws, LORA_NOALLOC_SCRATCH_BYTES, stream);
}

size_t lora_shrink_expand_counter_bytes(int64_t M)
{
    if (M < 0 || M > kMaxDim)
        return 0;
    return 16 + (size_t)8 * (size_t)((M + kRowBlock - 1) / kRowBlock);
}

int lora_shrink_expand_counted(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a, const uint16_t* B,
                               int64_t ld_b, float* h, int64_t ld_h, uint16_t* y, int64_t ld_y, int64_t M,
                               int64_t K, int32_t r, int64_t N, int32_t split_k, float shrink_scale,
                               float expand_scale, void* workspace, size_t ws_bytes, int32_t* counters,
                               size_t counter_bytes, void* stream)
{
    lora_shrink_plan_t pl;
    int st = check_shrink_expand(x, ld_x, A, ld_a, B, ld_b, h, ld_h, y, ld_y, M, K, r, N, split_k, &pl);
    if (st != LORA_OK)
        return st;
    // per row block: split_k x groups shrink workgroups, then one expand
    // workgroup per waves x 64 columns
    const int gt = group_tiles_for(M, split_k, pl.rank_tiles);
    const int64_t producers = (int64_t)split_k * ((pl.rank_tiles + gt - 1) / gt);
    const int64_t consumers = (N + pl.waves * 64 - 1) / (pl.waves * 64);
    if (((M + kRowBlock - 1) / kRowBlock) * (producers + consumers) > kMaxGrid)
        return LORA_ERR_SHAPE;
    if (M == 0 || N == 0)
        return LORA_OK;
    if (!workspace || !counters)
        return LORA_ERR_NULL;
    if (!aligned16(workspace) || (reinterpret_cast<uintptr_t>(counters) & 3u))
        return LORA_ERR_ALIGN;
    if (ws_bytes < workspace_bytes(M, r, split_k) || counter_bytes < lora_shrink_expand_counter_bytes(M))
        return LORA_ERR_WORKSPACE;
    ShrinkParams sp = shrink_params(x, ld_x, A, ld_a, M, r, pl, 1.0f);
    sp.out = static_cast<float*>(workspace);
    sp.ld_out = r;
    sp.split_stride = M * r;
    TreeParams t{};
    t.ws = static_cast<const float*>(workspace);
    t.split_stride = M * r;
    t.ldw = r;
    t.h = h;
    t.ld_h = ld_h;
    t.M = M;
    t.ncols = r;
    t.scale = shrink_scale;
    ExpandParams ep{};
    ep.B = B;
    ep.ld_b = ld_b;
    ep.y = y;
    ep.ld_y = ld_y;
    ep.M = M;
    ep.N = N;
    ep.r = r;
    ep.r_max = r;
    ep.scale = expand_scale;
    StreamParams q{};
    q.status = counters;
    q.counters = counters + 4;
    q.producers = (int32_t)producers;
    q.consumers = (int32_t)consumers;
    return launch_status(launch_shrink_expand_counted(sp, ep, t, q, pl.waves, gt, static_cast<hipStream_t>(stream)));
}

size_t lora_counted_workspace_bytes(int64_t M, int32_t r_max, int32_t split_k)
{
    const size_t w = workspace_bytes(M, r_max, split_k);
    return w > SIZE_MAX / 2 ? 0 : 2 * w;
}

size_t lora_shrink_counter_bytes(int64_t M)
{
    if (M < 0 || M > kMaxDim)
        return 0;
    return (size_t)4 * kMaxRankTiles * (size_t)((M + kRowBlock - 1) / kRowBlock);
}

int lora_shrink_splitk_counted(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a, float* h,
                               int64_t ld_h, int64_t M, int64_t K, int32_t r, int32_t split_k, float scale,
                               void* workspace, size_t ws_bytes, int32_t* counters, size_t counter_bytes,
                               void* stream)
{
    lora_shrink_plan_t pl;
    int st = check_shrink(x, ld_x, A, ld_a, h, ld_h, M, K, r, split_k, &pl);
    if (st != LORA_OK || M == 0)
        return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    ShrinkParams p = shrink_params(x, ld_x, A, ld_a, M, r, pl, scale);
    if (split_k == 1) {                         // one split: it is its own last arrival
        p.out = h;
        p.ld_out = ld_h;
        return launch_status(launch_shrink_partial_direct(p, pl.waves, pl.rank_tiles,
                                                          group_tiles_for(M, split_k, pl.rank_tiles), s));
    }
    if (!workspace || !counters)
        return LORA_ERR_NULL;
    if (!aligned16(workspace) || (reinterpret_cast<uintptr_t>(counters) & 3u))
        return LORA_ERR_ALIGN;
    if (ws_bytes < lora_counted_workspace_bytes(M, r, split_k) || counter_bytes < lora_shrink_counter_bytes(M))
        return LORA_ERR_WORKSPACE;
    p.out = static_cast<float*>(workspace);
    p.ld_out = r;
    p.split_stride = M * r;
    CounterParams c{};
    c.counters = counters;
    c.h = h;
    c.ld_h = ld_h;
    return launch_status(launch_shrink_counted(p, c, pl.waves, pl.rank_tiles,
                                               group_tiles_for(M, split_k, pl.rank_tiles), s));
}

size_t lora_sgmv_counter_bytes(int64_t M)
{
    if (M < 0 || M > kMaxDim)
        return 0;
    return (size_t)4 * kMaxRankTiles * (size_t)(M > 0 ? M : 1);
}

int lora_sgmv_shrink_counted(const uint16_t* x, int64_t ld_x, const uint16_t* const* A_ptrs, int64_t ld_a,
                             const int32_t* ranks, const float* scales, int32_t n_adapters, const void* plan,
                             size_t plan_bytes, float* h, int64_t ld_h, int64_t M, int64_t K, int32_t r_max,
                             int32_t split_k, void* workspace, size_t ws_bytes, int32_t* counters,
                             size_t counter_bytes, void* stream)
{
    if (M < 0 || M > kMaxDim || n_adapters < 1)
        return LORA_ERR_SHAPE;
    lora_shrink_plan_t pl;
    int st = make_plan(K, r_max, split_k, &pl);
    if (st != LORA_OK)
        return st;
    if (!sgmv_items_fit(M, split_k))
        return LORA_ERR_SHAPE;
    if (M == 0)
        return LORA_OK;
    if (!x || !A_ptrs || !ranks || !plan || !h || !workspace || !counters)
        return LORA_ERR_NULL;
    if (ld_x < K || ld_a < K || ld_h < r_max)
        return LORA_ERR_SHAPE;
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(h) & 3u) || !aligned16(plan) || !aligned16(workspace) ||
        (reinterpret_cast<uintptr_t>(counters) & 3u) || ld_x % 8 || ld_a % 8)
        return LORA_ERR_ALIGN;
    if (plan_bytes < lora_sgmv_plan_bytes(M) || ws_bytes < lora_counted_workspace_bytes(M, r_max, split_k) ||
        counter_bytes < lora_sgmv_counter_bytes(M))
        return LORA_ERR_WORKSPACE;
    ShrinkParams p{};
    p.x = x;
    p.ld_x = ld_x;
    p.ld_a = ld_a;
    p.A_ptrs = A_ptrs;
    p.ranks = ranks;
    p.tiles = static_cast<const int32_t*>(plan);
    p.out = static_cast<float*>(workspace);
    p.ld_out = r_max;
    p.split_stride = M * r_max;
    p.M = M;
    p.r = r_max;
    p.r_max = r_max;
    p.k_chunk = pl.k_chunk;
    p.k_steps = pl.k_steps;
    p.split_k = split_k;
    p.n_adapters = n_adapters;
    p.scale = 1.0f;
    CounterParams c{};
    c.counters = counters;
    c.h = h;
    c.ld_h = ld_h;
    c.scales = scales;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // large M: plan tiles of one adapter share the A loads, as in the two-pass
    // shrink before its A-in-registers kernel
    const int T = r_max <= 16 * kGroupTiles ? shrink_tiles_per_wg(M, split_k) : 1;
    if (T > 1) {
        const int64_t bound = (M + T - 1) / T * split_k;
        return launch_status(
            launch_sgmv_shrink_counted_multi(p, c, pl.waves, T, (int)(bound < 2048 ? bound : 2048), s));
    }
    const int gt = sgmv_group_tiles(M, split_k, r_max);
    const int grid = sgmv_grid(M, split_k, r_max, gt);
    return launch_status(launch_sgmv_shrink_counted(p, c, pl.waves, gt, grid, s));
}

size_t lora_sgmv_plan_bytes(int64_t M)
{
    if (M < 0 || M > kMaxDim)
        return 0;
    return (size_t)kPlanHeaderInts * 4 + (size_t)kPlanTileInts * 4 * (size_t)M;
}

int lora_sgmv_plan(const int32_t* token_adapter, int64_t M, int32_t n_adapters, void* plan,
                   size_t plan_bytes, void* stream)
{
    if (M < 0 || M > kMaxDim)
        return LORA_ERR_SHAPE;
    if (n_adapters < 1)
        return LORA_ERR_SHAPE;
    if (!plan)
        return LORA_ERR_NULL;
    if (!aligned16(plan))
        return LORA_ERR_ALIGN;
    if (plan_bytes < lora_sgmv_plan_bytes(M))
        return LORA_ERR_WORKSPACE;
    if (M > 0 && !token_adapter)
        return LORA_ERR_NULL;
    return launch_status(launch_sgmv_plan(token_adapter, M, n_adapters, static_cast<int32_t*>(plan),
                                          static_cast<hipStream_t>(stream)));
}

size_t lora_sgmv_workspace_bytes(int64_t M, int32_t r_max, int32_t split_k)
{
    return workspace_bytes(M, r_max, split_k);
}

int lora_sgmv_shrink(const uint16_t* x, int64_t ld_x, const uint16_t* const* A_ptrs, int64_t ld_a,
                     const int32_t* ranks, const float* scales, const int32_t* token_adapter, int32_t n_adapters,
                     const void* plan, size_t plan_bytes, float* h, int64_t ld_h, int64_t M, int64_t K,
                     int32_t r_max, int32_t split_k, void* workspace, size_t ws_bytes, void* stream)
{
    if (M < 0 || M > kMaxDim || n_adapters < 1)
        return LORA_ERR_SHAPE;
    lora_shrink_plan_t pl;
    int st = make_plan(K, r_max, split_k, &pl);
    if (st != LORA_OK)
        return st;
    if (!sgmv_items_fit(M, split_k))
        return LORA_ERR_SHAPE;
    if (M == 0)
        return LORA_OK;
    if (!x || !A_ptrs || !ranks || !token_adapter || !plan || !h || !workspace)
        return LORA_ERR_NULL;
    if (ld_x < K || ld_a < K || ld_h < r_max)
        return LORA_ERR_SHAPE;
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(h) & 3u) || !aligned16(plan) || !aligned16(workspace) ||
        ld_x % 8 || ld_a % 8)
        return LORA_ERR_ALIGN;
    if (plan_bytes < lora_sgmv_plan_bytes(M) || ws_bytes < workspace_bytes(M, r_max, split_k))
        return LORA_ERR_WORKSPACE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = launch_sgmv_partials(x, ld_x, A_ptrs, ld_a, ranks, n_adapters, plan, M, r_max, pl, workspace, s);
    if (st != LORA_OK)
        return st;
    const TreeParams t = sgmv_tree_params(workspace, M, r_max, h, ld_h, token_adapter, ranks, scales, n_adapters);
    return launch_status(launch_splitk_tree(t, split_k, true, s));
}

int lora_sgmv_shrink_atomic(const uint16_t* x, int64_t ld_x, const uint16_t* const* A_ptrs, int64_t ld_a,
                            const int32_t* ranks, const float* scales, int32_t n_adapters, const void* plan,
                            size_t plan_bytes, float* h, int64_t ld_h, int64_t M, int64_t K, int32_t r_max,
                            int32_t split_k, void* stream)
{
    if (M < 0 || M > kMaxDim || n_adapters < 1)
        return LORA_ERR_SHAPE;
    lora_shrink_plan_t pl;
    int st = make_plan(K, r_max, split_k, &pl);
    if (st != LORA_OK)
        return st;
    if (!sgmv_items_fit(M, split_k))
        return LORA_ERR_SHAPE;
    if (M == 0)
        return LORA_OK;
    if (!x || !A_ptrs || !ranks || !plan || !h)
        return LORA_ERR_NULL;
    if (ld_x < K || ld_a < K || ld_h < r_max)
        return LORA_ERR_SHAPE;
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(h) & 3u) || !aligned16(plan) || ld_x % 8 || ld_a % 8)
        return LORA_ERR_ALIGN;
    if (plan_bytes < lora_sgmv_plan_bytes(M))
        return LORA_ERR_WORKSPACE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = launch_status(launch_fill_zero(h, ld_h, M, r_max, s));
    if (st != LORA_OK)
        return st;
    return launch_sgmv_partials(x, ld_x, A_ptrs, ld_a, ranks, n_adapters, plan, M, r_max, pl, h, s, true, scales,
                                ld_h);
}

int lora_sgmv_shrink_expand(const uint16_t* x, int64_t ld_x, const uint16_t* const* A_ptrs, int64_t ld_a,
                            const uint16_t* const* B_ptrs, const int32_t* ranks, const float* shrink_scales,
                            const float* expand_scales, const int32_t* token_adapter, int32_t n_adapters,
                            const void* plan, size_t plan_bytes, float* h, int64_t ld_h, uint16_t* y, int64_t ld_y,
                            int64_t M, int64_t K, int64_t N, int32_t r_max, int32_t split_k, void* workspace,
                            size_t ws_bytes, void* stream)
{
    if (M < 0 || M > kMaxDim || N < 0 || N > kMaxDim || n_adapters < 1)
        return LORA_ERR_SHAPE;
    lora_shrink_plan_t pl;
    int st = make_plan(K, r_max, split_k, &pl);
    if (st != LORA_OK)
        return st;
    if (N % 8 != 0)
        return LORA_ERR_UNSUPPORTED;
    if (!sgmv_items_fit(M, split_k) ||
        ((M + kRowBlock - 1) / kRowBlock) * ((N + kExpandCols - 1) / kExpandCols) > kMaxGrid)
        return LORA_ERR_SHAPE;
    if (M == 0 || N == 0)
        return LORA_OK;
    if (!x || !A_ptrs || !B_ptrs || !ranks || !token_adapter || !plan || !y || !workspace)
        return LORA_ERR_NULL;
    if (ld_x < K || ld_a < K || ld_y < N || (h && ld_h < r_max))
        return LORA_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(y) || (reinterpret_cast<uintptr_t>(h) & 3u) || !aligned16(plan) ||
        !aligned16(workspace) || ld_x % 8 || ld_a % 8 || ld_y % 8)
        return LORA_ERR_ALIGN;
    if (plan_bytes < lora_sgmv_plan_bytes(M) || ws_bytes < workspace_bytes(M, r_max, split_k))
        return LORA_ERR_WORKSPACE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = launch_sgmv_partials(x, ld_x, A_ptrs, ld_a, ranks, n_adapters, plan, M, r_max, pl, workspace, s);
    if (st != LORA_OK)
        return st;
    // Every column block of the expand evaluates its rows' tree again, so the
    // tree goes into the expand only under the bounds of tree_in_expand;
    // otherwise the tree kernel writes h once (into the caller's h, or in
    // place into workspace slice 0, each element read then written by one
    // thread) and the expand reads it.  Measured on MI355X (cold inputs,
    // Split-K 8; tree in the expand / tree kernel + expand): 4 rank-64
    // adapters, N = 6144: M = 128: 14.7 / 15.7 us, M = 256: 17.6 / 17.5 us,
    // M = 512: 23.6 / 21.6 us; 4 rank-16 adapters, N = 4096, M = 1024: 20.5 /
    // 22.0 us; one rank-64 adapter per token, N = 4096: 32 tokens 18.8 / 19.7
    // us.  The bits are the same either way.
    float* hh = h ? h : static_cast<float*>(workspace);
    const int64_t ldh = h ? ld_h : r_max;
    const bool h_readable = aligned16(hh) && ldh % 4 == 0;
    const bool fuse = tree_in_expand(M, r_max, N, split_k) || !h_readable;
    const TreeParams t = sgmv_tree_params(workspace, M, r_max, fuse ? h : hh, fuse ? ld_h : ldh, token_adapter,
                                          ranks, shrink_scales, n_adapters);
    ExpandParams e{};
    e.B_ptrs = B_ptrs;
    e.ranks = ranks;
    e.scales = expand_scales;
    e.ids = token_adapter;
    e.y = y;
    e.ld_y = ld_y;
    e.M = M;
    e.N = N;
    e.r = r_max;
    e.r_max = r_max;
    e.n_adapters = n_adapters;
    e.scale = 1.0f;
    if (fuse)
        return launch_status(launch_sgmv_expand_combine(e, t, split_k, s));
    st = launch_status(launch_splitk_tree(t, split_k, true, s));
    if (st != LORA_OK)
        return st;
    e.h = hh;
    e.ld_h = ldh;
    return launch_status(launch_sgmv_expand(e, s));
}

int lora_sgmv_expand(const float* h, int64_t ld_h, const uint16_t* const* B_ptrs, const int32_t* ranks,
                     const float* scales, const int32_t* token_adapter, int32_t n_adapters, uint16_t* y,
                     int64_t ld_y, int64_t M, int64_t N, int32_t r_max, void* stream)
{
    if (M < 0 || M > kMaxDim || N < 0 || N > kMaxDim || n_adapters < 1)
        return LORA_ERR_SHAPE;
    if (r_max < 1 || r_max > kMaxRank || N % 8 != 0)
        return LORA_ERR_UNSUPPORTED;
    if (((M + kRowBlock - 1) / kRowBlock) * ((N + kExpandCols - 1) / kExpandCols) > kMaxGrid)
        return LORA_ERR_SHAPE;
    if (M == 0 || N == 0)
        return LORA_OK;
    if (!h || !B_ptrs || !ranks || !token_adapter || !y)
        return LORA_ERR_NULL;
    if (ld_h < r_max || ld_y < N)
        return LORA_ERR_SHAPE;
    if (!aligned16(h) || !aligned16(y) || ld_h % 4 || ld_y % 8)
        return LORA_ERR_ALIGN;
    ExpandParams p{};
    p.h = h;
    p.ld_h = ld_h;
    p.B_ptrs = B_ptrs;
    p.ranks = ranks;
    p.scales = scales;
    p.ids = token_adapter;
    p.y = y;
    p.ld_y = ld_y;
    p.M = M;
    p.N = N;
    p.r = r_max;
    p.r_max = r_max;
    p.n_adapters = n_adapters;
    p.scale = 1.0f;
    return launch_status(launch_sgmv_expand(p, static_cast<hipStream_t>(stream)));
}

#pragma GCC visibility pop
}  // extern "C"
