// Single-launch deterministic shrink + expand for gfx950: one grid, two roles.
//
// The two-launch schedule (Split-K partials, then tree + expand) pays for a
// second dependent dispatch and cannot start loading y and B before every
// partial is written.  Here one grid carries both halves, row block by row
// block: for each 16-token row block come first its S x G shrink workgroups
// (split s of the contraction, rank-tile group g), then its C expand
// workgroups (one per W x 64 output columns).
//
//   shrink workgroup: the Split-K work item of the two-launch path (same k
//       chunk, chains, wave tree), its fp32 partial stored to the workspace
//       with agent-scope stores; it waits for its stores to complete, then
//       adds 1 to its row block's arrival counter.
//   expand workgroup: loads its y tile and its B rows first - they do not
//       depend on the shrink - then waits until the row block's counter
//       reaches S x G, evaluates the fixed pairwise tree over the S slices
//       and the shrink-scale multiply into LDS (the first column block also
//       writes h), and finishes the expand exactly as the two-launch path.
//       It then adds 1 to the row block's departure counter; the last of the
//       C expand workgroups puts both counters back to 0 for the next call.
//
// Per element this is the arithmetic of the two-launch path (the partials,
// the tree over splits, the multiplies, the expand and its rounding are the
// same code), so the bits are the same whatever the schedule or the order of
// arrivals; the counters only say when the partials are all there
// (the completion-counter protocol of the paper's section 4.3, with the
// combine done by the consumers of the partials instead of the last writer).
//
// Why the wait always ends: workgroups are dispatched in increasing id, and
// every shrink workgroup of a row block has a smaller id than that row
// block's expand workgroups, so by the time an expand workgroup runs, all the
// shrink workgroups it waits for have been dispatched (or are running, or
// done); shrink workgroups never wait.  The wait is also bounded: after
// kSpinLimit polls an expand workgroup gives up, sets the status word and
// leaves y untouched.
//
// Memory ordering across XCDs (each has its own L2), at agent scope: the
// partials travel with agent-scope stores and loads; a shrink workgroup's
// barrier orders all its partial stores before thread 0's arrival add, a
// RELEASE read-modify-write; an expand workgroup's thread 0 polls the
// counter with relaxed loads and, once it reads S x G (a value written by
// the last of those release adds, whose release sequences the earlier adds
// continue), issues an ACQUIRE fence at agent scope, so every partial store
// happens before the barrier that lets the workgroup load the partials.
#include "device.h"
#include "kernels.h"
#include "shrink_tile.h"

namespace lora {

namespace {

constexpr int kHTileStride = 132;         // floats per LDS row of the h tile (128 + 4 padding)
constexpr int kSpinLimit = 1 << 21;       // polls before an expand workgroup gives up

template <int RT, int W>
constexpr int lds_floats()
{
    return red_floats<RT, W>() > kRowBlock * kHTileStride ? red_floats<RT, W>() : kRowBlock * kHTileStride;
}

template <int RT, int W, int KS>
__global__ __launch_bounds__(W * 64) void k_shrink_expand_counted(ShrinkParams p, ExpandParams e, TreeParams c,
                                                                  StreamParams q)
{
    __shared__ __align__(16) float lds[lds_floats<RT, W>()];
    __shared__ int ok;
    // 32-bit item decomposition: the grid is below 2^31 workgroups
    const uint32_t per_mb = (uint32_t)(q.producers + q.consumers);
    const uint32_t mb = blockIdx.x / per_mb;
    const uint32_t j = blockIdx.x - mb * per_mb;
    const int64_t row0 = (int64_t)mb * kRowBlock;
    const int64_t left = p.M - row0;
    const int nrows = left < kRowBlock ? (int)left : kRowBlock;
    int32_t* arrivals = q.counters + 2 * (int64_t)mb;
    int32_t* departures = arrivals + 1;

    if (j < (uint32_t)q.producers) {
        const int s = (int)(j % (uint32_t)p.split_k);
        const int grp = (int)(j / (uint32_t)p.split_k);
        shrink_tile<RT, W, kToWorkspaceCoherent>(p, row0, nrows, kFullMask, p.A, p.r, grp * 16 * RT, s, 1.0f, lds);
        __syncthreads();                      // every partial store of the workgroup ...
        if (threadIdx.x == 0)                 // ... happens before this release
            __hip_atomic_fetch_add(arrivals, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    const int cb = (int)(j - (uint32_t)q.producers);
    const int r = p.r;
    ExpandLane L = expand_lane(row0, nrows, (int64_t)cb * W * 64);
    const bool active = L.n_base < e.N;
    u16x8 yv[2];
    bf16x8 bop[4][KS];
    if (active)
        expand_load<KS>(L, e.y, e.ld_y, e.N, e.B, e.ld_b, r, yv, bop);

    if (threadIdx.x == 0) {
        int good = 1;
        int spins = 0;
        while (__hip_atomic_load(arrivals, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < q.producers) {
            if (++spins > kSpinLimit) {
                good = 0;
                __hip_atomic_store(q.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (good)                             // pairs with the producers' release adds
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        ok = good;
        // every expand workgroup of the row block has passed its wait once all
        // of them have departed: then the counters can be reset
        if (__hip_atomic_fetch_add(departures, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            q.consumers - 1) {
            __hip_atomic_store(arrivals, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(departures, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    if (!ok)
        return;

    float* hs = lds;
    const bool write_h = c.h != nullptr && cb == 0;
    for (int t = threadIdx.x; t < kRowBlock * r; t += W * 64) {
        const int row = t / r;
        const int col = t - row * r;
        if (row < nrows) {
            const float* w = c.ws + (row0 + row) * c.ldw + col;
            const float hv = __fmul_rn(split_tree(w, c.split_stride, p.split_k), c.scale);
            hs[row * kHTileStride + col] = hv;
            if (write_h)
                c.h[(row0 + row) * c.ld_h + col] = hv;
        }
    }
    __syncthreads();
    if (!active)
        return;
    expand_finish<KS>(L, e.y, e.ld_y, e.N, hs, kHTileStride, r, e.scale, yv, bop);
}

template <int RT, int W>
void launch_rw(const ShrinkParams& p, const ExpandParams& e, const TreeParams& c, const StreamParams& q,
               dim3 grid, hipStream_t st)
{
    switch (expand_steps(e.r)) {
    case 4: hipLaunchKernelGGL((k_shrink_expand_counted<RT, W, 4>), grid, dim3(W * 64), 0, st, p, e, c, q); break;
    case 2: hipLaunchKernelGGL((k_shrink_expand_counted<RT, W, 2>), grid, dim3(W * 64), 0, st, p, e, c, q); break;
    default: hipLaunchKernelGGL((k_shrink_expand_counted<RT, W, 1>), grid, dim3(W * 64), 0, st, p, e, c, q); break;
    }
}

template <int RT>
void launch_r(const ShrinkParams& p, const ExpandParams& e, const TreeParams& c, const StreamParams& q, int waves,
              dim3 grid, hipStream_t st)
{
    switch (waves) {
    case 1: launch_rw<RT, 1>(p, e, c, q, grid, st); break;
    case 2: launch_rw<RT, 2>(p, e, c, q, grid, st); break;
    case 4: launch_rw<RT, 4>(p, e, c, q, grid, st); break;
    default: launch_rw<RT, 8>(p, e, c, q, grid, st); break;
    }
}

}  // namespace

hipError_t launch_shrink_expand_counted(const ShrinkParams& p, const ExpandParams& e, const TreeParams& c,
                                        const StreamParams& q, int waves, int group_tiles, hipStream_t st)
{
    const int64_t mbs = (p.M + kRowBlock - 1) / kRowBlock;
    const dim3 grid((unsigned)(mbs * (q.producers + q.consumers)));
    if (group_tiles == 1)
        launch_r<1>(p, e, c, q, waves, grid, st);
    else
        launch_r<4>(p, e, c, q, waves, grid, st);
    return hipGetLastError();
}

}  // namespace lora
