// Multi-adapter work list, built on the device from per-token adapter ids.
//
// The paper's shrink operations carry, besides activations and weights, the
// token-to-adapter mapping (section 5.2).  A matrix-core tile needs one
// adapter for all its tokens, so the ids are turned into tiles of at most 16
// consecutive tokens with equal id: a run of L tokens becomes ceil(L/16)
// tiles starting at run offsets 0, 16, 32, ...; runs of ids outside
// [0, n_adapters) become tiles with adapter -1, which the shrinks zero and
// everything else skips.  Tiles are listed in token order.
//
// One workgroup of 1024 threads walks the ids in chunks of 1024.  Per chunk:
// the chunk's ids (normalised, plus the one before and the 15 after) are
// staged in LDS; a run starts at token i when its id differs from token
// i-1's; an inclusive max-scan of "i if a run starts at i" gives each token
// its run start (carried across chunks); tokens whose offset in the run is a
// multiple of 16 open a tile, whose length is read from the staged ids; an
// exclusive sum-scan of the openers gives the tile's slot.  Both scans use
// wavefront shuffles, then LDS across the 16 waves.  No host synchronisation
// is needed, so the plan can be built inside a captured stream and reused by
// every layer of a batch.
#include "device.h"
#include "kernels.h"

namespace lora {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;

__device__ __forceinline__ int norm_id(int32_t a, int32_t n)
{
    return (a < 0 || a >= n) ? -1 : a;
}

__global__ __launch_bounds__(kPlanThreads) void k_sgmv_plan(const int32_t* __restrict__ ids, int64_t M,
                                                            int32_t n_adapters, int32_t* __restrict__ plan)
{
    __shared__ int32_t s_max[kPlanWaves];
    __shared__ int32_t s_cnt[kPlanWaves];
    __shared__ int32_t s_carry_start;
    __shared__ int32_t s_carry_tiles;
    // ids[base - 1 .. base + 1024 + 15), normalised; slot 0 is token base - 1
    __shared__ int32_t s_ids[kPlanThreads + kRowBlock];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    if (tid == 0) {
        s_carry_start = 0;
        s_carry_tiles = 0;
    }
    __syncthreads();
    int32_t* tiles = plan + kPlanHeaderInts;

    for (int64_t base = 0; base < M; base += kPlanThreads) {
        for (int e = tid; e < kPlanThreads + kRowBlock; e += kPlanThreads) {
            const int64_t k = base - 1 + e;
            s_ids[e] = (k >= 0 && k < M) ? norm_id(ids[k], n_adapters) : -2;   // -2: outside [0, M)
        }
        __syncthreads();
        const int i = (int)(base + tid);
        const bool in = i < M;
        const int a = in ? s_ids[tid + 1] : -1;
        const bool run_start = in && (i == 0 || a != s_ids[tid]);

        // inclusive max-scan of run starts
        int v = run_start ? i : -1;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int o = __shfl_up(v, off, kWave);
            if (lane >= off)
                v = v > o ? v : o;
        }
        if (lane == kWave - 1)
            s_max[wave] = v;
        __syncthreads();
        int start = s_carry_start;
        int chunk_max = s_carry_start;
        for (int w = 0; w < kPlanWaves; ++w) {
            if (w < wave)
                start = start > s_max[w] ? start : s_max[w];
            chunk_max = chunk_max > s_max[w] ? chunk_max : s_max[w];
        }
        start = start > v ? start : v;

        const bool opens = in && ((i - start) % kRowBlock == 0);
        const int c = opens ? 1 : 0;
        int incl = c;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int o = __shfl_up(incl, off, kWave);
            if (lane >= off)
                incl += o;
        }
        if (lane == kWave - 1)
            s_cnt[wave] = incl;
        __syncthreads();
        int before = 0, total = 0;
        for (int w = 0; w < kPlanWaves; ++w) {
            if (w < wave)
                before += s_cnt[w];
            total += s_cnt[w];
        }
        if (opens) {
            const int slot = s_carry_tiles + before + incl - c;
            int n = 1;
            while (n < kRowBlock && s_ids[tid + 1 + n] == a)    // -2 past the end never matches
                ++n;
            tiles[3 * slot + 0] = i;
            tiles[3 * slot + 1] = n;
            tiles[3 * slot + 2] = a;
        }
        __syncthreads();                 // all reads of the carries and staged ids are done
        if (tid == 0) {
            s_carry_start = chunk_max;
            s_carry_tiles += total;
        }
        __syncthreads();
    }
    if (tid == 0) {
        plan[0] = s_carry_tiles;
        plan[1] = (int32_t)M;
        plan[2] = n_adapters;
        plan[3] = kPlanMagic;
    }
}

}  // namespace

hipError_t launch_sgmv_plan(const int32_t* ids, int64_t M, int32_t n_adapters, int32_t* plan, hipStream_t st)
{
    hipLaunchKernelGGL(k_sgmv_plan, dim3(1), dim3(kPlanThreads), 0, st, ids, M, n_adapters, plan);
    return hipGetLastError();
}

}  // namespace lora
