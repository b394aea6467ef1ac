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
// One workgroup of 1024 threads walks the ids in passes of up to 8192
// tokens; in a pass each thread owns T = ceil(tokens / 1024) <= 8
// consecutive tokens.  Per pass: the pass's ids (normalised, plus the one
// before and the 15 after) are staged in LDS with coalesced loads; a run
// starts at token i when its id differs from token i-1's; each thread finds
// the last run start among its tokens, and an exclusive max-scan of those
// over the threads (wavefront shuffles, then LDS across the 16 waves, plus
// the carry from earlier passes) gives each thread the run start its first
// token belongs to; walking its tokens again, each thread counts the tokens
// whose offset in their run is a multiple of 16 - they open a tile - and an
// exclusive sum-scan of the counts gives each thread its first tile slot; a
// third walk writes the tiles, whose length is read from the staged ids.  No
// host synchronisation is needed, so the plan can be built inside a captured
// stream and reused by every layer of a batch.
#include "device.h"
#include "kernels.h"

namespace lora {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kPlanPer = 8;                            // tokens per thread and pass, at most
constexpr int kPlanPass = kPlanThreads * kPlanPer;     // tokens per pass, at most

__device__ __forceinline__ int norm_id(int32_t a, int32_t n)
{
    return (a < 0 || a >= n) ? -1 : a;
}

// Inclusive scan over a wavefront with `op`, then the exclusive prefix over
// the earlier waves of the workgroup (through LDS) combined in: returns this
// thread's exclusive value; `total` receives the workgroup-wide result.
// s_wave must not be written again before every thread has passed another
// barrier (each scan of a pass has its own).
template <typename Op>
__device__ __forceinline__ int block_exclusive_scan(int v, int identity, Op op, int32_t* s_wave, int& total)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off, kWave);
        if (lane >= off)
            incl = op(incl, o);
    }
    const int excl_in_wave = __shfl_up(incl, 1, kWave);
    if (lane == kWave - 1)
        s_wave[wave] = incl;
    __syncthreads();
    int before = identity;
    total = identity;
    for (int w = 0; w < kPlanWaves; ++w) {
        if (w < wave)
            before = op(before, s_wave[w]);
        total = op(total, s_wave[w]);
    }
    return lane == 0 ? before : op(before, excl_in_wave);
}

__global__ __launch_bounds__(kPlanThreads) void k_sgmv_plan(const int32_t* __restrict__ ids, int64_t M,
                                                            int32_t n_adapters, int32_t* __restrict__ plan)
{
    __shared__ int32_t s_wave_max[kPlanWaves];
    __shared__ int32_t s_wave_sum[kPlanWaves];
    // ids[base - 1 .. base + pass + 15), normalised; slot 0 is token base - 1
    __shared__ int32_t s_ids[kPlanPass + kRowBlock];
    const int tid = threadIdx.x;
    int32_t* tiles = plan + kPlanHeaderInts;
    int carry_start = 0;                          // run start of the token before this pass
    int carry_tiles = 0;                          // tiles opened before this pass
    const auto vmax = [](int a, int b) { return a > b ? a : b; };
    const auto vadd = [](int a, int b) { return a + b; };

    for (int64_t base = 0; base < M; base += kPlanPass) {
        const int64_t left = M - base;
        const int len = left < kPlanPass ? (int)left : kPlanPass;          // tokens of this pass
        const int T = (len + kPlanThreads - 1) / kPlanThreads;             // tokens per thread (uniform)
        for (int e = tid; e < len + kRowBlock; e += kPlanThreads) {
            const int64_t k = base - 1 + e;
            s_ids[e] = (k >= 0 && k < M) ? norm_id(ids[k], n_adapters) : -2;   // -2: outside [0, M)
        }
        __syncthreads();
        const int first = tid * T;                // this thread's first token, relative to base
        // 1. the last run start among this thread's tokens (-1: none)
        int last = -1;
        for (int u = 0; u < T; ++u) {
            const int t = first + u;
            if (t < len && (base + t == 0 || s_ids[t + 1] != s_ids[t]))
                last = (int)(base + t);
        }
        int chunk_max;
        const int before = block_exclusive_scan(last, -1, vmax, s_wave_max, chunk_max);
        int start = vmax(carry_start, before);    // run start of the token before `first`
        // 2. tokens opening a tile
        int count = 0;
        {
            int rs = start;
            for (int u = 0; u < T; ++u) {
                const int t = first + u;
                if (t >= len)
                    break;
                const int i = (int)(base + t);
                if (i == 0 || s_ids[t + 1] != s_ids[t])
                    rs = i;
                count += ((i - rs) % kRowBlock == 0) ? 1 : 0;
            }
        }
        int total;
        int slot = carry_tiles + block_exclusive_scan(count, 0, vadd, s_wave_sum, total);
        // 3. the tiles
        {
            int rs = start;
            for (int u = 0; u < T; ++u) {
                const int t = first + u;
                if (t >= len)
                    break;
                const int i = (int)(base + t);
                if (i == 0 || s_ids[t + 1] != s_ids[t])
                    rs = i;
                if ((i - rs) % kRowBlock == 0) {
                    const int a = s_ids[t + 1];
                    int n = 1;
                    while (n < kRowBlock && s_ids[t + 1 + n] == a)     // -2 past the end never matches
                        ++n;
                    tiles[3 * slot + 0] = i;
                    tiles[3 * slot + 1] = n;
                    tiles[3 * slot + 2] = a;
                    ++slot;
                }
            }
        }
        carry_start = vmax(carry_start, chunk_max);
        carry_tiles += total;
        if (base + kPlanPass < M)                 // uniform
            __syncthreads();                      // every read of s_ids is done before the next pass
    }
    if (tid == 0) {
        plan[0] = carry_tiles;
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
