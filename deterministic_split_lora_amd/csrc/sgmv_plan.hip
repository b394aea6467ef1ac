// Multi-adapter work list, built on the device from per-token adapter ids.
//
// The paper's shrink operations carry, besides activations and weights, the
// token-to-adapter mapping (section 5.2).  A matrix-core tile computes one
// adapter for up to 16 rows; a tile entry is (first row, row span, adapter,
// row mask), its tokens the rows of the span whose mask bit is set.  Two
// tilings; blocks where the runs make at least two tiles per 16-token block
// and blocks make fewer tiles, else runs:
//   runs: a run of L consecutive tokens with equal id becomes ceil(L/16)
//     tiles starting at run offsets 0, 16, 32, ... (full masks), listed in
//     token order;
//   blocks (up to kBlockPlanTokens tokens): each aligned 16-token block gives
//     one tile per distinct id in it, masked to that id's tokens, listed by
//     adapter and then block.  Interleaved ids (decode tokens of many
//     requests with few adapters) give far fewer tiles this way.
// Ids outside [0, n_adapters) form tiles with adapter -1, which the shrinks
// zero and everything else skips.  Which tiling is chosen changes no bit of
// any result: every row's arithmetic is the same in any tile.
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
// third walk writes the tiles, whose length is read from the staged ids.  For
// the block tiling (a single pass), each thread counts its tokens whose id
// does not occur earlier in their 16-token block; if the blocks hold fewer
// (block, id) pairs than the runs make tiles, a sum-scan places one sort key
// (id + 1, block) per pair in LDS, a bitonic sort orders them by id and
// block, and each key becomes a tile masked to the block's tokens with that
// id.  No host synchronisation is needed, so the
// plan can be built inside a captured stream and reused by every layer of a
// batch.
#include "device.h"
#include "kernels.h"

namespace lora {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kPlanPer = 8;                            // tokens per thread and pass, at most
constexpr int kPlanPass = kPlanThreads * kPlanPer;     // tokens per pass, at most
constexpr int kBlockPlanTokens = 4096;                 // block tiling considered up to this many tokens
constexpr int kBlockBits = 8;                          // block index bits of a sort key (256 blocks)
constexpr int32_t kBlockPlanAdapters = 1 << 22;        // (id + 1) << kBlockBits stays below 2^31
static_assert(kBlockPlanTokens / kRowBlock <= (1 << kBlockBits), "block index must fit the key");
static_assert(kBlockPlanTokens / kRowBlock <= kPlanThreads, "one thread per block");
static_assert(kBlockPlanTokens <= kPlanPass, "block tiling works on one pass");
constexpr int kSortPer = kBlockPlanTokens / kPlanThreads;   // sort keys per thread
static_assert(kSortPer * kPlanThreads == kBlockPlanTokens && (kSortPer & (kSortPer - 1)) == 0, "sort layout");

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
    __shared__ int32_t s_wave_blk[kPlanWaves];
    __shared__ int32_t s_keys[kBlockPlanTokens];      // block tiling: (id + 1, block) sort keys
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
        // block tiling (one pass: base 0, carries 0), if it gives fewer tiles;
        // looked at only where the runs make at least two tiles per block
        // (every block gives at least one tile, so it cannot win by much
        // otherwise, and the plan's time stays that of the runs alone)
        if (M <= kBlockPlanTokens && n_adapters < kBlockPlanAdapters &&
            total >= 2 * ((len + kRowBlock - 1) / kRowBlock)) {                // uniform
            // which of this thread's tokens is the first of its id in its
            // 16-token block (compact loops: this kernel's time is mostly
            // latency, instruction fetch included)
            auto first_in_block = [&](int t) {
                const int a = s_ids[t + 1];
                const int b0 = t & ~(kRowBlock - 1);
                if (t > b0 && s_ids[t] == a)      // inside a run: settled by one read
                    return false;
#pragma unroll 1
                for (int q = b0; q < t - 1; ++q)
                    if (s_ids[q + 1] == a)
                        return false;
                return true;
            };
            int nfirst = 0;
#pragma unroll 1
            for (int u = 0; u < T; ++u) {
                const int t = first + u;
                if (t >= len)
                    break;
                nfirst += first_in_block(t) ? 1 : 0;
            }
            int pairs;
            const int pbase = block_exclusive_scan(nfirst, 0, vadd, s_wave_blk, pairs);
            if (pairs < total) {                  // uniform: both are workgroup-wide
                int j = pbase;
#pragma unroll 1
                for (int u = 0; u < T; ++u) {
                    const int t = first + u;
                    if (t >= len)
                        break;
                    if (first_in_block(t))
                        s_keys[j++] = ((s_ids[t + 1] + 1) << kBlockBits) | (t / kRowBlock);
                }
                // bitonic sort of the keys, ascending, kSortPer per thread in
                // registers (elements kSortPer tid + q): partners within a
                // thread swap in registers, within a wave through lane
                // shuffles, across waves through LDS
                int P = kSortPer;
                while (P < pairs)
                    P <<= 1;
                __syncthreads();                          // every key is in LDS
                int32_t v[kSortPer];
#pragma unroll
                for (int q = 0; q < kSortPer; ++q) {
                    const int e = kSortPer * tid + q;
                    v[q] = e < pairs ? s_keys[e] : INT32_MAX;
                }
                for (int k = 2; k <= P; k <<= 1) {
                    for (int j = k >> 1; j > 0; j >>= 1) {
                        if (j < kSortPer) {
#pragma unroll
                            for (int q = 0; q < kSortPer; ++q) {
                                const int q2 = q ^ j;
                                if (q2 > q) {
                                    const bool asc = ((kSortPer * tid + q) & k) == 0;
                                    const int32_t lo = v[q] < v[q2] ? v[q] : v[q2];
                                    const int32_t hi = v[q] < v[q2] ? v[q2] : v[q];
                                    v[q] = asc ? lo : hi;
                                    v[q2] = asc ? hi : lo;
                                }
                            }
                        } else {
                            const int lanes = j / kSortPer;        // partner thread: tid ^ lanes
                            int32_t pv[kSortPer];
                            if (lanes < kWave) {
#pragma unroll
                                for (int q = 0; q < kSortPer; ++q)
                                    pv[q] = __shfl_xor(v[q], lanes, kWave);
                            } else {
                                __syncthreads();                  // earlier reads of s_keys are done
#pragma unroll
                                for (int q = 0; q < kSortPer; ++q)
                                    s_keys[kSortPer * tid + q] = v[q];
                                __syncthreads();
#pragma unroll
                                for (int q = 0; q < kSortPer; ++q)
                                    pv[q] = s_keys[kSortPer * (tid ^ lanes) + q];
                            }
#pragma unroll
                            for (int q = 0; q < kSortPer; ++q) {
                                const int e = kSortPer * tid + q;
                                const bool asc = (e & k) == 0;
                                const bool lower = (tid & lanes) == 0;
                                const int32_t mn = v[q] < pv[q] ? v[q] : pv[q];
                                const int32_t mx = v[q] < pv[q] ? pv[q] : v[q];
                                v[q] = lower == asc ? mn : mx;
                            }
                        }
                    }
                }
                __syncthreads();                          // earlier reads of s_keys are done
#pragma unroll
                for (int q = 0; q < kSortPer; ++q)
                    s_keys[kSortPer * tid + q] = v[q];
                __syncthreads();
                for (int i = tid; i < pairs; i += kPlanThreads) {
                    const int32_t key = s_keys[i];
                    const int a = (key >> kBlockBits) - 1;
                    const int r0 = (key & ((1 << kBlockBits) - 1)) * kRowBlock;
                    const int cnt = len - r0 < kRowBlock ? len - r0 : kRowBlock;
                    uint32_t mask = 0;
#pragma unroll 1
                    for (int q = 0; q < cnt; ++q)
                        mask |= (s_ids[r0 + 1 + q] == a ? 1u : 0u) << q;
                    tiles[kPlanTileInts * i + 0] = r0;
                    tiles[kPlanTileInts * i + 1] = cnt;
                    tiles[kPlanTileInts * i + 2] = a;
                    tiles[kPlanTileInts * i + 3] = (int32_t)mask;
                }
                if (tid == 0) {
                    plan[0] = pairs;
                    plan[1] = (int32_t)M;
                    plan[2] = n_adapters;
                    plan[3] = kPlanMagic;
                }
                return;                           // uniform
            }
        }
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
                    tiles[kPlanTileInts * slot + 0] = i;
                    tiles[kPlanTileInts * slot + 1] = n;
                    tiles[kPlanTileInts * slot + 2] = a;
                    tiles[kPlanTileInts * slot + 3] = (int32_t)((1u << n) - 1u);
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
