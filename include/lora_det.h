/*
 * lora_det.h - deterministic Split-K LoRA shrink / expand for AMD MI355X (gfx950).
 *
 * A plain C interface: host scalars and device pointers only, no HIP or
 * framework types.  bf16 tensors are passed as `uint16_t*` (the IEEE binary32
 * upper half), fp32 as `float*`, a HIP stream as `void*` (NULL = the default
 * stream).
 *
 * The operation is the LoRA term of a linear layer, Eq. 1 of "Reproducible LoRA
 * Inference Through Deterministic Split-K Reduction" (Balusamy & Mohan):
 *     Y = X W^T + s (X A^T) B^T
 * split into the shrink  h = X A^T  (section 2: a narrow GEMM, H -> r) and the
 * expand  Y += s h B^T.  The shrink is parallelised with Split-K (section 2.1,
 * Eq. 3) and its partials are combined in a fixed order (section 4.3) so that
 * every output bit is reproducible.
 *
 * OPERAND LAYOUTS (row-major, element strides `ld_*`, innermost stride 1):
 *   x  bf16 [M][ld_x]   tokens x hidden; columns [0, K) used
 *   A  bf16 [r][ld_a]   the adapter's down projection stored as in Eq. 1
 *                       (A in R^{r x H}): row j holds rank j's K weights
 *   h  fp32 [M][ld_h]   shrink output; columns [0, r) written
 *   B  bf16 [N][ld_b]   the up projection as in Eq. 1 (B in R^{H_out x r})
 *   y  bf16 [M][ld_y]   updated in place; columns [0, N) touched
 * (As a math matrix, the product x.A of "hidden x rank" shape is x times the
 * transpose of this A; the two describe the same numbers.)
 *
 * OWNERSHIP.  Every tensor, workspace and plan buffer is allocated and owned by
 * the caller.  The library never allocates, frees or synchronises; it only
 * enqueues kernels on `stream` and returns.  Calls on one stream execute in
 * order; a workspace or plan buffer must not be shared by calls that may run
 * concurrently.  Outputs must not alias inputs or workspaces.
 *
 * ERRORS.  Every entry point returns LORA_OK (0) or a positive lora_status.
 * All argument checks happen on the host before any HIP call; on any error
 * nothing is enqueued.  M == 0 (or N == 0 for the expand) is a successful no-op.
 * LORA_ERR_LAUNCH reports a launch the HIP runtime refused.  No entry point
 * prints, aborts or throws.
 *
 * DETERMINISM.  For the deterministic entry points (everything except
 * lora_shrink_splitk_atomic and lora_sgmv_shrink_atomic) each output element's bits depend only on that
 * token's own input row, the adapter, K, r, split_k and the scale: not on M,
 * on the row's position in the batch, on other rows, on the stream or on
 * timing.  The Split-K plan (lora_shrink_plan) is a function of (K, split_k)
 * alone.
 *
 * SIGNATURE NOTES, for callers used to other LoRA kernel interfaces:
 *   - A is [r][K] and B is [N][r] (Eq. 1's orientation), not K x r and r x N:
 *     a caller holding A as [K][r] passes its transpose.  Both operands of
 *     every matrix-core step are then contiguous along the reduced dimension.
 *   - The multi-adapter shrinks take a device plan made by lora_sgmv_plan
 *     from the per-token adapter ids (tiles of at most 16 consecutive tokens
 *     with one adapter), not the ids alone; build it once per batch and reuse
 *     it for every layer.  lora_sgmv_shrink_counted and
 *     lora_sgmv_shrink_atomic read the ids only through the plan; the
 *     expands read token_adapter directly.
 *   - Adapters are passed as device arrays of A and B addresses, with one
 *     leading dimension ld_a for every A and every B_a packed as
 *     [N][r_a rounded up to 8], plus device arrays of ranks and
 *     (optionally) scales.
 *   - Split-K workspaces, counters and plans are caller buffers whose sizes
 *     the *_bytes functions return; every entry point takes leading
 *     dimensions and a stream.
 *   - The single-launch shrinks (lora_shrink_splitk_counted,
 *     lora_sgmv_shrink_counted) take a workspace of their own, twice the
 *     two-pass size (lora_counted_workspace_bytes), zero before the first
 *     call and left zero by every call.
 *
 * SUPPORTED (otherwise LORA_ERR_UNSUPPORTED / LORA_ERR_ALIGN):
 *   1 <= r <= 128 (lora_shrink_expand_fused: r <= 64);  split_k in {1, 2, 4, 8, 16};
 *   K % (32 * split_k) == 0;
 *   x, A, B, y, workspace: 16-byte aligned, ld_x, ld_a, ld_b, ld_y multiples of 8;
 *   h as written by the shrinks: 4-byte aligned, any ld_h >= r;
 *   h as read by the expands: 16-byte aligned, ld_h a multiple of 4;
 *   N a multiple of 8;
 *   M, K, N < 2^31.
 */
#ifndef LORA_DET_H
#define LORA_DET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_DET_ABI_VERSION 6

enum lora_status {
    LORA_OK = 0,
    LORA_ERR_NULL = 1,        /* a required pointer is NULL */
    LORA_ERR_SHAPE = 2,       /* negative size, or a leading dimension below the row width */
    LORA_ERR_UNSUPPORTED = 3, /* rank, split count or K divisibility outside the supported set */
    LORA_ERR_ALIGN = 4,       /* pointer or leading dimension breaks the 16-byte rule */
    LORA_ERR_WORKSPACE = 5,   /* workspace or plan buffer smaller than required */
    LORA_ERR_LAUNCH = 6,      /* the HIP runtime refused a kernel launch */
    LORA_ERR_SCRATCH = 7      /* lora_shrink_expand_noalloc: more workspace than its fixed buffer */
};

/* Returns LORA_DET_ABI_VERSION of the built library. */
int lora_abi_version(void);

/* Static text for a status code ("ok", "null pointer", ...); never NULL. */
const char* lora_status_str(int status);

/*
 * The static Split-K plan (host only, no HIP call).  Section 2.1 / Eq. 3 of
 * the paper split the reduction dimension into S subsets; here they are S
 * contiguous chunks of k_chunk = K / S (as Fig. 1 draws K0..K7).  Inside a
 * chunk, `waves` wavefronts each own k_chunk / waves consecutive k and run
 * `k_steps` 16x16x32 bf16 matrix-core steps over them in ascending k with an
 * fp32 accumulator; the wave results are added along a fixed pairwise tree.
 * The plan depends on (K, split_k) only - never on M.  rank_tiles = ceil(r/16),
 * row_block = 16 tokens per workgroup.
 * Returns LORA_ERR_NULL / LORA_ERR_UNSUPPORTED / LORA_ERR_SHAPE on bad input.
 */
typedef struct lora_shrink_plan_s {
    int32_t split_k;
    int32_t k_chunk;
    int32_t waves;
    int32_t k_steps;
    int32_t rank_tiles;
    int32_t row_block;
} lora_shrink_plan_t;

int lora_shrink_plan(int64_t K, int32_t r, int32_t split_k, lora_shrink_plan_t* plan);

/*
 * Bytes of fp32 workspace lora_shrink_splitk needs: split_k * M * r * 4
 * (0 when split_k == 1: that path writes h directly).  Layout, part of the ABI:
 * ws[s][i][j] at float offset (s * M + i) * r + j holds split s's partial sum
 * for token i, rank j.  No initialisation needed.  Returns 0 for invalid input.
 */
size_t lora_shrink_workspace_bytes(int64_t M, int32_t r, int32_t split_k);

/*
 * Deterministic Split-K shrink (paper section 4.3, Eq. 3):
 *     h[i][j] = scale * T( P_0[i][j], ..., P_{S-1}[i][j] )
 *     P_s[i][j] = sum over k in chunk s of x[i][k] * A[j][k]   (fp32)
 * where T is the fixed pairwise tree: (P0+P1), (P2+P3), ... then neighbours of
 * those, level by level, in fp32 - the order the paper's earlier two-kernel
 * deterministic design used - followed by one fp32 multiply by `scale`.
 * Two launches: the partial kernel writes ws, a second kernel applies T.
 * With split_k == 1 one launch writes h = scale * P_0 directly.
 * workspace: >= lora_shrink_workspace_bytes(M, r, split_k) bytes (may be NULL
 * when that is 0).
 */
int lora_shrink_splitk(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a,
                       float* h, int64_t ld_h, int64_t M, int64_t K, int32_t r,
                       int32_t split_k, float scale, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Atomic Split-K shrink, kept only as the nondeterministic contrast of paper
 * section 4.1: h is zeroed by a fill kernel (the output initialisation the
 * paper counts in its latency), then the partial kernel that lora_shrink_splitk
 * would run for these sizes (same work items and schedule) adds each split's
 * scale * P_s into h with hardware fp32 atomic adds, in whatever order the
 * splits finish, instead of storing P_s to a workspace.  The value agrees with
 * lora_shrink_splitk to rounding; the bits may differ between runs.
 */
int lora_shrink_splitk_atomic(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a,
                              float* h, int64_t ld_h, int64_t M, int64_t K, int32_t r,
                              int32_t split_k, float scale, void* stream);

/*
 * Expand (paper Eq. 1, the s (X A^T) B^T term added into Y):
 *     hb = bf16_rne(h[i][j])   (section 6.2: shrink outputs meet B as bf16)
 *     acc = sum_{j<r} hb[i][j] * B[n][j]      fp32 accumulation, matrix cores
 *     y[i][n] = bf16_rne( fma(scale, acc, y[i][n]) )
 * One launch, y updated in place.
 */
int lora_expand(const float* h, int64_t ld_h, const uint16_t* B, int64_t ld_b,
                uint16_t* y, int64_t ld_y, int64_t M, int32_t r, int64_t N, float scale,
                void* stream);

/*
 * Compensated expand (the GEMM compensation of "Demystifying Numerical
 * Instability in LLM Inference ... with HEAL", section 3, Eq. 10, with bf16
 * halves): h is split into hi = bf16_rne(h) and lo = bf16_rne(h - hi), both
 * are multiplied by B on the matrix cores, and the two fp32 results are added
 * before the update:
 *     acc = sum_j hi[i][j] B[n][j]  +  sum_j lo[i][j] B[n][j]
 *     y[i][n] = bf16_rne( fma(scale, acc, y[i][n]) )
 * The product then sees about 16 significant bits of h instead of 8, so two
 * fp32 shrink values that round to different bf16 values no longer give y
 * values 1 bf16 step apart.  Twice the matrix-core work of lora_expand, the
 * same memory traffic.  Arguments, layouts and errors as for lora_expand.
 */
int lora_expand_compensated(const float* h, int64_t ld_h, const uint16_t* B, int64_t ld_b,
                            uint16_t* y, int64_t ld_y, int64_t M, int32_t r, int64_t N, float scale,
                            void* stream);

/*
 * Single-launch deterministic Split-K shrink: the paper's final design
 * (section 4.3, Alg. 1 - per-tile arrival counters, the partials combined
 * inside the same launch).  Each split's workgroup adds 1 to its row block's
 * integer counter (agent-scope relaxed read-modify-write) when it starts, then
 * computes its fp32 partial.  The workgroup whose add returned split_k - 1
 * started last: it resets the counter to 0, keeps its own partial and reads
 * the other split_k - 1 from the workspace, then applies the same fixed
 * pairwise tree and scale as lora_shrink_splitk and writes h.  Bit for bit
 * the same h as lora_shrink_splitk, in one launch.
 * The partials move in TAGGED 64-bit workspace slots: low half the fp32
 * value, high half 1 once written, put back to 0 by the workgroup that
 * consumed it.  Writers store and the combining workgroup loads whole slots
 * with agent-scope atomic stores and loads, and waits until each slot shows
 * its tag: per-location coherence suffices, so no release or acquire is
 * issued (on gfx950 an agent-scope release writes back the XCD's L2).  The
 * combining workgroup waits only for workgroups that have already made their
 * add, which are resident and wait for nobody, so every wait ends; a slot
 * that never showed its partial (no correct launch) would give NaN in h.
 * workspace: lora_counted_workspace_bytes(M, r, split_k) bytes, 16-byte
 * aligned, ALL ZERO before the first call and left zero by every completed
 * call; it is this entry point's own (the two-pass entry points write other
 * values into a workspace).  Slot (s, i, j) is the 64-bit word
 * s * M * r + i * r + j.
 * counters: int32 [lora_shrink_counter_bytes(M) / 4] (8 per 16-token block, one
 * per 16-wide rank tile of a rank <= 128), 4-byte aligned, ALL ZERO
 * before the first call; every completed call leaves them zero again, so one
 * zero-initialised pair of buffers serves any number of calls on one stream
 * (not concurrent calls).  split_k == 1 needs neither workspace nor counters.
 */
size_t lora_counted_workspace_bytes(int64_t M, int32_t r_max, int32_t split_k);

size_t lora_shrink_counter_bytes(int64_t M);

int lora_shrink_splitk_counted(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a,
                               float* h, int64_t ld_h, int64_t M, int64_t K, int32_t r,
                               int32_t split_k, float scale, void* workspace, size_t workspace_bytes,
                               int32_t* counters, size_t counter_bytes, void* stream);

/*
 * The two halves of the deterministic pipeline, one launch each.
 *
 * lora_shrink_partials: the Split-K partial kernel of lora_shrink_splitk on its
 * own.  It writes ws[s][i][j] = P_s[i][j] (unscaled fp32 partial sums, layout
 * as documented for lora_shrink_workspace_bytes) and nothing else.  The
 * partials are the unit a row-parallel layer would exchange between devices
 * before the fixed-order combine.
 *
 * lora_expand_combine: for each 16-token block, evaluates the same fixed
 * pairwise tree over the split_k workspace slices and the multiply by
 * shrink_scale that lora_shrink_splitk's second pass applies, writes the
 * result to h when h is not NULL, and feeds it (rounded to bf16) into the
 * expand of lora_expand with expand_scale.  The workspace must hold split_k
 * slices of M x r floats.
 *
 * lora_shrink_expand: h and y bit for bit those of lora_shrink_splitk followed
 * by lora_expand, in fewer launches: the two calls above in order on one
 * stream; or (small M and A) the single launch of lora_shrink_expand_fused; or,
 * when ceil(N / 256) * split_k > 256 or M * r * ceil(N / 256) > 2^19 (every
 * column block re-evaluating the tree would cost more than a launch), the
 * partials, the tree kernel and the expand kernel - without h, h is then kept
 * in workspace slice 0 (when r % 4 == 0; with h, when h's rows are 16-byte
 * aligned).  The workspace content is undefined afterwards.
 *
 * workspace: >= lora_shrink_expand_workspace_bytes(M, r, split_k) bytes =
 * split_k * M * r * 4, also for split_k == 1.  Requirements: those of
 * lora_shrink_splitk and lora_expand together.
 */
size_t lora_shrink_expand_workspace_bytes(int64_t M, int32_t r, int32_t split_k);

int lora_shrink_partials(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a,
                         int64_t M, int64_t K, int32_t r, int32_t split_k,
                         void* workspace, size_t workspace_bytes, void* stream);

int lora_expand_combine(const void* workspace, size_t workspace_bytes, int32_t split_k,
                        float shrink_scale, const uint16_t* B, int64_t ld_b, float* h, int64_t ld_h,
                        uint16_t* y, int64_t ld_y, int64_t M, int32_t r, int64_t N,
                        float expand_scale, void* stream);

/*
 * lora_shrink_expand_fused: the same h and y in ONE launch and without a
 * workspace.  Each workgroup owns a 16-token block and 512 output columns and
 * recomputes that block's deterministic Split-K shrink - the same chunks,
 * matrix-core chains, wave tree and split tree as lora_shrink_splitk, held in
 * registers and LDS - before expanding it, so no workgroup depends on another.
 * lora_shrink_expand runs this schedule when it is the faster one (small M).
 * Ranks above 64 return LORA_ERR_UNSUPPORTED here (lora_shrink_expand takes
 * another schedule for them).
 */
/* Host only: how many kernel launches lora_shrink_expand makes for these sizes
   (1: the single-launch schedule, 2: partials then tree + expand, 3:
   partials, tree, expand - 2 instead when the h rows do not allow it, see
   above - 0: nothing to do), or -LORA_ERR_UNSUPPORTED for sizes it rejects. */
int lora_shrink_expand_launches(int64_t M, int64_t K, int32_t r, int64_t N, int32_t split_k);

int lora_shrink_expand_fused(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a,
                             const uint16_t* B, int64_t ld_b, float* h, int64_t ld_h,
                             uint16_t* y, int64_t ld_y, int64_t M, int64_t K, int32_t r, int64_t N,
                             int32_t split_k, float shrink_scale, float expand_scale, void* stream);

int lora_shrink_expand(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a,
                       const uint16_t* B, int64_t ld_b, float* h, int64_t ld_h,
                       uint16_t* y, int64_t ld_y, int64_t M, int64_t K, int32_t r, int64_t N,
                       int32_t split_k, float shrink_scale, float expand_scale,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * lora_shrink_expand_noalloc: lora_shrink_expand for callers that cannot
 * allocate device memory (code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid allocation).  Same arguments without the
 * workspace, same launches, same h and y bit for bit.  The Split-K workspace is
 * a fixed buffer of LORA_NOALLOC_SCRATCH_BYTES inside the library (a static
 * device array, one per device, created with the library's code object on that
 * device and held until the process ends); the call allocates nothing.
 *
 * Limit: split_k * M * r * 4 <= LORA_NOALLOC_SCRATCH_BYTES (8 MiB: e.g.
 * M <= 4096 at r = 64, split_k = 8), otherwise LORA_ERR_SCRATCH, checked on the
 * host before any HIP call.  The first call on a device looks the buffer's
 * address up (hipGetSymbolAddress, with that device current; LORA_ERR_LAUNCH
 * if it fails) and caches it.  The device is the stream's (the current device
 * for a NULL stream).
 *
 * Every call on one device uses the same buffer, which keeps the last call's
 * partials: calls that may overlap on one device (different streams, or
 * threads enqueueing concurrently) race on it and must be ordered by the
 * caller.  The buffer needs no clearing: each call writes every element it
 * later reads.
 */
#define LORA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

int lora_shrink_expand_noalloc(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a,
                               const uint16_t* B, int64_t ld_b, float* h, int64_t ld_h,
                               uint16_t* y, int64_t ld_y, int64_t M, int64_t K, int32_t r, int64_t N,
                               int32_t split_k, float shrink_scale, float expand_scale, void* stream);

/*
 * lora_shrink_expand_counted: the same h and y as lora_shrink_expand in ONE
 * launch, with a workspace and a counter buffer.  The grid holds, for each
 * 16-token block, its Split-K shrink workgroups (the partial kernel of
 * lora_shrink_partials with agent-scope atomic stores, then, after a barrier,
 * one agent-scope RELEASE add to the block's arrival counter) followed by its
 * expand workgroups, which load their y tile and B rows, wait until the
 * block's counter shows every partial, issue an agent-scope ACQUIRE fence,
 * then evaluate the
 * tree + expand of lora_expand_combine.  The wait is bounded; workgroups are
 * dispatched in increasing id and every shrink workgroup of a block precedes
 * the block's expand workgroups, so the wait ends once they have run.
 *
 * counters: int32 [lora_shrink_expand_counter_bytes(M) / 4], 4-byte aligned,
 * ALL ZERO before the first call.  Layout: counters[0] is a status word,
 * counters[1..3] are unused, then two counters (arrivals, departures) per
 * 16-token block.  Every completed call leaves the block counters zero, so one
 * buffer serves any number of calls, of any M up to the one it was sized for,
 * on one stream; calls that share a buffer must not overlap.  An expand
 * workgroup that waited too long (not expected) sets counters[0] to 1 and
 * leaves its part of y unchanged; the results of that call are then
 * incomplete and the whole buffer must be zeroed again before the next call.
 * workspace: as for lora_shrink_expand.  Other requirements: those of
 * lora_shrink_expand.
 */
size_t lora_shrink_expand_counter_bytes(int64_t M);

int lora_shrink_expand_counted(const uint16_t* x, int64_t ld_x, const uint16_t* A, int64_t ld_a,
                               const uint16_t* B, int64_t ld_b, float* h, int64_t ld_h,
                               uint16_t* y, int64_t ld_y, int64_t M, int64_t K, int32_t r, int64_t N,
                               int32_t split_k, float shrink_scale, float expand_scale,
                               void* workspace, size_t workspace_bytes, int32_t* counters,
                               size_t counter_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Multi-adapter (SGMV) variants.  The paper replays shrink operations with the
 * mapping of tokens to adapters (section 5.2); here each token i carries an
 * adapter id token_adapter[i].  Ids outside [0, n_adapters) mean "no LoRA":
 * the h row is written as zeros and the y row is left untouched.
 *
 * Adapter a has rank ranks[a] (1..r_max), weights A_ptrs[a] -> bf16
 * [ranks[a]][ld_a] and B_ptrs[a] -> bf16 [N][rb_a] with row stride
 * rb_a = ranks[a] rounded up to a multiple of 8 (contiguous when the rank is a
 * multiple of 8), and scale scales[a] (scales == NULL means 1).  A_ptrs, B_ptrs,
 * ranks, scales and token_adapter are DEVICE arrays; their contents are read by
 * the kernels, so the caller guarantees 1 <= ranks[a] <= r_max and valid,
 * 16-byte aligned weight pointers.  Each token's bits equal those of the
 * single-adapter call with that token's adapter.
 * ------------------------------------------------------------------------- */

/* Bytes of the plan buffer for M tokens: 16 + 16 * M. */
size_t lora_sgmv_plan_bytes(int64_t M);

/*
 * Builds the work list from the per-token ids, on the device and without a
 * host synchronisation: tiles of up to 16 tokens with one adapter, either
 * runs of equal id cut into pieces of at most 16 consecutive tokens, or (up
 * to 4096 tokens, where the runs give at least two tiles per 16-token block
 * and this gives fewer, e.g. for interleaved ids) one tile per distinct id of
 * each aligned 16-token block, masked to its tokens.
 * Tokens without a valid adapter get tiles marked -1.  The tiling changes no
 * output bit.  One launch of one workgroup.  The plan buffer (16-byte
 * aligned) is opaque; it stays valid for later sgmv calls with the same ids,
 * M and n_adapters and may be reused by both sgmv_shrink and sgmv_expand.
 * Its header records M and n_adapters. A multi-adapter shrink given a plan
 * made for other values processes no tile, so none of the stale entries is
 * followed. Its h is then not computed: the single launch leaves h as it
 * was, and the two-pass shrink's second pass reads whatever the workspace
 * holds.
 */
int lora_sgmv_plan(const int32_t* token_adapter, int64_t M, int32_t n_adapters,
                   void* plan, size_t plan_bytes, void* stream);

/* Workspace bytes for lora_sgmv_shrink: split_k * M * r_max * 4 (layout as
   for the single-adapter shrink with r_max columns).  0 for invalid input. */
size_t lora_sgmv_workspace_bytes(int64_t M, int32_t r_max, int32_t split_k);

/*
 * Multi-adapter deterministic Split-K shrink: per token, the single-adapter
 * shrink with its adapter's A, rank and scale; h columns in [rank, r_max) and
 * rows of tokens without an adapter are written as 0.  Two launches (partials
 * over the plan's tiles, then the fixed tree) for every split_k, including 1.
 */
int lora_sgmv_shrink(const uint16_t* x, int64_t ld_x, const uint16_t* const* A_ptrs, int64_t ld_a,
                     const int32_t* ranks, const float* scales, const int32_t* token_adapter,
                     int32_t n_adapters, const void* plan, size_t plan_bytes,
                     float* h, int64_t ld_h, int64_t M, int64_t K, int32_t r_max, int32_t split_k,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Multi-adapter single-launch shrink: lora_sgmv_shrink's result (same bits) in
 * one launch with the tagged-slot combine of lora_shrink_splitk_counted,
 * one counter per plan tile and rank group.  The plan must come from
 * lora_sgmv_plan with the same M and n_adapters (token ids are read from the
 * plan).
 * workspace: lora_counted_workspace_bytes(M, r_max, split_k) bytes, all zero
 * before the first call, left zero, not shared with other entry points.
 * counters: int32 [lora_sgmv_counter_bytes(M) / 4] (8 per possible tile), all
 * zero before the first call, left zero.
 */
size_t lora_sgmv_counter_bytes(int64_t M);

int lora_sgmv_shrink_counted(const uint16_t* x, int64_t ld_x, const uint16_t* const* A_ptrs,
                             int64_t ld_a, const int32_t* ranks, const float* scales,
                             int32_t n_adapters, const void* plan, size_t plan_bytes,
                             float* h, int64_t ld_h, int64_t M, int64_t K, int32_t r_max,
                             int32_t split_k, void* workspace, size_t workspace_bytes,
                             int32_t* counters, size_t counter_bytes, void* stream);

/*
 * lora_sgmv_shrink_atomic: the nondeterministic contrast for the multi-adapter
 * shrink (the atomic Split-K baseline of paper section 4.1, replayed with the
 * token-to-adapter mapping as in section 5.2).  h's first r_max columns are
 * zeroed by a fill kernel, then the partial kernel that lora_sgmv_shrink would
 * run (same work items, same plan) adds each split's partial times the
 * adapter's scale (scales[a], NULL = 1) into h with fp32 atomic adds, in
 * whatever order the splits finish.  Tokens without an adapter, and columns
 * from the adapter's rank on, stay zero.  No workspace.  Values agree with
 * lora_sgmv_shrink to rounding; the bits may differ between runs.  Arguments
 * as for lora_sgmv_shrink (the token ids are read from the plan).
 */
int lora_sgmv_shrink_atomic(const uint16_t* x, int64_t ld_x, const uint16_t* const* A_ptrs, int64_t ld_a,
                            const int32_t* ranks, const float* scales, int32_t n_adapters,
                            const void* plan, size_t plan_bytes, float* h, int64_t ld_h,
                            int64_t M, int64_t K, int32_t r_max, int32_t split_k, void* stream);

/*
 * Multi-adapter shrink + expand: the partial kernel of lora_sgmv_shrink, then
 * either (two launches) an expand that evaluates each token's h from the
 * Split-K workspace (the same fixed tree and shrink_scales[a] multiply as
 * lora_sgmv_shrink's second pass, zeros past the adapter's rank), writes it
 * to h when h is not NULL and applies lora_sgmv_expand's update with
 * expand_scales[a]; or (three launches, when ceil(N / 256) * split_k > 256
 * or M * r_max * ceil(N / 256) > 2^19, where every column block re-evaluating
 * the tree would cost more than a launch) the tree kernel, then
 * lora_sgmv_expand's kernel.  The three-launch schedule needs 16-byte h rows:
 * with h, a 16-byte aligned h with ld_h % 4 == 0; without h, it keeps h in
 * workspace slice 0 (when r_max % 4 == 0); otherwise it takes the two-launch
 * schedule.  Either way h and y are bit for bit
 * those of lora_sgmv_shrink(scales = shrink_scales) followed by
 * lora_sgmv_expand(scales = expand_scales); either scale array may be NULL
 * (all 1).  Arguments and requirements as for those two calls; h is
 * optional here (4-byte aligned, ld_h >= r_max when given); the workspace
 * content is undefined afterwards.
 */
int lora_sgmv_shrink_expand(const uint16_t* x, int64_t ld_x, const uint16_t* const* A_ptrs, int64_t ld_a,
                            const uint16_t* const* B_ptrs, const int32_t* ranks, const float* shrink_scales,
                            const float* expand_scales, const int32_t* token_adapter, int32_t n_adapters,
                            const void* plan, size_t plan_bytes, float* h, int64_t ld_h,
                            uint16_t* y, int64_t ld_y, int64_t M, int64_t K, int64_t N, int32_t r_max,
                            int32_t split_k, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Multi-adapter expand: per token i with an adapter (a = token_adapter[i] in
 * [0, n_adapters)), lora_expand with B_a, rank r_a and scale scales[a] (1 when
 * scales is NULL); rows of other tokens are neither read nor written.  One
 * launch, one workgroup per 16 tokens x 256 columns; a block whose tokens use
 * several adapters makes one matrix-core pass per adapter.  Each token's bits
 * equal the single-adapter lora_expand's with its adapter (they do not depend
 * on M, the token's neighbours or their adapters).
 * h: fp32 [M][ld_h], 16-byte aligned, ld_h % 4 == 0, columns < r_a read.
 * B_ptrs: device array of n_adapters pointers, B_a bf16 [N][round_up(r_a, 8)],
 * 16-byte aligned.  token_adapter: device int32 [M].
 */
int lora_sgmv_expand(const float* h, int64_t ld_h, const uint16_t* const* B_ptrs,
                     const int32_t* ranks, const float* scales, const int32_t* token_adapter,
                     int32_t n_adapters, uint16_t* y, int64_t ld_y,
                     int64_t M, int64_t N, int32_t r_max, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_DET_H */
