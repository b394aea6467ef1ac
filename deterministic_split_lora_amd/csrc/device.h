// Device-side building blocks shared by the gfx950 kernels of this library.
//
// The matrix-core primitive is V_MFMA_F32_16X16X32_BF16 (CDNA4): a 64-lane
// wavefront multiplies a 16x32 bf16 tile by a 32x16 bf16 tile and adds a 16x16
// fp32 accumulator.  Operand registers, per lane l (li = l % 16, g = l / 16):
//   src0 ("rows")    : 8 bf16 of row li, reduction slots 8g .. 8g+7
//   src1 ("columns") : 8 bf16 of column li, reduction slots 8g .. 8g+7
//   acc              : 4 fp32, output rows 4g .. 4g+3 of column li
// Both sources use the same slot layout, so any one-to-one assignment of real
// reduction indices to slots (the same for both) yields the same products.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kKStep = 32;      // reduction depth of one matrix-core step

__device__ __forceinline__ bf16x8 bf16x8_zero()
{
    return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// 16-byte load of 8 bf16 from device memory (the address is 16-byte aligned by
// the host checks).  The pointer is used as a global-memory pointer, so an
// adapter pointer read from a device array still gets a global load rather
// than a flat one.
typedef __attribute__((address_space(1))) const u32x4 global_u32x4;

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p)
{
    return __builtin_bit_cast(bf16x8, *(const global_u32x4*)(p));
}

// Raw buffer resource over `bytes` bytes from `base` (stride 0: offsets are
// byte offsets; stores at or past `bytes` are dropped by the hardware), and a
// 4-byte store through it at a per-lane byte offset.  The resource lives in
// scalar registers.
typedef __amdgpu_buffer_rsrc_t BufferRsrc;
constexpr int kBufferRsrcWord3 = 0x00020000;   // raw 32-bit data, CDNA buffer format

__device__ __forceinline__ BufferRsrc buffer_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferRsrcWord3);
}

__device__ __forceinline__ void buffer_store_f32(float v, BufferRsrc r, uint32_t byte_offset)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, (int)byte_offset, 0, 0);
}

// 4-byte fp32 atomic add through the same kind of resource (a vector memory
// atomic; used only by the nondeterministic contrast).
__device__ __forceinline__ void buffer_atomic_add_f32(float v, BufferRsrc r, uint32_t byte_offset)
{
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, r, (int)byte_offset, 0, 0);
}

// 8 bf16 starting at p of which only the first n exist (n < 8 only at a
// rank edge that is not a multiple of 8); missing ones read as +0 so that
// padded reduction slots contribute exact zeros.
__device__ __forceinline__ bf16x8 load_bf16x8_partial(const uint16_t* p, int n)
{
    if (n >= 8)
        return load_bf16x8(p);
    u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (e < n)
            v[e] = p[e];
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 rows, bf16x8 cols, f32x4 acc)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(rows, cols, acc, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b)
{
    return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// h[row][j0 .. j0+7] with columns >= r read as 0.
__device__ __forceinline__ void load_h8(const float* hp, int j0, int r, float (&f)[8])
{
    if (j0 + 8 <= r) {
        const float4 a = *reinterpret_cast<const float4*>(hp);
        const float4 b = *reinterpret_cast<const float4*>(hp + 4);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            f[e] = (j0 + e < r) ? hp[e] : 0.0f;
    }
}

// bf16(h[row][j0 .. j0+7]) with columns >= r read as 0.
__device__ __forceinline__ bf16x8 load_h_as_bf16(const float* hp, int j0, int r)
{
    float f[8];
    load_h8(hp, j0, r, f);
    u16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        v[e] = f32_to_bf16_bits(f[e]);
    return __builtin_bit_cast(bf16x8, v);
}

// The same for j0 + 8 <= r: two 16-byte loads, no per-element checks.
__device__ __forceinline__ bf16x8 load_h_as_bf16_whole(const float* hp)
{
    const float4 a = *reinterpret_cast<const float4*>(hp);
    const float4 b = *reinterpret_cast<const float4*>(hp + 4);
    const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    u16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        v[e] = f32_to_bf16_bits(f[e]);
    return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------
// Expand tile, shared by every kernel that expands (so the per-element
// arithmetic is literally the same code): a wavefront owns 16 tokens x 64
// output columns.  The matrix-core "row" operand is B (a row per output column)
// and the "column" operand is bf16(h) (a column per token); accumulator
// register v of lane (li, g) is output row 4g+v of column li.  Operand row m of
// tile t (0..3) stands for column  n_base + 16 (m / 4) + 4 t + (m % 4),  so lane
// (li, g) collects columns n_base + 16 g + 4 t + v - a contiguous run of 16 -
// for token li, and y moves with 16-byte loads and stores straight from the
// accumulators.  Per element: one matrix-core step over j < 32 (r <= 32), two
// (r <= 64) or four (r <= 128) with zero-padded reduction slots, then
// fma(scale, acc, y) and one rounding to bf16.
// ---------------------------------------------------------------------------
// Matrix-core steps of 32 the expand takes at rank r: 1 (r <= 32), 2 (r <= 64)
// or 4 (r <= 128).  Every expand kernel takes exactly this many for a token of
// rank r, whatever rank bound it was built for, so their bits agree.
__host__ __device__ constexpr int expand_steps(int r)
{
    return r <= 32 ? 1 : (r <= 64 ? 2 : 4);
}

template <int N>
struct Steps {
    static constexpr int value = N;
};

struct ExpandLane {
    int64_t row;        // this lane's token (clamped into the block)
    int64_t n_base;     // first column of this wave
    int li, g;
    bool row_ok;
};

__device__ __forceinline__ ExpandLane expand_lane(int64_t row0, int nrows, int64_t col0)
{
    ExpandLane L;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    L.li = lane & 15;
    L.g = lane >> 4;
    L.row_ok = L.li < nrows;
    L.row = row0 + (L.row_ok ? L.li : 0);
    L.n_base = col0 + wave * 64;
    return L;
}

// This lane's 16 y values (zeros for a row outside the block).
__device__ __forceinline__ void expand_load_y(const ExpandLane& L, const uint16_t* y, int64_t ld_y, int64_t N,
                                              u16x8 (&yv)[2])
{
    const int64_t n0 = L.n_base + 16 * L.g;
    const uint16_t* yp = y + L.row * ld_y + n0;
#pragma unroll
    for (int half = 0; half < 2; ++half)
        yv[half] = (L.row_ok && n0 + half * 8 < N) ? *reinterpret_cast<const u16x8*>(yp + half * 8)
                                                  : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
}

// This lane's B operand rows (KS steps of 32 over r; zeros past r and N).
// Rows of B hold ld_b >= r elements with ld_b a multiple of 8 (checked by
// every entry point), so the 8 elements from any j0 < r (j0 a multiple of 8)
// lie inside the row: each operand is one full 16-byte load, and only for a
// rank that is not a multiple of 8 are the elements from r on cleared
// afterwards (EDGE; the choice is uniform and made once, so the common case
// is one straight run of loads).  These kernels are latency-bound:
// per-element partial loads made their code a third longer and the step
// slower.
template <int KS, bool EDGE>
__device__ __forceinline__ void expand_load_b_run(const ExpandLane& L, int64_t N, const uint16_t* __restrict__ B,
                                                  int64_t ld_b, int r, bf16x8 (&bop)[4][KS])
{
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int64_t n = L.n_base + (L.li >> 2) * 16 + t * 4 + (L.li & 3);
        const bool n_ok = n < N;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int j0 = ks * kKStep + 8 * L.g;
            u32x4 v = (n_ok && j0 < r) ? *(const global_u32x4*)(B + n * ld_b + j0) : u32x4{0u, 0u, 0u, 0u};
            if constexpr (EDGE) {
                const int rem = r - j0;
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    v[d] &= (2 * d < rem ? 0x0000FFFFu : 0u) | (2 * d + 1 < rem ? 0xFFFF0000u : 0u);
            }
            bop[t][ks] = __builtin_bit_cast(bf16x8, v);
        }
    }
}

template <int KS>
__device__ __forceinline__ void expand_load_b(const ExpandLane& L, int64_t N, const uint16_t* __restrict__ B,
                                              int64_t ld_b, int r, bf16x8 (&bop)[4][KS])
{
    if ((r & 7) == 0)                              // uniform
        expand_load_b_run<KS, false>(L, N, B, ld_b, r, bop);
    else
        expand_load_b_run<KS, true>(L, N, B, ld_b, r, bop);
}

// Loads this lane's 16 y values and its B operand rows.
template <int KS>
__device__ __forceinline__ void expand_load(const ExpandLane& L, const uint16_t* y, int64_t ld_y, int64_t N,
                                            const uint16_t* __restrict__ B, int64_t ld_b, int r, u16x8 (&yv)[2],
                                            bf16x8 (&bop)[4][KS])
{
    expand_load_y(L, y, ld_y, N, yv);
    expand_load_b<KS>(L, N, B, ld_b, r, bop);
}

// The matrix-core steps and the updated y values of this lane's 16 columns,
// given its bf16(h) operand (its token's h[j], j = 32 ks + 8 g .. + 7, zeros
// from r on):  o = bf16(fma(scale, sum_j bf16(h[j]) B[n][j], y)).
template <int KS>
__device__ __forceinline__ void expand_mma(const bf16x8 (&hb)[KS], float scale, const u16x8 (&yv)[2],
                                           const bf16x8 (&bop)[4][KS], u16x8 (&o)[2])
{
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            acc[t] = mfma_16x16x32(bop[t][ks], hb[ks], acc[t]);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int idx = half * 8 + e;
            o[half][e] = f32_to_bf16_bits(__builtin_fmaf(scale, acc[idx >> 2][idx & 3], bf16_bits_to_f32(yv[half][e])));
        }
}

// expand_mma, then the lane's 16 y values stored straight to y.
template <int KS>
__device__ __forceinline__ void expand_mma_store(const ExpandLane& L, uint16_t* y, int64_t ld_y, int64_t N,
                                                 const bf16x8 (&hb)[KS], float scale, const u16x8 (&yv)[2],
                                                 const bf16x8 (&bop)[4][KS])
{
    u16x8 o[2];
    expand_mma<KS>(hb, scale, yv, bop, o);
    if (!L.row_ok)
        return;
    const int64_t n0 = L.n_base + 16 * L.g;
    uint16_t* yp = y + L.row * ld_y + n0;
#pragma unroll
    for (int half = 0; half < 2; ++half)
        if (n0 + half * 8 < N)
            *reinterpret_cast<u16x8*>(yp + half * 8) = o[half];
}

// bf16(h) of the block's token rows (hrows: row 0 of the block, stride ld_hr),
// the matrix-core steps, and the y update.  N % 8 == 0, so 8-column chunks
// are whole.
template <int KS>
__device__ __forceinline__ void expand_finish(const ExpandLane& L, uint16_t* y, int64_t ld_y, int64_t N,
                                              const float* hrows, int64_t ld_hr, int r, float scale,
                                              const u16x8 (&yv)[2], const bf16x8 (&bop)[4][KS])
{
    bf16x8 hb[KS];
    if ((r & 7) == 0) {                            // uniform: whole groups of 8 columns
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int j0 = ks * kKStep + 8 * L.g;
            hb[ks] = (L.row_ok && j0 < r) ? load_h_as_bf16_whole(hrows + L.li * ld_hr + j0) : bf16x8_zero();
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int j0 = ks * kKStep + 8 * L.g;
            hb[ks] = (L.row_ok && j0 < r) ? load_h_as_bf16(hrows + L.li * ld_hr + j0, j0, r) : bf16x8_zero();
        }
    }
    expand_mma_store<KS>(L, y, ld_y, N, hb, scale, yv, bop);
}

// Compensated expand: h is split into hi = bf16(h) and lo = bf16(h - hi)
// (h - hi is exact in fp32), both go through the matrix-core steps with the
// same B operands, and the two fp32 results are added before the epilogue:
//   acc = acc(hi) + acc(lo);  y = bf16(fma(scale, acc, y)).
__device__ __forceinline__ void split_hi_lo(float f, uint16_t& hi, uint16_t& lo)
{
    hi = f32_to_bf16_bits(f);
    lo = f32_to_bf16_bits(__fsub_rn(f, bf16_bits_to_f32(hi)));
}

// The matrix-core steps and updated y values of this lane's 16 columns, given
// its hi and lo operands (zeros from r on) - every compensated expand kernel
// runs exactly this code.
template <int KS>
__device__ __forceinline__ void expand_mma_comp(const bf16x8 (&hi)[KS], const bf16x8 (&lo)[KS], float scale,
                                                const u16x8 (&yv)[2], const bf16x8 (&bop)[4][KS], u16x8 (&o)[2])
{
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f32x4 ah = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 al = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            ah = mfma_16x16x32(bop[t][ks], hi[ks], ah);
            al = mfma_16x16x32(bop[t][ks], lo[ks], al);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
            acc[t][v] = __fadd_rn(ah[v], al[v]);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int idx = half * 8 + e;
            o[half][e] = f32_to_bf16_bits(__builtin_fmaf(scale, acc[idx >> 2][idx & 3], bf16_bits_to_f32(yv[half][e])));
        }
}

template <int KS>
__device__ __forceinline__ void expand_finish_comp(const ExpandLane& L, uint16_t* y, int64_t ld_y, int64_t N,
                                                   const float* hrows, int64_t ld_hr, int r, float scale,
                                                   const u16x8 (&yv)[2], const bf16x8 (&bop)[4][KS])
{
    bf16x8 hi[KS], lo[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int j0 = ks * kKStep + 8 * L.g;
        u16x8 vh = {0, 0, 0, 0, 0, 0, 0, 0}, vl = {0, 0, 0, 0, 0, 0, 0, 0};
        if (L.row_ok && j0 < r) {
            float f[8];
            load_h8(hrows + L.li * ld_hr + j0, j0, r, f);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint16_t a, b;
                split_hi_lo(f[e], a, b);
                vh[e] = a;
                vl[e] = b;
            }
        }
        hi[ks] = __builtin_bit_cast(bf16x8, vh);
        lo[ks] = __builtin_bit_cast(bf16x8, vl);
    }
    u16x8 o[2];
    expand_mma_comp<KS>(hi, lo, scale, yv, bop, o);
    if (!L.row_ok)
        return;
    const int64_t n0 = L.n_base + 16 * L.g;
    uint16_t* yp = y + L.row * ld_y + n0;
#pragma unroll
    for (int half = 0; half < 2; ++half)
        if (n0 + half * 8 < N)
            *reinterpret_cast<u16x8*>(yp + half * 8) = o[half];
}

// ---------------------------------------------------------------------------
// Staging of an h tile for the expands that walk several 16-token tiles per
// workgroup: 16 rows x round_up(r, 8) columns of bf16(h) in LDS (row stride
// kHbStride), zeros past r and for rows outside the tile.  Each of the first
// 16 * round_up(r, 8) / HC threads converts one group of HC (4 or 8) columns,
// read with 16-byte loads (h is 16-byte aligned with ld_h % 4 == 0, so a
// 4-column part that starts below r ends inside the row's ld_h).  HC = 4
// covers ranks <= 64 with 256 threads, HC = 8 ranks <= 128.
// ---------------------------------------------------------------------------
constexpr int kHbStride = 136;            // bf16 per LDS row (128 + 8 padding)

struct HStageSlot {
    int row;
    int col;
    bool on;
};

template <int HC>
__device__ __forceinline__ HStageSlot h_stage_slot(int r)
{
    const int q = ((r + 7) & ~7) / HC;    // column groups per row
    HStageSlot s;
    s.row = (int)threadIdx.x / q;
    s.col = ((int)threadIdx.x - s.row * q) * HC;
    s.on = s.row < 16;
    return s;
}

// The slot's HC h values as stored (zeros for rows outside the tile; the
// columns from r on are cleared by h_put / h_put_comp).  Nothing here uses
// the loaded values, so the loads stay in flight until the tile is put into
// LDS - a prefetch of the next tile is not waited for at once (a wait for it
// would also wait for every older load of the wave).
template <int HC>
__device__ __forceinline__ void h_load(const HStageSlot& s, const float* h, int64_t ld_h, int64_t row0, int nrows,
                                       int r, float (&f)[HC])
{
#pragma unroll
    for (int e = 0; e < HC; ++e)
        f[e] = 0.f;
    if (!s.on || s.row >= nrows || s.col >= r)
        return;
    const float* hp = h + (row0 + s.row) * ld_h + s.col;
    const float4 v = *reinterpret_cast<const float4*>(hp);
    f[0] = v.x;
    f[1] = v.y;
    f[2] = v.z;
    f[3] = v.w;
    if constexpr (HC == 8) {
        if (s.col + 4 < r) {
            const float4 w = *reinterpret_cast<const float4*>(hp + 4);
            f[4] = w.x;
            f[5] = w.y;
            f[6] = w.z;
            f[7] = w.w;
        }
    }
}

// ... and their bf16 roundings put into the LDS tile, zeros from column r on.
template <int HC>
__device__ __forceinline__ void h_put(const HStageSlot& s, const float (&f)[HC], int r, uint16_t* tile)
{
    if (!s.on)
        return;
    uint16_t* d = tile + s.row * kHbStride + s.col;
#pragma unroll
    for (int e = 0; e < HC; ++e)
        d[e] = f32_to_bf16_bits(s.col + e < r ? f[e] : 0.f);
}

// ... or, for the compensated expand, the hi and lo halves of each value put
// into two LDS tiles.
template <int HC>
__device__ __forceinline__ void h_put_comp(const HStageSlot& s, const float (&f)[HC], int r, uint16_t* hi_tile,
                                           uint16_t* lo_tile)
{
    if (!s.on)
        return;
    uint16_t* dh = hi_tile + s.row * kHbStride + s.col;
    uint16_t* dl = lo_tile + s.row * kHbStride + s.col;
#pragma unroll
    for (int e = 0; e < HC; ++e) {
        uint16_t vh, vl;
        split_hi_lo(s.col + e < r ? f[e] : 0.f, vh, vl);
        dh[e] = vh;
        dl[e] = vl;
    }
}

// This lane's bf16(h) operand from a staged tile, zeros from column `r` on
// (r may be below the staged width: a lower adapter rank).
template <int KS>
__device__ __forceinline__ void hb_from_tile(const ExpandLane& L, const uint16_t* tile, int r, bf16x8 (&hb)[KS])
{
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int j0 = ks * kKStep + 8 * L.g;
        if (!L.row_ok || j0 >= r) {
            hb[ks] = bf16x8_zero();
            continue;
        }
        u16x8 v = *reinterpret_cast<const u16x8*>(tile + L.li * kHbStride + j0);
        if (j0 + 8 > r) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (j0 + e >= r)
                    v[e] = 0;
        }
        hb[ks] = __builtin_bit_cast(bf16x8, v);
    }
}

// Tables the kernels only read (plan entries, adapter weight pointers,
// ranks, scales), at a wave-uniform index, through the constant address
// space: scalar loads, also in kernels whose own stores keep the compiler from
// proving the tables unchanged.  It would otherwise use vector loads, whose
// wait (the vector-memory counter retires in order) also covers every older
// load or atomic of the wave.
template <typename T>
__device__ __forceinline__ T table_load(const T* t, int i)
{
    return ((const __attribute__((address_space(4))) T*)t)[i];
}

// Fixed pairwise tree over N values: v[0]+v[1], v[2]+v[3], ... then the same on
// the results, level by level; every add is one fp32 rounding.  N is a power
// of two.  The result is left in v[0].
template <int N>
__device__ __forceinline__ float pairwise_tree(float* v)
{
#pragma unroll
    for (int width = N; width > 1; width >>= 1) {
#pragma unroll
        for (int q = 0; q < width / 2; ++q)
            v[q] = __fadd_rn(v[2 * q], v[2 * q + 1]);
    }
    return v[0];
}

}  // namespace lora
