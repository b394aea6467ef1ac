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

// 16-byte load of 8 bf16 (the address is 16-byte aligned by the host checks).
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p)
{
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
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
