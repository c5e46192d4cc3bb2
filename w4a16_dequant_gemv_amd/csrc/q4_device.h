// q4_device.h -- device-side types and helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From &v)
{
    static_assert(sizeof(To) == sizeof(From), "size mismatch");
    return __builtin_bit_cast(To, v);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h)
{
    return (float)bitcast<_Float16>(h);
}

// One packed word holds codes c0..c7 (c_t in bits 4t..4t+3).  OR-ing a code
// into the mantissa of the half 1024.0 (0x6400) gives the exact half 1024 + c,
// so four AND-OR operations produce the pairs (c0,c4), (c1,c5), (c2,c6),
// (c3,c7), each as two halves 1024 + c.
__device__ __forceinline__ void unpack_biased_pairs(uint32_t w, uint32_t h[4])
{
    h[0] = (w & 0x000F000Fu) | 0x64006400u;
    h[1] = ((w >> 4) & 0x000F000Fu) | 0x64006400u;
    h[2] = ((w >> 8) & 0x000F000Fu) | 0x64006400u;
    h[3] = ((w >> 12) & 0x000F000Fu) | 0x64006400u;
}

// Eight dequantized weights s * (c - z) in the pair order above.  The
// subtraction (1024 + c) - (1024 + z) is exact in fp16; the product with s
// is the only rounding (to fp16).
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t w, f16x2 bias, f16x2 scale)
{
    uint32_t h[4];
    unpack_biased_pairs(w, h);
    f16x8 r;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f16x2 v = (bitcast<f16x2>(h[t]) - bias) * scale;
        r[2 * t] = v[0];
        r[2 * t + 1] = v[1];
    }
    return r;
}

// Reorders eight consecutive halves x0..x7 (as four dwords) into the pair
// order (x0,x4), (x1,x5), (x2,x6), (x3,x7) used by dequant8_f16.
__device__ __forceinline__ f16x8 pair_order(u32x4 d)
{
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);
    r[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);
    r[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
    r[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
    return bitcast<f16x8>(r);
}
