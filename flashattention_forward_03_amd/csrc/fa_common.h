// Shared device helpers of the gfx950 attention kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32x16 MFMA, fp32 accumulate.  Operand lane layout (checked on gfx950):
// A (32 rows x 16 k): lane l holds row l%32, k = 8*(l/32) .. +7.
// B (16 k x 32 cols): lane l holds col l%32, k = 8*(l/32) .. +7.
// C (32 x 32): register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, col l%32.
template <bool BF16>
__device__ __forceinline__ f32x16_t mma32(u32x4_t a, u32x4_t b, f32x16_t c)
{
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Two fp32 -> packed 16-bit pair (round to nearest even), lo in bits 0..15.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    if constexpr (BF16) {
        bf16x2_t v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        f16x2_t v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
}

template <bool BF16>
__device__ __forceinline__ float lo16(uint32_t x)
{
    if constexpr (BF16)
        return __uint_as_float(x << 16);
    else
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
}

template <bool BF16>
__device__ __forceinline__ float hi16(uint32_t x)
{
    if constexpr (BF16)
        return __uint_as_float(x & 0xffff0000u);
    else
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of x held by lane l^32 (the other half of the wave).
__device__ __forceinline__ float other_half(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const bool lower = (threadIdx.x & 32) == 0;
    return __uint_as_float(lower ? r[1] : r[0]);
}

// Sum over the 16 lanes of a DPP row (lanes 16k .. 16k+15), result in all of them.
__device__ __forceinline__ float row16_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)); // row_half_mirror
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)); // row_mirror
    return x;
}

// Sum over aligned groups of 8 lanes.
__device__ __forceinline__ float row8_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    return x;
}

__device__ __forceinline__ u32x4_t load16(const uint16_t *p)
{
    return *reinterpret_cast<const u32x4_t *>(p);
}

// Round-robin dispatch places workgroup g on XCD g % 8.  Renumber so that
// each XCD receives a contiguous range of logical work ids (work that shares
// K/V then shares that XCD's L2).
__device__ __forceinline__ int xcd_contiguous_id(int g, int G)
{
    const int per = G >> 3, rem = G & 7, x = g & 7, i = g >> 3;
    return x * per + (x < rem ? x : rem) + i;
}

}  // namespace fa
