// elem.h -- the 16-bit storage types of the cache and of the call's tensors.
//
// operator-development.md ("Public interfaces") types the cached-row softmax
// for FP16 and BF16 inputs, reducing in FP32 and rounding only the caller's
// output.  Every kernel of this library is written once over a storage type
// E picked at compile time; E supplies:
//   to_f / lo / hi   exact widening of one code (lo / hi: the halves of a
//                    32-bit word) to FP32;
//   from_f           FP32 -> code, round to nearest even (any FP32 input);
//   cvt2 / pack2     two finite FP32 values -> a packed pair by the gfx950
//                    conversion instruction (round to nearest even);
//   part<NPART>      the split of an FP32 value into NPART codes whose sum
//                    carries it into the matrix cores (see each type);
//   mma16 / mma32    v_mfma_f32_16x16x32_* / v_mfma_f32_32x32x16_* on 8-code
//                    operands, FP32 accumulation;
//   sum2             acc + the two codes of a packed pair (v_dot2c_f32_*).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mllm {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// BF16: the top half of an FP32 value.
struct Bf16 {
    typedef bf16x8 vec8;
    typedef bf16x2 vec2;
    static constexpr int code = 1;  // MLLM_BF16
    static constexpr uint16_t qnan = 0x7fc0;
    // parts of an FP32 query or weight: three reproduce it exactly (8 + 8 + 8
    // significant bits); two carry it to 2^-16 relative
    static constexpr int max_parts = 3;

    __device__ static float to_f(uint32_t h) { return __uint_as_float(h << 16); }
    __device__ static float lo(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ static float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
    // round to nearest even; NaN stays a quiet NaN
    __device__ static uint32_t from_f(float f)
    {
        const uint32_t u = __float_as_uint(f);
        if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu))
            return (u >> 16) | 0x40u;
        return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    }
    __device__ static vec2 cvt2(float a, float b)
    {
        return __builtin_convertvector(f32x2{a, b}, bf16x2);
    }
    __device__ static uint32_t pack2(float a, float b) { return __builtin_bit_cast(uint32_t, cvt2(a, b)); }
    // part p of x: with three parts hi + mid + lo == x exactly (each remainder
    // is exact and the last has at most 8 significant bits); with two parts
    // the remainder is rounded to nearest
    template <int NPART>
    __device__ static uint32_t part(float x, int p)
    {
        const uint32_t h = __float_as_uint(x) & 0xffff0000u;
        if (p == 0)
            return h >> 16;
        const float r1 = x - __uint_as_float(h);
        if (NPART == 2)  // the conversion instruction: nearest even, as from_f
            return __builtin_bit_cast(uint16_t, (__bf16)r1);
        const uint32_t mid = __float_as_uint(r1) & 0xffff0000u;
        if (p == 1)
            return mid >> 16;
        const float r2 = r1 - __uint_as_float(mid);
        return __float_as_uint(r2) >> 16;
    }
    __device__ static f32x4 mma16(vec8 a, vec8 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static f32x16 mma32(vec8 a, vec8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static float sum2(vec2 p, float acc)
    {
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(p, one, acc, false);
    }
};

// FP16: IEEE binary16.
struct F16 {
    typedef f16x8 vec8;
    typedef f16x2 vec2;
    static constexpr int code = 2;  // MLLM_F16
    static constexpr uint16_t qnan = 0x7e00;
    // two parts carry an FP32 value to 2^-22 relative (11 + 11 significant
    // bits; below the FP16 normal range to 2^-25 absolute).  An FP32 value of
    // magnitude 65520 or more has no FP16 part: such a rotated query (from
    // inputs near the FP16 maximum) is outside what this path supports.
    static constexpr int max_parts = 2;

    __device__ static float to_f(uint32_t h)
    {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    }
    __device__ static float lo(uint32_t w) { return to_f(w & 0xffffu); }
    __device__ static float hi(uint32_t w) { return to_f(w >> 16); }
    // the conversion instruction: round to nearest even, overflow to
    // infinity, subnormals kept, NaN quiet
    __device__ static uint32_t from_f(float f)
    {
        return __builtin_bit_cast(uint16_t, (_Float16)f);
    }
    __device__ static vec2 cvt2(float a, float b)
    {
        return __builtin_convertvector(f32x2{a, b}, f16x2);
    }
    __device__ static uint32_t pack2(float a, float b) { return __builtin_bit_cast(uint32_t, cvt2(a, b)); }
    // part 0 = x rounded to FP16; part 1 = the exact remainder rounded to FP16
    template <int NPART>
    __device__ static uint32_t part(float x, int p)
    {
        static_assert(NPART == 2, "FP16 splits into two parts");
        const _Float16 h = (_Float16)x;
        if (p == 0)
            return __builtin_bit_cast(uint16_t, h);
        return __builtin_bit_cast(uint16_t, (_Float16)(x - (float)h));
    }
    __device__ static f32x4 mma16(vec8 a, vec8 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    __device__ static f32x16 mma32(vec8 a, vec8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static float sum2(vec2 p, float acc)
    {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(p, one, acc, false);
    }
};

}  // namespace mllm
