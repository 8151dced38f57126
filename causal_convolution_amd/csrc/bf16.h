// bf16 <-> fp32 conversions shared by the kernels (bf16 values are handled as
// their 16-bit patterns; widening is exact, narrowing rounds to nearest even).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace wanvae {

__device__ inline float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ inline uint32_t f32_to_bf16_bits(float f) {
    __bf16 b = static_cast<__bf16>(f);  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b));
}

// two values rounded to nearest even and packed, lo in bits 0..15 (one
// v_cvt_pk_bf16_f32)
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float float2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, bf16x2_t));
}

}  // namespace wanvae
