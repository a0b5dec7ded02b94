// Small device helpers shared by the fp8g kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8g {

// Saturating E4M3FN cast of four fp32 values, packed little-endian into one
// dword (value i in byte i).  Magnitudes are clamped to 448 first, so the
// hardware convert (round to nearest even, OCP E4M3FN on gfx950) never sees
// an out-of-range input; the sign of zero is kept.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
    a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
    b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
    c = __builtin_fminf(__builtin_fmaxf(c, -448.0f), 448.0f);
    d = __builtin_fminf(__builtin_fmaxf(d, -448.0f), 448.0f);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);  // bytes 0,1
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);       // bytes 2,3
    return (uint32_t)r;
}

// Saturating OCP E5M2 cast of four fp32 values (byte i = value i): clamped to
// 57344 first, then the hardware convert (round to nearest even); sign of zero kept.
__device__ __forceinline__ uint32_t e5m2_pack4(float a, float b, float c, float d) {
    a = __builtin_fminf(__builtin_fmaxf(a, -57344.0f), 57344.0f);
    b = __builtin_fminf(__builtin_fmaxf(b, -57344.0f), 57344.0f);
    c = __builtin_fminf(__builtin_fmaxf(c, -57344.0f), 57344.0f);
    d = __builtin_fminf(__builtin_fmaxf(d, -57344.0f), 57344.0f);
    int r = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);  // bytes 0,1
    r = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, r, true);       // bytes 2,3
    return (uint32_t)r;
}

__device__ __forceinline__ uint8_t e4m3_one(float a) {
    return (uint8_t)(e4m3_pack4(a, 0.0f, 0.0f, 0.0f) & 0xFFu);
}

// Two fp32 values -> two bf16 (round to nearest even) packed low / high, with
// the gfx950 conversion instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

}  // namespace fp8g
