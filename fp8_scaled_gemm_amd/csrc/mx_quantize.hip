// MXFP8 block quantizer: fp32 [rows, cols] -> E4M3 codes [rows, cols] and one
// UE8M0 scale code per 32 consecutive elements of a row.
//
// Block layout: one unsigned-byte scale per 32 elements of K, the scale tensor
// shaped (rows, cols / 32), as on the page "[sglang] FlashInfer v0.6.7 MXFP8
// Gemm 통합", section 1.  Per block j of a row:
//   amax = max |x| over its 32 elements
//   e    = the smallest integer with amax <= 448 * 2^e, clamped to [-127, 127]
//          (-127 for an all-zero block); code = e + 127 (UE8M0: 2^(code-127))
//   q    = E4M3_RNE(x * 2^-e)  -- an exact power-of-two scaling; by the choice
//          of e no element exceeds 448, so the cast never saturates.
// e from the bit fields of amax = m 2^E (1 <= m < 2): 448 2^e = 1.75 2^(e+8), so
// e = E - 8 when m <= 1.75 and E - 7 when m > 1.75 (significand bits above
// 0x600000); subnormal amax is first scaled by 2^24 (exact).
//
// HBM-bound: 4 bytes read, 1 + 1/32 bytes written per element.  The matrix is
// a flat array of blocks (cols % 32 == 0, so no block straddles rows): lane L
// holds 4 consecutive elements, eight lanes one block, whose amax is three
// xor-shuffles away.  Loads and stores carry the non-temporal hint.

#include "device_common.h"
#include "launch.h"

namespace fp8g {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int MX_UNROLL = 4;         // float4 loads in flight per lane and iteration
constexpr int MX_THREADS = 256;

__device__ __forceinline__ int mx_exponent(float amax) {
    const uint32_t u0 = __builtin_bit_cast(uint32_t, amax);
    const bool sub = (u0 >> 23) == 0;                          // zero or subnormal
    const uint32_t u = sub ? __builtin_bit_cast(uint32_t, amax * 16777216.0f) : u0;
    const int E = (int)(u >> 23) - 127 - (sub ? 24 : 0);
    const int e = E - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return u0 == 0 ? -127 : min(max(e, -127), 127);
}

__global__ __launch_bounds__(MX_THREADS) void quantize_mx_kernel(const v4f* __restrict__ x, int64_t nvec,
                                                                  uint32_t* __restrict__ q, uint8_t* __restrict__ sc) {
    const int tid = threadIdx.x;
    const int64_t step = (int64_t)gridDim.x * MX_THREADS * MX_UNROLL;
    for (int64_t base = (int64_t)blockIdx.x * MX_THREADS * MX_UNROLL; base < nvec; base += step) {
        v4f v[MX_UNROLL];
#pragma unroll
        for (int u = 0; u < MX_UNROLL; ++u) {
            const int64_t idx = base + u * MX_THREADS + tid;
            v[u] = idx < nvec ? __builtin_nontemporal_load(x + idx) : (v4f){0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < MX_UNROLL; ++u) {
            // vector idx belongs to block idx / 8; idx % 8 == tid % 8, so the eight
            // lanes of a block are an aligned group of eight
            float a = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[u].x), __builtin_fabsf(v[u].y)),
                                      __builtin_fmaxf(__builtin_fabsf(v[u].z), __builtin_fabsf(v[u].w)));
            a = __builtin_fmaxf(a, __shfl_xor(a, 1, 64));
            a = __builtin_fmaxf(a, __shfl_xor(a, 2, 64));
            a = __builtin_fmaxf(a, __shfl_xor(a, 4, 64));
            const int e = mx_exponent(a);
            const int64_t idx = base + u * MX_THREADS + tid;
            if (idx < nvec) {
                if ((tid & 7) == 0) sc[idx >> 3] = (uint8_t)(e + 127);
                const uint32_t w = e4m3_pack4(__builtin_amdgcn_ldexpf(v[u].x, -e), __builtin_amdgcn_ldexpf(v[u].y, -e),
                                              __builtin_amdgcn_ldexpf(v[u].z, -e), __builtin_amdgcn_ldexpf(v[u].w, -e));
                __builtin_nontemporal_store(w, q + idx);
            }
        }
    }
}

hipError_t launch_quantize_mx(const float* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* scale,
                              hipStream_t stream) {
    const int64_t nvec = rows * cols / 4;   // cols % 32 == 0
    if (nvec == 0) return hipSuccess;
    const int64_t per_block = (int64_t)MX_THREADS * MX_UNROLL;
    int64_t blocks = (nvec + per_block - 1) / per_block;
    if (blocks > 8192) blocks = 8192;       // grid-stride beyond: 32 workgroups per CU
    quantize_mx_kernel<<<dim3((unsigned)blocks), dim3(MX_THREADS), 0, stream>>>(
        reinterpret_cast<const v4f*>(x), nvec, reinterpret_cast<uint32_t*>(q), scale);
    return hipGetLastError();
}

}  // namespace fp8g
