// Row-wise E4M3 quantizer: s[r] = amax_r / 448, q = E4M3_RNE_SAT(x / s[r]).
//
// Scale rule: abs_max / 448 (page "FP8 推理基础设施（五）：从 DeepGEMM 到
// vLLM", `_calibrate_scales`), one scale per row (per token for activations,
// per output channel for weights, as the DeepGEMM call's scale_a / scale_b on
// the same page).
//
// HBM-bound: 4 bytes read + 1 byte written per element.  One wavefront owns
// one row; when the row fits (up to 8192 fp32 per wave) it is loaded once
// into registers with 16-byte loads, reduced with a 64-lane butterfly, and
// converted from registers, so every element crosses HBM once.  Longer rows
// take a second, cached pass.  Divisions are IEEE fp32 (correctly rounded;
// this file is built without fast-math), so the codes are bit-identical to
// the definition.

#include "device_common.h"
#include "launch.h"

namespace fp8g {

constexpr int QROWS_PER_BLOCK = 4;   // 4 waves of 64 lanes, one row each

__device__ __forceinline__ float quant_div(float x, float s, bool zero_scale) {
    return zero_scale ? x * 0.0f : x / s;   // signed zero for an all-zero scale
}

// cols % 4 == 0 and rows start 16-byte aligned: float4 loads, dword stores.
template <int VPL>
__global__ __launch_bounds__(256) void quantize_rows_vec(const float* __restrict__ x, int64_t rows,
                                                         int64_t cols, uint8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * QROWS_PER_BLOCK + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float4* xr = reinterpret_cast<const float4*>(x + row * cols);
    uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * cols);
    const int64_t nv = cols >> 2;

    if (nv <= 64 * VPL) {
        // single pass: the whole row lives in registers
        float4 v[VPL];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int64_t idx = lane + 64 * i;
            if (idx < nv) {
                v[i] = xr[idx];
            } else {
                v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[i].x), __builtin_fabsf(v[i].y)),
                                                         __builtin_fmaxf(__builtin_fabsf(v[i].z), __builtin_fabsf(v[i].w))));
        }
        amax = wave_max(amax);
        const float s = amax / 448.0f;
        const bool z = (s == 0.0f);
        if (lane == 0) scale[row] = s;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int64_t idx = lane + 64 * i;
            if (idx < nv) {
                qr[idx] = e4m3_pack4(quant_div(v[i].x, s, z), quant_div(v[i].y, s, z),
                                     quant_div(v[i].z, s, z), quant_div(v[i].w, s, z));
            }
        }
        return;
    }

    // two passes for rows longer than the register budget
    float amax = 0.0f;
    for (int64_t idx = lane; idx < nv; idx += 64) {
        const float4 t = xr[idx];
        amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(t.x), __builtin_fabsf(t.y)),
                                                     __builtin_fmaxf(__builtin_fabsf(t.z), __builtin_fabsf(t.w))));
    }
    amax = wave_max(amax);
    const float s = amax / 448.0f;
    const bool z = (s == 0.0f);
    if (lane == 0) scale[row] = s;
    for (int64_t idx = lane; idx < nv; idx += 64) {
        const float4 t = xr[idx];
        qr[idx] = e4m3_pack4(quant_div(t.x, s, z), quant_div(t.y, s, z), quant_div(t.z, s, z),
                             quant_div(t.w, s, z));
    }
}

// Any cols: element-wise loads and byte stores, two passes.
__global__ __launch_bounds__(256) void quantize_rows_scalar(const float* __restrict__ x, int64_t rows,
                                                            int64_t cols, uint8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * QROWS_PER_BLOCK + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float* xr = x + row * cols;
    uint8_t* qr = q + row * cols;
    float amax = 0.0f;
    for (int64_t c = lane; c < cols; c += 64) amax = __builtin_fmaxf(amax, __builtin_fabsf(xr[c]));
    amax = wave_max(amax);
    const float s = amax / 448.0f;
    const bool z = (s == 0.0f);
    if (lane == 0) scale[row] = s;
    for (int64_t c = lane; c < cols; c += 64) qr[c] = e4m3_one(quant_div(xr[c], s, z));
}

hipError_t launch_quantize_rowwise(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* scale,
                                   hipStream_t stream) {
    const int64_t blocks = (rows + QROWS_PER_BLOCK - 1) / QROWS_PER_BLOCK;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks), block(256);
    if (cols % 4 == 0) {
        const int64_t nv = cols / 4;
        if (nv <= 64) quantize_rows_vec<1><<<grid, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 128) quantize_rows_vec<2><<<grid, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 256) quantize_rows_vec<4><<<grid, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 512) quantize_rows_vec<8><<<grid, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 1024) quantize_rows_vec<16><<<grid, block, 0, stream>>>(x, rows, cols, q, scale);
        else quantize_rows_vec<32><<<grid, block, 0, stream>>>(x, rows, cols, q, scale);
    } else {
        quantize_rows_scalar<<<grid, block, 0, stream>>>(x, rows, cols, q, scale);
    }
    return hipGetLastError();
}

}  // namespace fp8g
