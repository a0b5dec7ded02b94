// Internal launchers called by the C ABI after argument checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8g {

hipError_t launch_quantize_rowwise(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* scale,
                                   hipStream_t stream);

// MXFP8 block quantizer (cols % 32 == 0): UE8M0 scale codes [rows, cols / 32]
hipError_t launch_quantize_mx(const float* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* scale,
                              hipStream_t stream);

// mode (a): per-token x per-channel fp32 scales
hipError_t launch_gemm_scaled(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                              const float* sa, const float* sb, void* D, int out_f32, hipStream_t stream);

// mode (b): UE8M0 scales, one per 32 K elements of every row
hipError_t launch_gemm_mx(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                          const uint8_t* ea, const uint8_t* eb, void* D, int out_f32, hipStream_t stream);

}  // namespace fp8g
