// Internal launchers called by the C ABI after argument checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8g {

hipError_t launch_quantize_rowwise(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* scale,
                                   hipStream_t stream);

// row-wise (per_tensor == 0) or per-tensor quantizer on fp32 (in_bf16 == 0) or bf16
// input, to E4M3 (out_e5m2 == 0) or E5M2 codes
hipError_t launch_quantize(const void* x, int in_bf16, int64_t rows, int64_t cols, int per_tensor, int out_e5m2,
                           uint8_t* q, float* scale, hipStream_t stream);

// MXFP8 block quantizer (cols % 32 == 0): UE8M0 scale codes [rows, cols / 32]
hipError_t launch_quantize_mx(const float* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* scale,
                              hipStream_t stream);

// MLA key rows: k [T, H, 192] = k_nope [T, H, 128] ++ k_rope [T, R, 64] (R = 1 or H)
hipError_t launch_concat_mla_k(void* k, const void* k_nope, const void* k_rope, int64_t tokens, int64_t heads,
                               int64_t rope_heads, int elem_bytes, hipStream_t stream);

// mode (a): per-token x per-channel fp32 scales; fmt_a, fmt_b: 0 = E4M3, 1 = E5M2
hipError_t launch_gemm_scaled(int64_t m, int64_t n, int64_t k, const uint8_t* A, int fmt_a, const uint8_t* B,
                              int fmt_b, const float* sa, const float* sb, void* D, int out_f32,
                              hipStream_t stream);

// mode (a), E4M3 operands, with the library's fixed device array as split
// workspace (no allocation); hipErrorOutOfMemory: the device has more CUs
// than the array serves
hipError_t launch_gemm_scaled_noalloc(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                                      const float* sa, const float* sb, void* D, int out_f32, hipStream_t stream);

// mode (b): UE8M0 scales, one per 32 K elements of every row
hipError_t launch_gemm_mx(int64_t m, int64_t n, int64_t k, const uint8_t* A, int fmt_a, const uint8_t* B,
                          int fmt_b, const uint8_t* ea, const uint8_t* eb, void* D, int out_f32,
                          hipStream_t stream);

// the schedule a GEMM launch takes on a device with `cus` CUs (host only):
// tile rows and columns, split count of the split tiles (1: none) and their
// number; hipErrorInvalidValue beyond the 32-bit offset limits
hipError_t schedule_gemm(int64_t m, int64_t n, int64_t k, int mx, int cus, int* tile_m, int* tile_n, int* split,
                         int* split_tiles);

// roof probes: matrix-core rate (blocks x 256 threads, iters rounds of 4
// chains) and streaming bandwidth (bytes read, bytes / write_ratio written)
hipError_t launch_roof_mfma(int64_t blocks, int64_t iters, float* sink, hipStream_t stream);
hipError_t launch_roof_stream(const void* src, int64_t bytes, void* dst, int write_ratio, int nt,
                              hipStream_t stream);

}  // namespace fp8g
