// Roof probes: the matrix-core rate and the streaming bandwidth this part
// reaches at the moment they run, measured beside the hot path so that its
// kernels can be judged against what the chip delivers at the same clock and
// power state, not only against the nominal peaks (the page on FP8 inference
// of a 7B model on an RTX 4060, section 4.1, checks core utilisation and
// memory bandwidth).
//
// roof_mfma_kernel: every wave runs `iters` rounds of four independent chains
// of V_MFMA_SCALE_F32_32X32X64_F8F6F4 (the GEMMs' instruction, neutral
// scales), no memory traffic: 4 * 131072 flops per wave and round.
// roof_stream_kernel: a stream of 16-byte vectors, 16 bytes read and 16
// (copy) or 4 (the fp32 quantizer's 4:1 read/write mix) written per lane and
// vector, non-temporal loads and write-back or non-temporal stores (which of
// the two is faster depends on whether the output stays in the infinity
// cache), each workgroup one contiguous 32 KB chunk with all of a lane's 8
// loads in flight before its stores.

#include "launch.h"

namespace fp8g {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void roof_mfma_kernel(int iters, int seed, float* __restrict__ sink) {
    const int t = (int)threadIdx.x + seed;
    const v8i x = {t, t + 1, t + 2, t + 3, t + 4, t + 5, t + 6, t + 7};
    const v8i y = {seed, t, 3 * t, 5, t ^ 9, 11, 13, 2 * t};
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c0, 0, 0, 0, 127, 0, 127);
        c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(y, x, c1, 0, 0, 0, 127, 0, 127);
        c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, x, c2, 0, 0, 0, 127, 0, 127);
        c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(y, y, c3, 0, 0, 0, 127, 0, 127);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
    if (s == -1.0f) sink[0] = s;   // keeps the chains live; practically never taken
}

template <int WR, bool NT>
__global__ __launch_bounds__(256) void roof_stream_kernel(const v4u* __restrict__ src, int64_t n,
                                                          void* __restrict__ dst) {
    // each workgroup one contiguous chunk of 256 * U vectors, all U loads of a
    // lane in flight before its stores (as the row-wise quantizer keeps a
    // row); whole chunks without per-lane range checks
    constexpr int U = 8;
    const int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x;
    const bool whole = (int64_t)(blockIdx.x + 1) * 256 * U <= n;   // uniform
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * 256;
        v[u] = (whole || i < n) ? __builtin_nontemporal_load(src + i) : (v4u){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * 256;
        if (whole || i < n) {
            if constexpr (WR == 16) {
                if constexpr (NT) __builtin_nontemporal_store(v[u], reinterpret_cast<v4u*>(dst) + i);
                else reinterpret_cast<v4u*>(dst)[i] = v[u];
            } else {
                const unsigned int w = v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
                if constexpr (NT) __builtin_nontemporal_store(w, reinterpret_cast<unsigned int*>(dst) + i);
                else reinterpret_cast<unsigned int*>(dst)[i] = w;
            }
        }
    }
}

hipError_t launch_roof_mfma(int64_t blocks, int64_t iters, float* sink, hipStream_t stream) {
    roof_mfma_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>((int)iters, 3, sink);
    return hipGetLastError();
}

hipError_t launch_roof_stream(const void* src, int64_t bytes, void* dst, int write_ratio, int nt, hipStream_t stream) {
    const int64_t n = bytes / 16;
    if (n == 0) return hipSuccess;
    const int64_t grid = (n + 256 * 8 - 1) / (256 * 8);
    if (grid >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const v4u* s = reinterpret_cast<const v4u*>(src);
    const dim3 g((unsigned)grid), b(256);
    if (write_ratio == 1) {
        if (nt) roof_stream_kernel<16, true><<<g, b, 0, stream>>>(s, n, dst);
        else roof_stream_kernel<16, false><<<g, b, 0, stream>>>(s, n, dst);
    } else {
        if (nt) roof_stream_kernel<4, true><<<g, b, 0, stream>>>(s, n, dst);
        else roof_stream_kernel<4, false><<<g, b, 0, stream>>>(s, n, dst);
    }
    return hipGetLastError();
}

}  // namespace fp8g
