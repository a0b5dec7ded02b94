// Row-wise E4M3 quantizer: s[r] = amax_r / 448, q = E4M3_RNE_SAT(x / s[r]).
//
// Scale rule: abs_max / 448 (page "FP8 推理基础设施（五）：从 DeepGEMM 到
// vLLM", `_calibrate_scales`), one scale per row (per token for activations,
// per output channel for weights, as the DeepGEMM call's scale_a / scale_b on
// the same page).
//
// HBM-bound: 4 bytes read + 1 byte written per element, each crossing HBM once
// (the row is held in registers between the amax and the cast; loads and
// stores carry the non-temporal hint, since nothing is reused).  Rows up to
// 1024 columns: one wavefront per row, four rows per workgroup.  Longer rows:
// one 256-thread workgroup per row, amax reduced across its four waves through
// LDS; rows beyond 16384 columns take a second, cached pass.
//
// The quotient x / s must be the correctly rounded fp32 division (the codes
// are bit-identical to the definition).  Instead of one IEEE division per
// element it uses y = RN(1/s), computed once per row, and Markstein's
// correction: q0 = RN(x y), e = x - q0 s (exact, by fma), q = RN(q0 + e y),
// which equals RN(x / s) when y is the correctly rounded reciprocal and no
// intermediate underflows (P. Markstein, "Computation of elementary functions
// on the IBM RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990).  A
// quotient small enough to underflow casts to a signed zero either way (E4M3
// codes below 2^-10 round to zero), and rows whose scale is below the
// smallest normal fp32 (where 1/s may overflow) use the IEEE division.  This
// file is built without fast-math.

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace fp8g {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int QROWS_PER_BLOCK = 4;          // per-wave kernel: 4 waves of 64 lanes, one row each
constexpr float FLT_MIN_NORMAL = 1.17549435e-38f;

// Per-row divisor: the scale, its correctly rounded reciprocal, and the path.
struct RowDiv {
    float s, y;
    bool zero;    // s == 0: signed zeros
    bool ieee;    // s below the smallest normal: plain IEEE division
};

// amax is the same in every lane; readfirstlane makes that visible to the
// compiler, so the path is chosen once per row with a scalar branch.
__device__ __forceinline__ RowDiv row_div(float amax) {
    amax = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, amax)));
    RowDiv d;
    d.s = amax / 448.0f;
    d.y = 1.0f / d.s;
    d.zero = (d.s == 0.0f);
    d.ieee = (d.s < FLT_MIN_NORMAL);
    return d;
}

// PATH 0: Markstein quotient; 1: IEEE division; 2: signed zero (s == 0)
template <int PATH>
__device__ __forceinline__ float quot(float x, const RowDiv& d) {
    if constexpr (PATH == 2) {
        return x * 0.0f;
    } else if constexpr (PATH == 1) {
        return x / d.s;
    } else {
        const float q0 = x * d.y;
        const float e = __builtin_fmaf(-q0, d.s, x);
        // x = -0 gives e = +0 and q0 + e y = +0; the quotient has x's sign (s > 0)
        return __builtin_copysignf(__builtin_fmaf(e, d.y, q0), x);
    }
}

template <int PATH>
__device__ __forceinline__ uint32_t quant4(const v4f& v, const RowDiv& d) {
    return e4m3_pack4(quot<PATH>(v.x, d), quot<PATH>(v.y, d), quot<PATH>(v.z, d), quot<PATH>(v.w, d));
}

// f(path_tag) with the row's path as a compile-time constant
template <typename F>
__device__ __forceinline__ void by_path(const RowDiv& d, F&& f) {
    if (d.zero) f(std::integral_constant<int, 2>{});
    else if (d.ieee) f(std::integral_constant<int, 1>{});
    else f(std::integral_constant<int, 0>{});
}

__device__ __forceinline__ float amax4(const v4f& v) {
    return __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v.x), __builtin_fabsf(v.y)),
                           __builtin_fmaxf(__builtin_fabsf(v.z), __builtin_fabsf(v.w)));
}

// cols % 4 == 0, rows 16-byte aligned, cols <= 256 * VPL: one wave per row.
template <int VPL>
__global__ __launch_bounds__(256) void quantize_rows_wave(const float* __restrict__ x, int64_t rows, int64_t cols,
                                                          uint8_t* __restrict__ q, float* __restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * QROWS_PER_BLOCK + (threadIdx.x >> 6);
    if (row >= rows) return;
    const v4f* xr = reinterpret_cast<const v4f*>(x + row * cols);
    uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * cols);
    const int64_t nv = cols >> 2;
    v4f v[VPL];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int64_t idx = lane + 64 * i;
        v[i] = idx < nv ? __builtin_nontemporal_load(xr + idx) : (v4f){0.f, 0.f, 0.f, 0.f};
        amax = __builtin_fmaxf(amax, amax4(v[i]));
    }
    const RowDiv d = row_div(wave_max(amax));
    if (lane == 0) scale[row] = d.s;
    by_path(d, [&](auto path) {
        constexpr int P = decltype(path)::value;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int64_t idx = lane + 64 * i;
            if (idx < nv) __builtin_nontemporal_store(quant4<P>(v[i], d), qr + idx);
        }
    });
}

// cols % 4 == 0, rows 16-byte aligned: one 256-thread workgroup per row.
// VPL > 0: the row (cols <= 1024 * VPL) lives in registers; VPL == 0: two
// passes over the row (the second one mostly from cache).
template <int VPL>
__global__ __launch_bounds__(256) void quantize_rows_wg(const float* __restrict__ x, int64_t rows, int64_t cols,
                                                        uint8_t* __restrict__ q, float* __restrict__ scale) {
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t row = blockIdx.x;
    const v4f* xr = reinterpret_cast<const v4f*>(x + row * cols);
    uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * cols);
    const int64_t nv = cols >> 2;
    constexpr int NR = VPL > 0 ? VPL : 1;
    v4f v[NR];
    float amax = 0.0f;
    if constexpr (VPL > 0) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int64_t idx = tid + 256 * i;
            v[i] = idx < nv ? __builtin_nontemporal_load(xr + idx) : (v4f){0.f, 0.f, 0.f, 0.f};
            amax = __builtin_fmaxf(amax, amax4(v[i]));
        }
    } else {
        for (int64_t idx = tid; idx < nv; idx += 256) amax = __builtin_fmaxf(amax, amax4(xr[idx]));
    }
    amax = wave_max(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    const RowDiv d = row_div(__builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3])));
    if (tid == 0) scale[row] = d.s;
    by_path(d, [&](auto path) {
        constexpr int P = decltype(path)::value;
        if constexpr (VPL > 0) {
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int64_t idx = tid + 256 * i;
                if (idx < nv) __builtin_nontemporal_store(quant4<P>(v[i], d), qr + idx);
            }
        } else {
            for (int64_t idx = tid; idx < nv; idx += 256) __builtin_nontemporal_store(quant4<P>(xr[idx], d), qr + idx);
        }
    });
}

// Any cols: element-wise loads and byte stores, two passes, one wave per row.
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
    const RowDiv d = row_div(wave_max(amax));
    if (lane == 0) scale[row] = d.s;
    by_path(d, [&](auto path) {
        constexpr int P = decltype(path)::value;
        for (int64_t c = lane; c < cols; c += 64) qr[c] = e4m3_one(quot<P>(xr[c], d));
    });
}

hipError_t launch_quantize_rowwise(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* scale,
                                   hipStream_t stream) {
    const dim3 block(256);
    const int64_t wave_blocks = (rows + QROWS_PER_BLOCK - 1) / QROWS_PER_BLOCK;
    if (rows > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 gw((unsigned)wave_blocks), gr((unsigned)rows);
    if (cols % 4 == 0) {
        const int64_t nv = cols / 4;
        if (nv <= 64) quantize_rows_wave<1><<<gw, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 128) quantize_rows_wave<2><<<gw, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 256) quantize_rows_wave<4><<<gw, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 512) quantize_rows_wg<2><<<gr, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 1024) quantize_rows_wg<4><<<gr, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 2048) quantize_rows_wg<8><<<gr, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 4096) quantize_rows_wg<16><<<gr, block, 0, stream>>>(x, rows, cols, q, scale);
        else quantize_rows_wg<0><<<gr, block, 0, stream>>>(x, rows, cols, q, scale);
    } else {
        quantize_rows_scalar<<<gw, block, 0, stream>>>(x, rows, cols, q, scale);
    }
    return hipGetLastError();
}

}  // namespace fp8g
