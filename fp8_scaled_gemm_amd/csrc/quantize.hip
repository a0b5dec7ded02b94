// FP8 quantizers with a scale of amax / 448 (E4M3 output) or amax / 57344
// (E5M2 output): one scale per row (per token for activations, per output
// channel for weights), or one per tensor; fp32 or bf16 input.
//
// Scale rule: abs_max / 448, the E4M3 maximum (page "FP8 推理基础设施（五）：
// 从 DeepGEMM 到 vLLM", `_calibrate_scales`, which takes abs_max over a whole
// tensor: the per-tensor mode); one scale per row, as the per-token scale_a /
// per-channel scale_b of the same page's DeepGEMM call (the row-wise mode).
// bf16 input: the precision models are usually deployed in (page on FP8 vLLM
// for AMD Instinct, introduction); a bf16 value converts to fp32 exactly, so
// the result is that of the fp32 quantizer on the converted tensor.  E5M2
// output: the same rule with that format's largest finite value (57344), as
// the page on FlashInfer's concat_mla_k with FP8 inputs takes E5M2 beside E4M3.
//
// HBM-bound: 4 (fp32) or 2 (bf16) bytes read + 1 byte written per element.
// Loads are 16 bytes per lane (4 fp32 or 8 bf16 elements).  Row-wise: rows up
// to 256 loads per wave take one wavefront per row, four rows per workgroup;
// longer rows one 256-thread workgroup per row (amax reduced across its four
// waves through LDS); the row stays in registers between the amax and the
// cast up to 16 loads per lane, longer rows take a second, cached pass.
// Per-tensor: one pass for the amax (one atomic max per workgroup), one for
// the cast.  Loads and stores of streamed data carry the non-temporal hint.
//
// The quotient x / s must be the correctly rounded fp32 division (the codes
// are bit-identical to the definition).  Instead of one IEEE division per
// element it uses y = RN(1/s), computed once per row (tensor), and Markstein's
// correction: q0 = RN(x y), e = x - q0 s (exact, by fma), q = RN(q0 + e y),
// which equals RN(x / s) when y is the correctly rounded reciprocal and no
// intermediate underflows (P. Markstein, "Computation of elementary functions
// on the IBM RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990).  A
// quotient small enough to underflow casts to a signed zero either way (values
// below 2^-10 round to zero in E4M3, below 2^-17 in E5M2), and scales below
// the smallest normal fp32 (where 1/s may overflow) use the IEEE division.
// This file is built without fast-math.

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace fp8g {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int QROWS_PER_BLOCK = 4;          // per-wave kernel: 4 waves of 64 lanes, one row each
constexpr float FLT_MIN_NORMAL = 1.17549435e-38f;

// ---- output formats: the largest finite magnitude (the divisor of amax) and
// the saturating round-to-nearest-even cast of four values into one dword
struct OutE4M3 {
    static constexpr float MAX = 448.0f;
    __device__ __forceinline__ static uint32_t pack4(float a, float b, float c, float d) {
        return e4m3_pack4(a, b, c, d);
    }
};

struct OutE5M2 {
    static constexpr float MAX = 57344.0f;
    __device__ __forceinline__ static uint32_t pack4(float a, float b, float c, float d) {
        return e5m2_pack4(a, b, c, d);
    }
};

template <class O>
__device__ __forceinline__ uint8_t cast_one(float a) {
    return (uint8_t)(O::pack4(a, 0.0f, 0.0f, 0.0f) & 0xFFu);
}

// Per-row (per-tensor) divisor: the scale, its correctly rounded reciprocal, the path.
struct RowDiv {
    float s, y;
    bool zero;    // s == 0: signed zeros
    bool ieee;    // s below the smallest normal: plain IEEE division
};

// amax is the same in every lane; readfirstlane makes that visible to the
// compiler, so the path is chosen once with a scalar branch.
template <class O>
__device__ __forceinline__ RowDiv row_div(float amax) {
    amax = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, amax)));
    RowDiv d;
    d.s = amax / O::MAX;
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

// f(path_tag) with the path as a compile-time constant
template <typename F>
__device__ __forceinline__ void by_path(const RowDiv& d, F&& f) {
    if (d.zero) f(std::integral_constant<int, 2>{});
    else if (d.ieee) f(std::integral_constant<int, 1>{});
    else f(std::integral_constant<int, 0>{});
}

__device__ __forceinline__ float amax2(float a, float b) { return __builtin_fmaxf(__builtin_fabsf(a), __builtin_fabsf(b)); }

// ---- input vectors: 16 bytes of input = EPL elements -> EPL bytes of codes.
struct InF32 {
    static constexpr int EPL = 4;
    v4f v;
    __device__ __forceinline__ void load_nt(const void* base, int64_t idx) {
        v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(base) + idx);
    }
    __device__ __forceinline__ void load(const void* base, int64_t idx) { v = reinterpret_cast<const v4f*>(base)[idx]; }
    __device__ __forceinline__ void zero() { v = (v4f){0.f, 0.f, 0.f, 0.f}; }
    __device__ __forceinline__ float amax() const { return __builtin_fmaxf(amax2(v.x, v.y), amax2(v.z, v.w)); }
    template <class O, int P>
    __device__ __forceinline__ void store(uint8_t* q, int64_t idx, const RowDiv& d) const {
        const uint32_t w = O::pack4(quot<P>(v.x, d), quot<P>(v.y, d), quot<P>(v.z, d), quot<P>(v.w, d));
        __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(q) + idx);
    }
    __device__ __forceinline__ static float scalar(const void* base, int64_t i) {
        return reinterpret_cast<const float*>(base)[i];
    }
};

struct InBF16 {
    static constexpr int EPL = 8;
    v4u r;   // element 2i in the low half of dword i
    __device__ __forceinline__ static float lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
    __device__ __forceinline__ static float hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
    __device__ __forceinline__ void load_nt(const void* base, int64_t idx) {
        r = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(base) + idx);
    }
    __device__ __forceinline__ void load(const void* base, int64_t idx) { r = reinterpret_cast<const v4u*>(base)[idx]; }
    __device__ __forceinline__ void zero() { r = (v4u){0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ float amax() const {
        const uint32_t a = r.x, b = r.y, c = r.z, e = r.w;   // scalar copies of the dwords
        return __builtin_fmaxf(__builtin_fmaxf(amax2(lo(a), hi(a)), amax2(lo(b), hi(b))),
                               __builtin_fmaxf(amax2(lo(c), hi(c)), amax2(lo(e), hi(e))));
    }
    template <class O, int P>
    __device__ __forceinline__ void store(uint8_t* q, int64_t idx, const RowDiv& d) const {
        const uint32_t a = r.x, b = r.y, c = r.z, e = r.w;
        const v2u w = {O::pack4(quot<P>(lo(a), d), quot<P>(hi(a), d), quot<P>(lo(b), d), quot<P>(hi(b), d)),
                       O::pack4(quot<P>(lo(c), d), quot<P>(hi(c), d), quot<P>(lo(e), d), quot<P>(hi(e), d))};
        __builtin_nontemporal_store(w, reinterpret_cast<v2u*>(q) + idx);
    }
    __device__ __forceinline__ static float scalar(const void* base, int64_t i) {
        return __builtin_bit_cast(float, (uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
    }
};

template <class V>
__device__ __forceinline__ const uint8_t* row_base(const void* x, int64_t row, int64_t cols) {
    return reinterpret_cast<const uint8_t*>(x) + row * cols * (int64_t)(16 / V::EPL);
}

// cols % EPL == 0, rows 16-byte aligned, cols <= 64 * VPL * EPL: one wave per row.
template <class V, class O, int VPL>
__global__ __launch_bounds__(256) void quantize_rows_wave(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                          uint8_t* __restrict__ q, float* __restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * QROWS_PER_BLOCK + (threadIdx.x >> 6);
    if (row >= rows) return;
    const uint8_t* xr = row_base<V>(x, row, cols);
    uint8_t* qr = q + row * cols;
    const int64_t nv = cols / V::EPL;
    V v[VPL];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int64_t idx = lane + 64 * i;
        if (idx < nv) v[i].load_nt(xr, idx); else v[i].zero();
        amax = __builtin_fmaxf(amax, v[i].amax());
    }
    const RowDiv d = row_div<O>(wave_max(amax));
    if (lane == 0) scale[row] = d.s;
    by_path(d, [&](auto path) {
        constexpr int P = decltype(path)::value;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int64_t idx = lane + 64 * i;
            if (idx < nv) v[i].template store<O, P>(qr, idx, d);
        }
    });
}

__device__ __forceinline__ float block_max(float v, float* red) {
    const int tid = threadIdx.x;
    v = wave_max(v);
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    return __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
}

// cols % EPL == 0, rows 16-byte aligned: one 256-thread workgroup per row.
// VPL > 0: the row (cols <= 256 * VPL * EPL) lives in registers; VPL == 0:
// two passes over the row (the second one mostly from cache).
template <class V, class O, int VPL>
__global__ __launch_bounds__(256) void quantize_rows_wg(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                        uint8_t* __restrict__ q, float* __restrict__ scale) {
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const uint8_t* xr = row_base<V>(x, row, cols);
    uint8_t* qr = q + row * cols;
    const int64_t nv = cols / V::EPL;
    constexpr int NR = VPL > 0 ? VPL : 1;
    V v[NR];
    float amax = 0.0f;
    if constexpr (VPL > 0) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int64_t idx = tid + 256 * i;
            if (idx < nv) v[i].load_nt(xr, idx); else v[i].zero();
            amax = __builtin_fmaxf(amax, v[i].amax());
        }
    } else {
        for (int64_t idx = tid; idx < nv; idx += 256) {
            v[0].load(xr, idx);
            amax = __builtin_fmaxf(amax, v[0].amax());
        }
    }
    const RowDiv d = row_div<O>(block_max(amax, red));
    if (tid == 0) scale[row] = d.s;
    by_path(d, [&](auto path) {
        constexpr int P = decltype(path)::value;
        if constexpr (VPL > 0) {
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int64_t idx = tid + 256 * i;
                if (idx < nv) v[i].template store<O, P>(qr, idx, d);
            }
        } else {
            for (int64_t idx = tid; idx < nv; idx += 256) {
                V t;
                t.load(xr, idx);
                t.template store<O, P>(qr, idx, d);
            }
        }
    });
}

// Any cols: element-wise loads and byte stores, two passes, one wave per row.
template <class V, class O>
__global__ __launch_bounds__(256) void quantize_rows_scalar(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                            uint8_t* __restrict__ q, float* __restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * QROWS_PER_BLOCK + (threadIdx.x >> 6);
    if (row >= rows) return;
    uint8_t* qr = q + row * cols;
    float amax = 0.0f;
    for (int64_t c = lane; c < cols; c += 64) amax = __builtin_fmaxf(amax, __builtin_fabsf(V::scalar(x, row * cols + c)));
    const RowDiv d = row_div<O>(wave_max(amax));
    if (lane == 0) scale[row] = d.s;
    by_path(d, [&](auto path) {
        constexpr int P = decltype(path)::value;
        for (int64_t c = lane; c < cols; c += 64) qr[c] = cast_one<O>(quot<P>(V::scalar(x, row * cols + c), d));
    });
}

// ---- per tensor: n elements as one row.  The scale slot first holds the bits
// of amax (non-negative floats order like their bit patterns, so an unsigned
// atomic max finds it), then amax / MAX.
constexpr int TQ_UNROLL = 4;

__global__ void tensor_scale_clear(float* __restrict__ scale) {
    if (threadIdx.x == 0) scale[0] = 0.0f;
}

template <class V>
__global__ __launch_bounds__(256) void tensor_amax(const void* __restrict__ x, int64_t n, float* __restrict__ slot) {
    __shared__ float red[4];
    const int64_t nv = n / V::EPL;
    const int64_t step = (int64_t)gridDim.x * 256 * TQ_UNROLL;
    float amax = 0.0f;
    for (int64_t base = (int64_t)blockIdx.x * 256 * TQ_UNROLL; base < nv; base += step) {
        V v[TQ_UNROLL];
#pragma unroll
        for (int u = 0; u < TQ_UNROLL; ++u) {
            const int64_t idx = base + u * 256 + threadIdx.x;
            if (idx < nv) v[u].load(x, idx); else v[u].zero();
        }
#pragma unroll
        for (int u = 0; u < TQ_UNROLL; ++u) amax = __builtin_fmaxf(amax, v[u].amax());
    }
    if (blockIdx.x == 0)   // the elements past the last whole vector
        for (int64_t i = nv * V::EPL + threadIdx.x; i < n; i += 256) amax = __builtin_fmaxf(amax, __builtin_fabsf(V::scalar(x, i)));
    amax = block_max(amax, red);
    if (threadIdx.x == 0)
        __hip_atomic_fetch_max(reinterpret_cast<unsigned int*>(slot), __builtin_bit_cast(unsigned int, amax),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class V, class O>
__global__ __launch_bounds__(256) void tensor_quant(const void* __restrict__ x, int64_t n, uint8_t* __restrict__ q,
                                                    const float* __restrict__ slot) {
    const RowDiv d = row_div<O>(slot[0]);   // the slot holds amax here
    const int64_t nv = n / V::EPL;
    const int64_t step = (int64_t)gridDim.x * 256 * TQ_UNROLL;
    by_path(d, [&](auto path) {
        constexpr int P = decltype(path)::value;
        for (int64_t base = (int64_t)blockIdx.x * 256 * TQ_UNROLL; base < nv; base += step) {
            V v[TQ_UNROLL];
#pragma unroll
            for (int u = 0; u < TQ_UNROLL; ++u) {
                const int64_t idx = base + u * 256 + threadIdx.x;
                if (idx < nv) v[u].load_nt(x, idx); else v[u].zero();
            }
#pragma unroll
            for (int u = 0; u < TQ_UNROLL; ++u) {
                const int64_t idx = base + u * 256 + threadIdx.x;
                if (idx < nv) v[u].template store<O, P>(q, idx, d);
            }
        }
        if (blockIdx.x == 0)
            for (int64_t i = nv * V::EPL + threadIdx.x; i < n; i += 256) q[i] = cast_one<O>(quot<P>(V::scalar(x, i), d));
    });
}

template <class O>
__global__ void tensor_scale_finish(float* __restrict__ scale) {
    if (threadIdx.x == 0) scale[0] = scale[0] / O::MAX;   // amax -> amax / MAX, as each workgroup computed it
}

// ---- launchers
template <class V, class O>
static hipError_t launch_rows(const void* x, int64_t rows, int64_t cols, uint8_t* q, float* scale, hipStream_t stream) {
    const dim3 block(256);
    const int64_t wave_blocks = (rows + QROWS_PER_BLOCK - 1) / QROWS_PER_BLOCK;
    if (rows > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 gw((unsigned)wave_blocks), gr((unsigned)rows);
    if (cols % V::EPL == 0) {
        const int64_t nv = cols / V::EPL;   // 16-byte loads per row
        if (nv <= 64) quantize_rows_wave<V, O, 1><<<gw, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 128) quantize_rows_wave<V, O, 2><<<gw, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 256) quantize_rows_wave<V, O, 4><<<gw, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 512) quantize_rows_wg<V, O, 2><<<gr, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 1024) quantize_rows_wg<V, O, 4><<<gr, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 2048) quantize_rows_wg<V, O, 8><<<gr, block, 0, stream>>>(x, rows, cols, q, scale);
        else if (nv <= 4096) quantize_rows_wg<V, O, 16><<<gr, block, 0, stream>>>(x, rows, cols, q, scale);
        else quantize_rows_wg<V, O, 0><<<gr, block, 0, stream>>>(x, rows, cols, q, scale);
    } else {
        quantize_rows_scalar<V, O><<<gw, block, 0, stream>>>(x, rows, cols, q, scale);
    }
    return hipGetLastError();
}

template <class V, class O>
static hipError_t launch_tensor(const void* x, int64_t n, uint8_t* q, float* scale, hipStream_t stream) {
    const int64_t nv = n / V::EPL;
    int64_t blocks = (nv + 256 * TQ_UNROLL - 1) / (256 * TQ_UNROLL);
    if (blocks < 1) blocks = 1;
    if (blocks > 2048) blocks = 2048;   // grid-stride beyond: 8 workgroups per CU
    const dim3 grid((unsigned)blocks), block(256);
    tensor_scale_clear<<<1, 64, 0, stream>>>(scale);
    tensor_amax<V><<<grid, block, 0, stream>>>(x, n, scale);
    tensor_quant<V, O><<<grid, block, 0, stream>>>(x, n, q, scale);
    tensor_scale_finish<O><<<1, 64, 0, stream>>>(scale);
    return hipGetLastError();
}

template <class O>
static hipError_t launch_fmt(const void* x, int in_bf16, int64_t rows, int64_t cols, int per_tensor, uint8_t* q,
                             float* scale, hipStream_t stream) {
    if (per_tensor)
        return in_bf16 ? launch_tensor<InBF16, O>(x, rows * cols, q, scale, stream)
                       : launch_tensor<InF32, O>(x, rows * cols, q, scale, stream);
    return in_bf16 ? launch_rows<InBF16, O>(x, rows, cols, q, scale, stream)
                   : launch_rows<InF32, O>(x, rows, cols, q, scale, stream);
}

hipError_t launch_quantize_rowwise(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* scale,
                                   hipStream_t stream) {
    return launch_rows<InF32, OutE4M3>(x, rows, cols, q, scale, stream);
}

hipError_t launch_quantize(const void* x, int in_bf16, int64_t rows, int64_t cols, int per_tensor, int out_e5m2,
                           uint8_t* q, float* scale, hipStream_t stream) {
    return out_e5m2 ? launch_fmt<OutE5M2>(x, in_bf16, rows, cols, per_tensor, q, scale, stream)
                    : launch_fmt<OutE4M3>(x, in_bf16, rows, cols, per_tensor, q, scale, stream);
}

}  // namespace fp8g
