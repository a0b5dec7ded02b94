// C ABI of fp8g: host-side argument checks, then one kernel launch on the
// caller's stream.  Every check runs before any HIP call, so a rejected call
// queues nothing and touches no device.

#include "fp8g.h"

#include <stdint.h>

#include "launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

// a * b * c, or -1 on overflow past 2^62
int64_t mul3(int64_t a, int64_t b, int64_t c) {
    const int64_t lim = (int64_t)1 << 62;
    if (a == 0 || b == 0 || c == 0) return 0;
    if (a > lim / b) return -1;
    const int64_t ab = a * b;
    if (ab > lim / c) return -1;
    return ab * c;
}

constexpr int64_t GEMM_K_LIMIT = (int64_t)1 << 23;
constexpr int64_t ROWS_LIMIT = (int64_t)1 << 31;   // the row-wise quantizers launch one workgroup (wave) per row

int check_gemm_common(int64_t m, int64_t n, int64_t k, const void* A, const void* B, const void* sa,
                      const void* sb, int64_t sa_bytes, int64_t sb_bytes, const void* D, int out_dtype) {
    if (m < 0 || n < 0 || k < 0) return FP8G_ERR_SHAPE;
    if (out_dtype != FP8G_OUT_BF16 && out_dtype != FP8G_OUT_F32) return FP8G_ERR_DTYPE;
    if (m == 0 || n == 0) return FP8G_OK;  // nothing to write
    const int64_t esz = out_dtype == FP8G_OUT_F32 ? 4 : 2;
    const int64_t a_bytes = mul3(m, k, 1), b_bytes = mul3(n, k, 1), d_bytes = mul3(m, n, esz);
    if (a_bytes < 0 || b_bytes < 0 || d_bytes < 0) return FP8G_ERR_UNSUPPORTED;
    // the kernels address a 256-row panel of A, B (k bytes per row) or D (n
    // elements per row) with 32-bit offsets below 2^31
    if (k >= GEMM_K_LIMIT || m >= ((int64_t)1 << 31) || n > (((int64_t)1 << 31) / (256 * esz)))
        return FP8G_ERR_UNSUPPORTED;
    if (!D) return FP8G_ERR_NULL;
    if (k > 0 && (!A || !B)) return FP8G_ERR_NULL;
    if (sa_bytes > 0 && !sa) return FP8G_ERR_NULL;
    if (sb_bytes > 0 && !sb) return FP8G_ERR_NULL;
    if (!aligned16(D) || (A && !aligned16(A)) || (B && !aligned16(B)) || (sa && !aligned16(sa)) ||
        (sb && !aligned16(sb)))
        return FP8G_ERR_ALIGN;
    const Range d = range_of(D, d_bytes);
    if (overlaps(d, range_of(A, a_bytes)) || overlaps(d, range_of(B, b_bytes)) ||
        overlaps(d, range_of(sa, sa_bytes)) || overlaps(d, range_of(sb, sb_bytes)))
        return FP8G_ERR_OVERLAP;
    return -1;  // go on
}

bool valid_fmt(int f) { return f == FP8G_FMT_E4M3 || f == FP8G_FMT_E5M2; }

int hip_status(hipError_t e) { return e == hipSuccess ? FP8G_OK : FP8G_ERR_HIP; }

}  // namespace

extern "C" {

int fp8_quantize_rowwise(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* scale,
                         hipStream_t stream) {
    if (rows < 0 || cols < 0) return FP8G_ERR_SHAPE;
    if (rows == 0) return FP8G_OK;
    const int64_t n = mul3(rows, cols, 1);
    if (n < 0 || n > ((int64_t)1 << 60) || rows >= ROWS_LIMIT) return FP8G_ERR_UNSUPPORTED;
    if (!scale) return FP8G_ERR_NULL;
    if (n > 0 && (!x || !q)) return FP8G_ERR_NULL;
    if (!aligned16(scale) || (x && !aligned16(x)) || (q && !aligned16(q))) return FP8G_ERR_ALIGN;
    const Range rx = range_of(x, n * 4), rq = range_of(q, n), rs = range_of(scale, rows * 4);
    if (overlaps(rq, rx) || overlaps(rs, rx) || overlaps(rq, rs)) return FP8G_ERR_OVERLAP;
    return hip_status(fp8g::launch_quantize_rowwise(x, rows, cols, q, scale, stream));
}

int fp8_quantize_ex(const void* x, int in_dtype, int64_t rows, int64_t cols, int granularity, int out_fmt,
                    uint8_t* q, float* scale, hipStream_t stream) {
    if (rows < 0 || cols < 0) return FP8G_ERR_SHAPE;
    if (in_dtype != FP8G_IN_F32 && in_dtype != FP8G_IN_BF16) return FP8G_ERR_DTYPE;
    if (granularity != FP8G_SCALE_PER_ROW && granularity != FP8G_SCALE_PER_TENSOR) return FP8G_ERR_DTYPE;
    if (!valid_fmt(out_fmt)) return FP8G_ERR_DTYPE;
    const bool per_tensor = granularity == FP8G_SCALE_PER_TENSOR;
    if (!per_tensor && rows == 0) return FP8G_OK;
    const int64_t n = mul3(rows, cols, 1);
    if (n < 0 || n > ((int64_t)1 << 60) || (!per_tensor && rows >= ROWS_LIMIT)) return FP8G_ERR_UNSUPPORTED;
    if (!scale) return FP8G_ERR_NULL;
    if (n > 0 && (!x || !q)) return FP8G_ERR_NULL;
    if (!aligned16(scale) || (x && !aligned16(x)) || (q && !aligned16(q))) return FP8G_ERR_ALIGN;
    const int64_t esz = in_dtype == FP8G_IN_BF16 ? 2 : 4;
    const Range rx = range_of(x, n * esz), rq = range_of(q, n), rs = range_of(scale, per_tensor ? 4 : rows * 4);
    if (overlaps(rq, rx) || overlaps(rs, rx) || overlaps(rq, rs)) return FP8G_ERR_OVERLAP;
    return hip_status(fp8g::launch_quantize(x, in_dtype == FP8G_IN_BF16, rows, cols, per_tensor,
                                            out_fmt == FP8G_FMT_E5M2, q, scale, stream));
}

int mxfp8_quantize(const float* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* scale, hipStream_t stream) {
    if (rows < 0 || cols < 0 || cols % 32 != 0) return FP8G_ERR_SHAPE;
    const int64_t n = mul3(rows, cols, 1);
    if (n < 0 || n > ((int64_t)1 << 60)) return FP8G_ERR_UNSUPPORTED;
    if (n == 0) return FP8G_OK;
    if (!x || !q || !scale) return FP8G_ERR_NULL;
    if (!aligned16(x) || !aligned16(q) || !aligned16(scale)) return FP8G_ERR_ALIGN;
    const Range rx = range_of(x, n * 4), rq = range_of(q, n), rs = range_of(scale, n / 32);
    if (overlaps(rq, rx) || overlaps(rs, rx) || overlaps(rq, rs)) return FP8G_ERR_OVERLAP;
    return hip_status(fp8g::launch_quantize_mx(x, rows, cols, q, scale, stream));
}

int fp8_gemm_scaled_ex(int64_t m, int64_t n, int64_t k, const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b,
                       const float* scale_a, const float* scale_b, void* D, int out_dtype, hipStream_t stream) {
    if (m < 0 || n < 0 || k < 0) return FP8G_ERR_SHAPE;
    if (!valid_fmt(fmt_a) || !valid_fmt(fmt_b)) return FP8G_ERR_DTYPE;
    const int st = check_gemm_common(m, n, k, A, B, scale_a, scale_b, m * 4, n * 4, D, out_dtype);
    if (st >= 0) return st;
    if (k % 16 != 0) return FP8G_ERR_UNSUPPORTED;
    return hip_status(fp8g::launch_gemm_scaled(m, n, k, A, fmt_a, B, fmt_b, scale_a, scale_b, D,
                                               out_dtype == FP8G_OUT_F32, stream));
}

int fp8_gemm_scaled(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B, const float* scale_a,
                    const float* scale_b, void* D, int out_dtype, hipStream_t stream) {
    return fp8_gemm_scaled_ex(m, n, k, A, FP8G_FMT_E4M3, B, FP8G_FMT_E4M3, scale_a, scale_b, D, out_dtype, stream);
}

int fp8_gemm_scaled_noalloc(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                            const float* scale_a, const float* scale_b, void* D, int out_dtype, hipStream_t stream) {
    if (m < 0 || n < 0 || k < 0) return FP8G_ERR_SHAPE;
    const int st = check_gemm_common(m, n, k, A, B, scale_a, scale_b, m * 4, n * 4, D, out_dtype);
    if (st >= 0) return st;
    if (k % 16 != 0) return FP8G_ERR_UNSUPPORTED;
    const hipError_t e = fp8g::launch_gemm_scaled_noalloc(m, n, k, A, B, scale_a, scale_b, D,
                                                          out_dtype == FP8G_OUT_F32, stream);
    return e == hipErrorOutOfMemory ? FP8G_ERR_UNSUPPORTED : hip_status(e);
}

int mxfp8_gemm_ex(int64_t m, int64_t n, int64_t k, const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b,
                  const uint8_t* scale_a, const uint8_t* scale_b, void* D, int out_dtype, hipStream_t stream) {
    if (m < 0 || n < 0 || k < 0 || k % 32 != 0) return FP8G_ERR_SHAPE;
    if (!valid_fmt(fmt_a) || !valid_fmt(fmt_b)) return FP8G_ERR_DTYPE;
    const int st = check_gemm_common(m, n, k, A, B, scale_a, scale_b, m * (k / 32), n * (k / 32), D, out_dtype);
    if (st >= 0) return st;
    return hip_status(fp8g::launch_gemm_mx(m, n, k, A, fmt_a, B, fmt_b, scale_a, scale_b, D,
                                           out_dtype == FP8G_OUT_F32, stream));
}

int mxfp8_gemm(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B, const uint8_t* scale_a,
               const uint8_t* scale_b, void* D, int out_dtype, hipStream_t stream) {
    return mxfp8_gemm_ex(m, n, k, A, FP8G_FMT_E4M3, B, FP8G_FMT_E4M3, scale_a, scale_b, D, out_dtype, stream);
}

int concat_mla_k(void* k, const void* k_nope, const void* k_rope, int64_t tokens, int64_t heads,
                 int64_t rope_heads, int elem_bytes, hipStream_t stream) {
    if (tokens < 0 || heads < 0) return FP8G_ERR_SHAPE;
    if (elem_bytes != 1 && elem_bytes != 2) return FP8G_ERR_DTYPE;
    if (tokens == 0 || heads == 0) return FP8G_OK;
    if (rope_heads != 1 && rope_heads != heads) return FP8G_ERR_SHAPE;
    const int64_t k_bytes = mul3(tokens, heads, 192 * elem_bytes);
    const int64_t n_bytes = mul3(tokens, heads, 128 * elem_bytes);
    const int64_t r_bytes = mul3(tokens, rope_heads, 64 * elem_bytes);
    if (k_bytes < 0 || n_bytes < 0 || r_bytes < 0 || k_bytes > ((int64_t)1 << 60)) return FP8G_ERR_UNSUPPORTED;
    if (!k || !k_nope || !k_rope) return FP8G_ERR_NULL;
    if (!aligned16(k) || !aligned16(k_nope) || !aligned16(k_rope)) return FP8G_ERR_ALIGN;
    const Range rk = range_of(k, k_bytes);
    if (overlaps(rk, range_of(k_nope, n_bytes)) || overlaps(rk, range_of(k_rope, r_bytes))) return FP8G_ERR_OVERLAP;
    return hip_status(fp8g::launch_concat_mla_k(k, k_nope, k_rope, tokens, heads, rope_heads, elem_bytes, stream));
}

int fp8g_gemm_schedule(int64_t m, int64_t n, int64_t k, int mode, int cus, int* tile_m, int* tile_n, int* split,
                       int* split_tiles) {
    if (m < 0 || n < 0 || k < 0 || cus < 1) return FP8G_ERR_SHAPE;
    if (mode != 0 && mode != 1) return FP8G_ERR_DTYPE;
    if (!tile_m || !tile_n || !split || !split_tiles) return FP8G_ERR_NULL;
    if (fp8g::schedule_gemm(m, n, k, mode, cus, tile_m, tile_n, split, split_tiles) != hipSuccess)
        return FP8G_ERR_UNSUPPORTED;
    return FP8G_OK;
}

int fp8g_roof_mfma(int64_t blocks, int64_t iters, float* sink, hipStream_t stream) {
    if (blocks < 1 || iters < 1 || blocks >= ((int64_t)1 << 31) || iters >= ((int64_t)1 << 31)) return FP8G_ERR_SHAPE;
    if (!sink) return FP8G_ERR_NULL;
    return hip_status(fp8g::launch_roof_mfma(blocks, iters, sink, stream));
}

int fp8g_roof_stream(const void* src, int64_t bytes, void* dst, int write_ratio, int nontemporal_stores,
                     hipStream_t stream) {
    if (bytes < 0 || bytes % 16 != 0 || (write_ratio != 1 && write_ratio != 4)) return FP8G_ERR_SHAPE;
    if (nontemporal_stores != 0 && nontemporal_stores != 1) return FP8G_ERR_DTYPE;
    if (bytes == 0) return FP8G_OK;
    if (!src || !dst) return FP8G_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst)) return FP8G_ERR_ALIGN;
    if (overlaps(range_of(src, bytes), range_of(dst, bytes / write_ratio))) return FP8G_ERR_OVERLAP;
    return hip_status(fp8g::launch_roof_stream(src, bytes, dst, write_ratio, nontemporal_stores, stream));
}

const char* fp8g_status_string(int status) {
    switch (status) {
        case FP8G_OK: return "ok";
        case FP8G_ERR_NULL: return "a required pointer is NULL";
        case FP8G_ERR_SHAPE: return "invalid shape (negative extent, or k / cols not a multiple of 32 for MXFP8)";
        case FP8G_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case FP8G_ERR_DTYPE: return "unknown output dtype, operand format, input dtype, granularity or element size";
        case FP8G_ERR_OVERLAP: return "an output overlaps an input or another output";
        case FP8G_ERR_UNSUPPORTED: return "outside the library's limits (GEMM: k % 16, k >= 2^23, m >= 2^31, a 256-row panel of D over 2^31 bytes; quantizer rows >= 2^31; size overflow)";
        case FP8G_ERR_HIP: return "the HIP runtime rejected the launch";
        default: return "unknown status";
    }
}

}  // extern "C"
