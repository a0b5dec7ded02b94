// Plain C++ oracle -- test infrastructure (never linked into the library).
//
// The same definitions as the numpy oracle (oracle/*.py), written again
// independently in plain scalar C++ with double-precision accumulation, so
// that the two can be checked against each other and the cast can be checked
// exhaustively over all 2^32 fp32 bit patterns.
//
//   * FP8 decode from the bit fields: OCP E4M3FN (bias 7, NaN only at
//     S.1111.111, largest 448 -- the constant of `_calibrate_scales` on the
//     page "FP8 推理基础设施（五）：从 DeepGEMM 到 vLLM") and OCP E5M2 (bias 15,
//     IEEE-style Inf/NaN, largest 57344 -- the second FP8 type of the page on
//     FlashInfer's concat_mla_k with FP8 inputs).
//   * The saturating round-to-nearest-even cast, twice: as the definition
//     (the nearest of the format's decoded magnitudes, ties to the even code)
//     and as integer bit manipulation of the fp32 input.
//   * The row-wise quantizer: s = fp32(amax / MAX), q = cast(fp32(x / s)).
//   * The MX block quantizer (page "[sglang] FlashInfer v0.6.7 MXFP8 Gemm
//     통합", section 1): per 32 elements of a row the smallest power of two
//     2^e with amax <= 448 * 2^e, q = cast(x * 2^-e), scale code e + 127.
//   * Mode (a): D = sa[m] sb[n] sum_k dec(A[m,k]) dec(B[n,k]) in double, and
//     mode (b): D = sum_j 2^(ea+eb-254) sum_{t<32} dec dec (the MXFP8 page,
//     sections 1-2), plain loops, each with the weight of the error bound
//     (the same sums over |products|).
//   * The matrix-core truncation term T of the error bound (the same
//     definition as oracle.gemm.alignment_term).
//
// The quantizers, GEMMs and T split their rows or output columns over host
// threads, for checks of full-size results; every output is still one
// sequential loop, so the thread count does not change any result.
//
// Build: g++ -O2 -shared -fPIC -pthread (no vector intrinsics).  C entry points only.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// format description: exponent bits, mantissa bits, bias, IEEE-style specials
struct Fmt {
    int ebits, mbits, bias;
    bool ieee;      // true: all-ones exponent is Inf/NaN (E5M2); false: only S.1111.111 is NaN (E4M3FN)
    int max_code;   // largest finite magnitude code (0x7E / 0x7B)
};
constexpr Fmt E4M3{4, 3, 7, false, 0x7E};
constexpr Fmt E5M2{5, 2, 15, true, 0x7B};

const Fmt& fmt_of(int f) { return f == 1 ? E5M2 : E4M3; }

// fn(lo, hi) over [0, n) in `threads` contiguous ranges (<= 0: all hardware threads).
template <class Fn>
void parallel_ranges(int64_t n, int threads, Fn fn) {
    int nt = threads > 0 ? threads : (int)std::max(1u, std::thread::hardware_concurrency());
    nt = (int)std::min<int64_t>(nt, std::max<int64_t>(n, 1));
    if (nt <= 1) {
        fn((int64_t)0, n);
        return;
    }
    std::vector<std::thread> pool;
    for (int i = 0; i < nt; ++i) pool.emplace_back(fn, n * i / nt, n * (i + 1) / nt);
    for (auto& th : pool) th.join();
}

double decode(const Fmt& F, uint8_t c) {
    const int s = c >> 7;
    const int e = (c >> F.mbits) & ((1 << F.ebits) - 1);
    const int m = c & ((1 << F.mbits) - 1);
    const int emax = (1 << F.ebits) - 1;
    double mag;
    if (F.ieee && e == emax) {
        mag = m == 0 ? INFINITY : NAN;
    } else if (!F.ieee && e == emax && m == (1 << F.mbits) - 1) {
        mag = NAN;
    } else if (e == 0) {
        mag = std::ldexp((double)m, 1 - F.bias - F.mbits);
    } else {
        mag = std::ldexp((double)((1 << F.mbits) + m), e - F.bias - F.mbits);
    }
    return s ? -mag : mag;
}

float bits_to_float(uint32_t u) {
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}
uint32_t float_to_bits(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return u;
}

// The non-negative finite magnitudes of a format, codes 0 .. max_code (ascending).
struct Mags {
    double v[128];
    explicit Mags(const Fmt& F) {
        for (int c = 0; c <= F.max_code; ++c) v[c] = decode(F, (uint8_t)c);
    }
};
const Mags& mags_of(const Fmt& F) {
    static const Mags e4(E4M3), e5(E5M2);   // initialised once (thread-safe)
    return F.ebits == 5 ? e5 : e4;
}

// The definition: nearest of the non-negative finite magnitudes, ties to the
// even code, saturating, sign copied; NaN gives 0x7F with the sign.
uint8_t encode_nearest(const Fmt& F, float x) {
    const uint8_t sign = (uint8_t)(float_to_bits(x) >> 31) << 7;
    if (std::isnan(x)) return (uint8_t)(0x7F | sign);
    const double* mag = mags_of(F).v;
    const double a = std::fabs((double)x);
    if (a >= mag[F.max_code]) return (uint8_t)(F.max_code | sign);
    int lo = 0, hi = F.max_code;   // mag[lo] <= a < mag[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (mag[mid] <= a) lo = mid; else hi = mid;
    }
    const double mid = (mag[lo] + mag[hi]) * 0.5;   // exact in double
    int c;
    if (a > mid) c = hi;
    else if (a < mid) c = lo;
    else c = (lo % 2 == 0) ? lo : hi;
    return (uint8_t)(c | sign);
}

// The same cast by integer arithmetic on the fp32 fields: align the 24-bit
// significand to the code's last mantissa place and round half to even.
uint8_t encode_bits(const Fmt& F, float x) {
    const uint32_t u = float_to_bits(x);
    const uint8_t sign = (uint8_t)(u >> 31) << 7;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return (uint8_t)(0x7F | sign);                       // NaN
    const uint32_t top = float_to_bits((float)mags_of(F).v[F.max_code]);
    if (a >= top) return (uint8_t)(F.max_code | sign);                         // saturate (Inf too)
    if (a < 0x00800000u) return sign;                                          // zero, fp32 subnormal: below half the smallest code
    const int e = (int)(a >> 23) - 127;                                        // x = sig * 2^(e-23)
    const uint32_t sig = (a & 0x7FFFFFu) | 0x800000u;
    const int emin = 1 - F.bias;                                               // smallest normal exponent
    // target unit: 2^(e - mbits) for normals, 2^(emin - mbits) below them
    const int unit = (e >= emin ? e : emin) - F.mbits;
    const int shift = 23 - (e - unit);                                         // sig >> shift = x / 2^unit
    uint32_t q;
    if (shift >= 32) {
        q = 0;                                                                 // far below half a unit
    } else {
        q = sig >> shift;
        const uint32_t rem = sig & ((1u << shift) - 1u);
        const uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (q & 1u))) ++q;
    }
    // q counts units of 2^unit: for normals 2^mbits <= q <= 2^(mbits+1)
    // (the top rolls into the next binade), below them q <= 2^mbits
    uint32_t code;
    if (e >= emin) {
        int E = e + F.bias;
        if (q == (2u << F.mbits)) { q >>= 1; ++E; }
        code = ((uint32_t)E << F.mbits) | (q - (1u << F.mbits));
    } else {
        code = q;   // subnormal codes; q == 2^mbits is the smallest normal code
    }
    if (code > (uint32_t)F.max_code) code = (uint32_t)F.max_code;
    return (uint8_t)(code | sign);
}

}  // namespace

extern "C" {

double fp8o_decode(int fmt, uint8_t c) { return decode(fmt_of(fmt), c); }
uint8_t fp8o_encode_nearest(int fmt, float x) { return encode_nearest(fmt_of(fmt), x); }
uint8_t fp8o_encode_bits(int fmt, float x) { return encode_bits(fmt_of(fmt), x); }

// Every fp32 pattern in [lo, hi): both casts; returns the number of patterns
// where they differ and the first one in *first (unchanged if none).
int64_t fp8o_cast_sweep(int fmt, uint64_t lo, uint64_t hi, uint32_t* first) {
    const Fmt& F = fmt_of(fmt);
    int64_t bad = 0;
    for (uint64_t p = lo; p < hi; ++p) {
        const float x = bits_to_float((uint32_t)p);
        if (encode_nearest(F, x) != encode_bits(F, x)) {
            if (bad == 0 && first) *first = (uint32_t)p;
            ++bad;
        }
    }
    return bad;
}

// Batch cast (definition) of n floats.
void fp8o_encode_array(int fmt, const float* x, int64_t n, uint8_t* q) {
    const Fmt& F = fmt_of(fmt);
    for (int64_t i = 0; i < n; ++i) q[i] = encode_nearest(F, x[i]);
}

// Row-wise quantizer: s[r] = fp32(max_c |x| / MAX); q = cast(fp32(x / s)); s == 0 gives signed zeros.
void fp8o_quantize_rowwise(int fmt, const float* x, int64_t rows, int64_t cols, uint8_t* q, float* s, int threads) {
    const Fmt& F = fmt_of(fmt);
    const float maxv = (float)mags_of(F).v[F.max_code];
    parallel_ranges(rows, threads, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; ++r) {
            float amax = 0.0f;
            for (int64_t c = 0; c < cols; ++c) amax = std::fmax(amax, std::fabs(x[r * cols + c]));
            const float sr = amax / maxv;
            s[r] = sr;
            for (int64_t c = 0; c < cols; ++c) {
                const float v = x[r * cols + c];
                const float y = sr == 0.0f ? std::copysign(0.0f, v) : v / sr;
                q[r * cols + c] = encode_nearest(F, y);
            }
        }
    });
}

// MX block quantizer, E4M3 elements and UE8M0 scales, blocks of 32 along a
// row (cols % 32 == 0, finite inputs): e = the smallest integer with
// amax <= 448 * 2^e, at least -127 (an all-zero block takes -127);
// q = cast(x * 2^-e), exact in double and in fp32 wherever the cast can give a
// nonzero code; the scale code is e + 127.
void fp8o_mx_quantize(const float* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* e, int threads) {
    const int64_t nb = cols / 32;
    const double maxv = mags_of(E4M3).v[E4M3.max_code];
    parallel_ranges(rows, threads, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t j = 0; j < nb; ++j) {
                const float* xb = x + r * cols + 32 * j;
                double amax = 0.0;
                for (int t = 0; t < 32; ++t) amax = std::max(amax, std::fabs((double)xb[t]));
                int ex = -127;
                if (amax > 0.0) {
                    int fe;
                    std::frexp(amax, &fe);   // 2^(fe-1) <= amax < 2^fe, so 448 * 2^(fe-10) < amax
                    ex = fe - 10;
                    while (amax > std::ldexp(maxv, ex)) ++ex;
                    ex = std::max(ex, -127);
                }
                e[r * nb + j] = (uint8_t)(ex + 127);
                for (int t = 0; t < 32; ++t)
                    q[r * cols + 32 * j + t] = encode_nearest(E4M3, (float)std::ldexp((double)xb[t], -ex));
            }
    });
}

// Mode (a) in double: D[m,n] = sa[m] sb[n] sum_k dec(A[m,k]) dec(B[n,k]), and
// (W not null) the bound's weight W[m,n] = |sa[m] sb[n]| sum_k |dec(A[m,k]) dec(B[n,k])|.
void fp8o_gemm_scaled(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K, const uint8_t* A, const uint8_t* B,
                      const float* sa, const float* sb, double* D, double* W, int threads) {
    double da[256], db[256];
    for (int c = 0; c < 256; ++c) {
        da[c] = decode(fmt_of(fmt_a), (uint8_t)c);
        db[c] = decode(fmt_of(fmt_b), (uint8_t)c);
    }
    parallel_ranges(N, threads, [&](int64_t n0, int64_t n1) {
        for (int64_t n = n0; n < n1; ++n)
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0, mag = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const double p = da[A[m * K + k]] * db[B[n * K + k]];
                    acc += p;
                    mag += std::fabs(p);
                }
                D[m * N + n] = acc * (double)sa[m] * (double)sb[n];
                if (W) W[m * N + n] = mag * std::fabs((double)sa[m]) * std::fabs((double)sb[n]);
            }
    });
}

// Mode (b) in double: D[m,n] = sum_j 2^(ea[m,j]-127) 2^(eb[n,j]-127) sum_{t<32} dec(A) dec(B),
// and (W not null) W[m,n], the same sum over |products|.
void fp8o_gemm_mx(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K, const uint8_t* A, const uint8_t* B,
                  const uint8_t* ea, const uint8_t* eb, double* D, double* W, int threads) {
    double da[256], db[256];
    for (int c = 0; c < 256; ++c) {
        da[c] = decode(fmt_of(fmt_a), (uint8_t)c);
        db[c] = decode(fmt_of(fmt_b), (uint8_t)c);
    }
    const int64_t nb = K / 32;
    parallel_ranges(N, threads, [&](int64_t n0, int64_t n1) {
        for (int64_t n = n0; n < n1; ++n)
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0, mag = 0.0;
                for (int64_t j = 0; j < nb; ++j) {
                    double blk = 0.0, bmag = 0.0;
                    for (int64_t t = 0; t < 32; ++t) {
                        const double p = da[A[m * K + 32 * j + t]] * db[B[n * K + 32 * j + t]];
                        blk += p;
                        bmag += std::fabs(p);
                    }
                    const int x = (int)ea[m * nb + j] + (int)eb[n * nb + j] - 254;
                    acc += std::ldexp(blk, x);
                    mag += std::ldexp(bmag, x);
                }
                D[m * N + n] = acc;
                if (W) W[m * N + n] = mag;
            }
    });
}

// Matrix-core truncation term, unscaled: T[m,n] = sum over runs g of 8
// consecutive K values of sum_t [p_t off the grid] min(|p_t|, grid_g), with
// p_t = dec(A[m,t]) dec(B[n,t]), grid_g = 2^(E_g - 13) and E_g the largest
// exponent sum x_a + x_b of the run (x: the unbiased exponent field, zeros
// and subnormals at the format's smallest normal exponent; a ragged last run
// is padded with zero codes).  Mode (b) (ea, eb not null): each run's sum is
// multiplied by 2^(ea + eb - 254) of its 32-element block.  NaN and infinity
// codes are outside the contract (the caller rejects them).  Columns are split
// over `threads` threads (<= 0: all hardware threads).
void fp8o_alignment_term(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K, const uint8_t* A, const uint8_t* B,
                         const uint8_t* ea, const uint8_t* eb, double* T, int threads) {
    const Fmt& FA = fmt_of(fmt_a);
    const Fmt& FB = fmt_of(fmt_b);
    // magnitude of every code, and its exponent as the matrix core aligns it
    double mag_a[128], mag_b[128];
    int ex_a[128], ex_b[128];
    for (int c = 0; c < 128; ++c) {
        mag_a[c] = std::fabs(decode(FA, (uint8_t)c));
        mag_b[c] = std::fabs(decode(FB, (uint8_t)c));
        ex_a[c] = std::max((c >> FA.mbits) & ((1 << FA.ebits) - 1), 1) - FA.bias;
        ex_b[c] = std::max((c >> FB.mbits) & ((1 << FB.ebits) - 1), 1) - FB.bias;
    }
    const int64_t G = (K + 7) / 8;
    const int64_t nb = K / 32;
    auto code = [](const uint8_t* row, int64_t k, int64_t K) -> int { return k < K ? (row[k] & 0x7F) : 0; };
    auto work = [&](int64_t n0, int64_t n1) {
        for (int64_t n = n0; n < n1; ++n) {
            const uint8_t* b = B + n * K;
            for (int64_t m = 0; m < M; ++m) {
                const uint8_t* a = A + m * K;
                double total = 0.0, block = 0.0;
                for (int64_t g = 0; g < G; ++g) {
                    int ca[8], cb[8];
                    int E = -1000;
                    for (int t = 0; t < 8; ++t) {
                        ca[t] = code(a, 8 * g + t, K);
                        cb[t] = code(b, 8 * g + t, K);
                        E = std::max(E, ex_a[ca[t]] + ex_b[cb[t]]);
                    }
                    const double grid = std::ldexp(1.0, E - 13);
                    double run = 0.0;
                    for (int t = 0; t < 8; ++t) {
                        const double p = mag_a[ca[t]] * mag_b[cb[t]];
                        const double q = p / grid;   // exact: grid is a power of two
                        if (q != std::floor(q)) run += std::min(p, grid);
                    }
                    if (ea) {
                        block += run;
                        if (g % 4 == 3 || g == G - 1) {
                            const int64_t j = g / 4;
                            if (j < nb) total += std::ldexp(block, (int)ea[m * nb + j] + (int)eb[n * nb + j] - 254);
                            block = 0.0;
                        }
                    } else {
                        total += run;
                    }
                }
                T[m * N + n] = total;
            }
        }
    };
    parallel_ranges(N, threads, work);
}

}  // extern "C"
