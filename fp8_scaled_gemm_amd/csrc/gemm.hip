// FP8 (E4M3) scaled GEMM on the gfx950 matrix cores, two scaling modes.
//
//   mode (a)  D[m,n] = sa[m] sb[n] sum_k A[m,k] B[n,k]
//             per-token / per-channel fp32 scales, as the DeepGEMM call on the
//             page "FP8 推理基础设施（五）：从 DeepGEMM 到 vLLM".
//   mode (b)  D[m,n] = sum_j 2^(ea[m,j]-127) 2^(eb[n,j]-127) sum_{t<32} A[m,32j+t] B[n,32j+t]
//             MXFP8: one UE8M0 scale per 32 K elements of every row, as on the
//             page "[sglang] FlashInfer v0.6.7 MXFP8 Gemm 통합", sections 1-2.
//
// Both operands are K-major bytes (A [M,K], B [N,K]).  The work is a dense
// contraction (2MNK flops at arithmetic intensity in the thousands), so it is
// bound by the matrix cores, not HBM.
//
// Tiling: a 256-thread workgroup (4 waves, 2x2) owns a 256x256 output tile and
// walks K in 128-byte stages; each wave owns 128x128 = 4x4 blocks of the 32x32
// matrix-core tile, i.e. 256 fp32 accumulators per lane.  Every 32x32x64 step
// is one V_MFMA_SCALE_F32_32X32X64_F8F6F4; mode (a) passes the neutral scale
// code 127 (2^0) and applies sa, sb in the epilogue, mode (b) passes the
// operands' block scales.
//
// LDS: two stages of A and B tiles, 2 x (32 + 32) KB.  Rows are 128 bytes
// (eight 16-byte chunks); chunk c of row r lives at chunk slot c ^ (r & 7),
// so the 16-byte fragment reads of eight consecutive rows and the coalesced
// fills (one row per eight lanes) both touch 32 distinct banks.  Global loads
// for stage s+1 are in flight while stage s feeds the matrix cores; one
// barrier per stage.
//
// Operand roles: the matrix-core "A" operand is fed from B's rows (n) and the
// "B" operand from A's rows (m), so each lane's accumulator block holds one m
// and four consecutive n per group of registers: 8-byte (bf16) or 16-byte
// (fp32) row-contiguous stores in the epilogue.
//
// Workgroup -> tile order: consecutive workgroup ids go round-robin to the 8
// XCDs; the mapping gives each XCD a contiguous run of tiles, walked in
// groups of GROUP_M tile-rows, so the tiles an XCD runs together share A and
// B panels in its own L2.

#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace fp8g {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 256;        // tile rows (m)
constexpr int BN = 256;        // tile cols (n)
constexpr int BK = 128;        // bytes of K per stage
constexpr int NTHREADS = 256;
constexpr int WT = 128;        // wave tile edge
constexpr int NB = WT / 32;    // 32x32 blocks per wave-tile edge
constexpr int NUM_XCD = 8;
constexpr int GROUP_M = 8;

constexpr int TILE_BYTES = BM * BK;             // 32 KB, one operand, one stage
constexpr int STAGE_BYTES = 2 * TILE_BYTES;     // A + B
constexpr int LDS_BYTES = 2 * STAGE_BYTES;      // double buffered: 128 KB
constexpr int CHUNKS_PER_THREAD = TILE_BYTES / 16 / NTHREADS;   // 8

struct TileCoord {
    int tm, tn;
};

__device__ __forceinline__ TileCoord tile_of_block(int bid, int total, int tiles_m, int tiles_n) {
    // XCD-contiguous runs: bid % 8 is the XCD the hardware picks.
    const int q = total / NUM_XCD, r = total % NUM_XCD;
    const int xcd = bid % NUM_XCD, slot = bid / NUM_XCD;
    const int t = (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
    // grouped walk: GROUP_M tile-rows at a time, columns inside a group
    const int per_group = GROUP_M * tiles_n;
    const int g = t / per_group;
    const int first_m = g * GROUP_M;
    const int gm = min(GROUP_M, tiles_m - first_m);
    const int in = t - g * per_group;
    TileCoord c;
    c.tm = first_m + in % gm;
    c.tn = in / gm;
    return c;
}

__device__ __forceinline__ uint32_t swz(int row, int chunk) {
    return (uint32_t)(row * BK + ((chunk ^ (row & 7)) << 4));
}

// One 16-byte chunk of an operand row, or zeros past K.
__device__ __forceinline__ uint4 load_chunk(const uint8_t* __restrict__ base, int64_t row, int64_t ld,
                                            int64_t kbyte, int64_t K) {
    if (kbyte < K) return *reinterpret_cast<const uint4*>(base + row * ld + kbyte);
    return make_uint4(0u, 0u, 0u, 0u);
}

// Four UE8M0 bytes (blocks kb .. kb+3) of one row; 127 (2^0) past the end.
__device__ __forceinline__ uint32_t load_scale4(const uint8_t* __restrict__ e, int64_t row, int64_t nblk,
                                                int64_t kb, bool aligned) {
    const uint8_t* p = e + row * nblk + kb;
    if (aligned && kb + 4 <= nblk) return *reinterpret_cast<const uint32_t*>(p);
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) v |= (uint32_t)((kb + i < nblk) ? p[i] : (uint8_t)127) << (8 * i);
    return v;
}

template <bool MX, bool OUT_F32>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_fp8_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
    const float* __restrict__ sa, const float* __restrict__ sb, const uint8_t* __restrict__ ea,
    const uint8_t* __restrict__ eb, void* __restrict__ Dv) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const TileCoord tc = tile_of_block(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n);
    const int m0 = tc.tm * BM, n0 = tc.tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int l32 = lane & 31, lhi = lane >> 5;

    // ---- global -> LDS fill assignment: chunk id = tid + 256 p, row = id / 8, chunk = id % 8
    int frow[CHUNKS_PER_THREAD];
    int fchk[CHUNKS_PER_THREAD];
#pragma unroll
    for (int p = 0; p < CHUNKS_PER_THREAD; ++p) {
        const int id = tid + NTHREADS * p;
        frow[p] = id >> 3;
        fchk[p] = id & 7;
    }

    const int nk = (K + BK - 1) / BK;
    const int64_t nblk = K / 32;                        // MX scale bytes per row
    const bool scale_aligned = (nblk % 4) == 0;

    uint4 ra[CHUNKS_PER_THREAD], rb[CHUNKS_PER_THREAD];
    auto gload = [&](int s) {
        const int64_t k0 = (int64_t)s * BK;
#pragma unroll
        for (int p = 0; p < CHUNKS_PER_THREAD; ++p) {
            const int64_t kb = k0 + fchk[p] * 16;
            const int64_t am = min(m0 + frow[p], M - 1);
            const int64_t bn = min(n0 + frow[p], N - 1);
            ra[p] = load_chunk(A, am, K, kb, K);
            rb[p] = load_chunk(B, bn, K, kb, K);
        }
    };
    auto lstore = [&](int buf) {
        uint8_t* sA = smem + buf * STAGE_BYTES;
        uint8_t* sB = sA + TILE_BYTES;
#pragma unroll
        for (int p = 0; p < CHUNKS_PER_THREAD; ++p) {
            *reinterpret_cast<uint4*>(sA + swz(frow[p], fchk[p])) = ra[p];
            *reinterpret_cast<uint4*>(sB + swz(frow[p], fchk[p])) = rb[p];
        }
    };

    // MX scales: per lane, one dword (the 4 blocks of this stage) for each of
    // its 4 m-rows and 4 n-rows, shifted right by 8*lhi so that byte 0 / byte 2
    // hold the block this lane half scales in k-step 0 / 1.
    uint32_t sca[NB], scb[NB];
    uint32_t nsca[NB], nscb[NB];
    auto sload = [&](int s) {
        if constexpr (MX) {
            const int64_t kb = (int64_t)s * (BK / 32);
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int64_t am = min(m0 + wm * WT + i * 32 + l32, M - 1);
                const int64_t bn = min(n0 + wn * WT + i * 32 + l32, N - 1);
                nsca[i] = load_scale4(ea, am, nblk, kb, scale_aligned) >> (8 * lhi);
                nscb[i] = load_scale4(eb, bn, nblk, kb, scale_aligned) >> (8 * lhi);
            }
        }
    };

    v16f acc[NB][NB];   // [n block][m block]
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = (v16f){};

    if (nk > 0) {
        gload(0);
        sload(0);
        lstore(0);
    }
    __syncthreads();

    for (int s = 0; s < nk; ++s) {
        const int buf = s & 1;
        if constexpr (MX) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                sca[i] = nsca[i];
                scb[i] = nscb[i];
            }
        }
        const bool more = (s + 1) < nk;
        if (more) {
            gload(s + 1);
            sload(s + 1);
        }

        const uint8_t* sA = smem + buf * STAGE_BYTES;
        const uint8_t* sB = sA + TILE_BYTES;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            // The matrix core reads a lane's 32 operand bytes as two 16-byte
            // halves: bytes 0-15 belong to K block 0 of the 64-wide step and
            // bytes 16-31 to block 1; lanes 32-63 hold the upper 16 of each
            // block.  So this lane takes chunks ks*4 + lhi and ks*4 + 2 + lhi,
            // and the scale of block 0 / 1 of the step comes from lanes
            // 0-31 / 32-63 (shifted byte 0 for ks = 0, byte 2 for ks = 1).
            const int c0 = ks * 4 + lhi, c1 = c0 + 2;
            v8i fa[NB], fb[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int rn = wn * WT + i * 32 + l32;
                const int rm = wm * WT + i * 32 + l32;
                const uint4 b0 = *reinterpret_cast<const uint4*>(sB + swz(rn, c0));
                const uint4 b1 = *reinterpret_cast<const uint4*>(sB + swz(rn, c1));
                const uint4 a0 = *reinterpret_cast<const uint4*>(sA + swz(rm, c0));
                const uint4 a1 = *reinterpret_cast<const uint4*>(sA + swz(rm, c1));
                fb[i] = (v8i){(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
                fa[i] = (v8i){(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            }
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    if constexpr (MX) {
                        if (ks == 0)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                fb[i], fa[j], acc[i][j], 0, 0, 0, (int)scb[i], 0, (int)sca[j]);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                fb[i], fa[j], acc[i][j], 0, 0, 2, (int)scb[i], 2, (int)sca[j]);
                    } else {
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fb[i], fa[j], acc[i][j], 0, 0, 0, 127, 0, 127);
                    }
                }
        }

        if (more) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds m = .. + l32, and n = .. + 8g + 4*lhi + t (t = 0..3) in acc[.][.][4g+t]
    const bool vec_ok = (N % 4) == 0;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int m = m0 + wm * WT + j * 32 + l32;
        if (m >= M) continue;
        float smv = 1.0f;
        if constexpr (!MX) smv = sa[m];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WT + i * 32 + 8 * g + 4 * lhi;
                if (n >= N) continue;
                float v[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    float r = acc[i][j][4 * g + t];
                    if constexpr (!MX) {
                        const float snv = (n + t < N) ? sb[n + t] : 0.0f;
                        r = r * smv * snv;
                    }
                    v[t] = r;
                }
                const int64_t off = (int64_t)m * N + n;
                if constexpr (OUT_F32) {
                    float* D = reinterpret_cast<float*>(Dv);
                    if (vec_ok) {
                        *reinterpret_cast<float4*>(D + off) = make_float4(v[0], v[1], v[2], v[3]);
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            if (n + t < N) D[off + t] = v[t];
                    }
                } else {
                    uint16_t* D = reinterpret_cast<uint16_t*>(Dv);
                    if (vec_ok) {
                        const uint32_t lo = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
                        const uint32_t hi = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
                        *reinterpret_cast<uint2*>(D + off) = make_uint2(lo, hi);
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            if (n + t < N) D[off + t] = (uint16_t)bf16_bits(v[t]);
                    }
                }
            }
        }
    }
}

template <bool MX, bool OUT_F32>
static hipError_t launch_one(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                             const float* sa, const float* sb, const uint8_t* ea, const uint8_t* eb, void* D,
                             hipStream_t stream) {
    auto kern = gemm_fp8_kernel<MX, OUT_F32>;
    // 128 KB of dynamic LDS is above the default launch limit; raise it once.
    static std::once_flag once;
    static hipError_t attr_status = hipSuccess;
    std::call_once(once, [&] {
        attr_status = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    });
    if (attr_status != hipSuccess) return attr_status;
    const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
    kern<<<dim3((unsigned)tiles), dim3(NTHREADS), LDS_BYTES, stream>>>((int)m, (int)n, (int)k, A, B, sa, sb,
                                                                       ea, eb, D);
    return hipGetLastError();
}

static bool fits_int(int64_t m, int64_t n, int64_t k) {
    const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
    return m < (1LL << 31) && n < (1LL << 31) && k < (1LL << 31) && tiles < (1LL << 31);
}

hipError_t launch_gemm_scaled(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                              const float* sa, const float* sb, void* D, int out_f32, hipStream_t stream) {
    if (!fits_int(m, n, k)) return hipErrorInvalidValue;
    return out_f32 ? launch_one<false, true>(m, n, k, A, B, sa, sb, nullptr, nullptr, D, stream)
                   : launch_one<false, false>(m, n, k, A, B, sa, sb, nullptr, nullptr, D, stream);
}

hipError_t launch_gemm_mx(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                          const uint8_t* ea, const uint8_t* eb, void* D, int out_f32, hipStream_t stream) {
    if (!fits_int(m, n, k)) return hipErrorInvalidValue;
    return out_f32 ? launch_one<true, true>(m, n, k, A, B, nullptr, nullptr, ea, eb, D, stream)
                   : launch_one<true, false>(m, n, k, A, B, nullptr, nullptr, ea, eb, D, stream);
}

}  // namespace fp8g
