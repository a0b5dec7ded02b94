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
// Pipeline, per 128-byte stage s (one wave per SIMD, so the order of the
// instruction stream is the schedule):
//   steps 0-15   k-step 0 on the matrix cores, interleaved with the LDS reads
//                of the k-step-1 fragments and half of the fill items (write a
//                16-byte chunk of stage s+1 from registers to LDS, then reload
//                that register with the chunk of stage s+2);
//   steps 16-23  k-step 1, with the other half of the fill items;
//   barrier;
//   steps 24-31  the rest of k-step 1, with the LDS reads of stage s+1's
//                k-step-0 fragments.
// Every global load has one whole stage (~2000 cycles) to land, and the LDS
// and vector-memory traffic is spread evenly instead of arriving in bursts
// that would block the issue of matrix-core instructions.
//
// LDS: two stages of A and B tiles, 2 x (32 + 32) KB.  Rows are 128 bytes
// (eight 16-byte chunks); chunk c of row r lives at chunk slot c ^ key(r),
// key(r) = (r & 7) ^ ((r >> 3) & 1), so the 16-byte fragment reads of 16
// consecutive rows and the coalesced fills (one row per eight lanes) touch
// distinct banks (measured: the plain c ^ (r & 7) left a 2-way conflict).
//
// Global loads are raw buffer loads over the tile's row panel: one 32-bit
// per-thread offset serves all chunks (row steps and the stage go in SGPRs),
// and rows past M / N fall outside the buffer and read as zero.
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
//
// Matrix-core results must never be consumed under a lane-divergent branch:
// the compiler may then move the instruction into that branch, where it runs
// with a partial EXEC mask yet still writes every lane.  Here they feed only
// the loop-carried accumulators and the epilogue after the loop.

#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace fp8g {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

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

// sched_group_barrier masks
constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100, SG_DS_WRITE = 0x200;
constexpr int BUF_DW3 = 0x00020000;   // raw (untyped) buffer descriptor word 3, 32-bit data format

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

// Swizzle key of a row: the 16-byte fragment reads of 16 consecutive rows
// (one LDS cycle of a 128-bit read: 64 banks of 4 bytes) must land on 16
// distinct 16-byte bank groups; with 128-byte rows two rows share a 256-byte
// bank line, so rows of one parity need 8 distinct slots -- (r & 7) ^ (r >> 3 & 1)
// gives that and also keeps any 8 consecutive rows distinct.
__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ uint32_t swz(int row, int chunk) {
    return (uint32_t)(row * BK + ((chunk ^ swz_key(row)) << 4));
}

// Buffer resource over `bytes` bytes at p: loads at or past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t panel(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, BUF_DW3);
}

template <bool MX, bool OUT_F32, bool KTAIL>
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

    const int nk = (K + BK - 1) / BK;
    const int nblk = K / 32;                            // MX scale bytes per row

    // ---- global -> registers: thread tid fills tile row tid/8 + 32p (p < 8),
    // 16-byte chunk tid%8 of every stage, for both operands.
    const uint32_t rows_a = (uint32_t)min(BM, M - m0), rows_b = (uint32_t)min(BN, N - n0);
    const __amdgpu_buffer_rsrc_t rsA = panel(A + (int64_t)m0 * K, rows_a * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t rsB = panel(B + (int64_t)n0 * K, rows_b * (uint32_t)K);
    const uint32_t voff = (uint32_t)(tid >> 3) * (uint32_t)K + (uint32_t)(tid & 7) * 16u;
    const uint32_t row_step = 32u * (uint32_t)K;

    v4u ra[CHUNKS_PER_THREAD], rb[CHUNKS_PER_THREAD];
    auto gload = [&](int st) {
        const uint32_t k0 = (uint32_t)st * BK;
#pragma unroll
        for (int p = 0; p < CHUNKS_PER_THREAD; ++p) {
            ra[p] = __builtin_amdgcn_raw_buffer_load_b128(rsA, voff, k0 + p * row_step, 0);
            rb[p] = __builtin_amdgcn_raw_buffer_load_b128(rsB, voff, k0 + p * row_step, 0);
        }
    };
    // registers -> LDS (swizzled); row tid/8 + 32p keeps the swizzle key of row tid/8
    // (the key depends on row % 16 only).
    // With a K tail, chunks past K (which read the next row) are zeroed here.
    const uint32_t lds_w = swz(tid >> 3, tid & 7);
    auto lstore = [&](int buf, int st) {
        uint8_t* sA = smem + buf * STAGE_BYTES + lds_w;
        uint8_t* sB = sA + TILE_BYTES;
        uint32_t keep = 0xFFFFFFFFu;
        if constexpr (KTAIL) keep = ((st * BK + (tid & 7) * 16) < K) ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int p = 0; p < CHUNKS_PER_THREAD; ++p) {
            v4u a = ra[p], b = rb[p];
            if constexpr (KTAIL) {
                a &= keep;
                b &= keep;
            }
            *reinterpret_cast<v4u*>(sA + p * (32 * BK)) = a;
            *reinterpret_cast<v4u*>(sB + p * (32 * BK)) = b;
        }
    };

    // The matrix core reads a lane's 32 operand bytes as two 16-byte halves:
    // bytes 0-15 belong to K block 0 of the 64-wide step and bytes 16-31 to
    // block 1; lanes 32-63 hold the upper 16 of each block.  So in k-step ks
    // this lane takes chunks ks*4 + lhi and ks*4 + 2 + lhi, and the scale of
    // block 0 / 1 of the step comes from lanes 0-31 / 32-63.
    const int rsw = swz_key(l32);   // swizzle key of this lane's rows (row % 16 == l32 % 16)
    uint32_t fa_off[2][2], fb_off[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t sl = (uint32_t)(((ks * 4 + 2 * h + lhi) ^ rsw) << 4);
            fa_off[ks][h] = (uint32_t)((wm * WT + l32) * BK) + sl;
            fb_off[ks][h] = (uint32_t)(TILE_BYTES + (wn * WT + l32) * BK) + sl;
        }
    auto read_frags = [&](int buf, int ks, v8i* fa, v8i* fb) {
        const uint8_t* s0 = smem + buf * STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const v4u b0 = *reinterpret_cast<const v4u*>(s0 + fb_off[ks][0] + i * 32 * BK);
            const v4u b1 = *reinterpret_cast<const v4u*>(s0 + fb_off[ks][1] + i * 32 * BK);
            const v4u a0 = *reinterpret_cast<const v4u*>(s0 + fa_off[ks][0] + i * 32 * BK);
            const v4u a1 = *reinterpret_cast<const v4u*>(s0 + fa_off[ks][1] + i * 32 * BK);
            fb[i] = (v8i){(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
            fa[i] = (v8i){(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        }
    };

    // MX scales: per lane, one dword (the 4 blocks of a stage) for each of its
    // 4 m-rows and 4 n-rows, shifted right by 8*lhi so that byte 0 / byte 2
    // hold the block this lane half scales in k-step 0 / 1.  Rows past M / N
    // read 0 (their data is zero too).
    uint32_t sca[NB], scb[NB], nsca[NB], nscb[NB];
    __amdgpu_buffer_rsrc_t rsEA = rsA, rsEB = rsB;
    uint32_t ea_off = 0, eb_off = 0;
    if constexpr (MX) {
        rsEA = panel(ea + (int64_t)m0 * nblk, rows_a * (uint32_t)nblk);
        rsEB = panel(eb + (int64_t)n0 * nblk, rows_b * (uint32_t)nblk);
        ea_off = (uint32_t)(wm * WT + l32) * (uint32_t)nblk;
        eb_off = (uint32_t)(wn * WT + l32) * (uint32_t)nblk;
    }
    auto sload = [&](int st) {
        if constexpr (MX) {
            const int kb = st * (BK / 32);
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const uint32_t ro = (uint32_t)(i * 32 * nblk + kb);
                uint32_t va, vb;
                if constexpr (!KTAIL) {
                    va = __builtin_amdgcn_raw_buffer_load_b32(rsEA, ea_off, ro, 0);
                    vb = __builtin_amdgcn_raw_buffer_load_b32(rsEB, eb_off, ro, 0);
                } else {
                    // rows of nblk bytes (not a multiple of 4): gather bytes; 2^0 past the row end
                    va = vb = 0;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const bool in = kb + t < nblk;
                        const uint32_t xa = __builtin_amdgcn_raw_buffer_load_b8(rsEA, ea_off, ro + t, 0);
                        const uint32_t xb = __builtin_amdgcn_raw_buffer_load_b8(rsEB, eb_off, ro + t, 0);
                        va |= (in ? xa : 127u) << (8 * t);
                        vb |= (in ? xb : 127u) << (8 * t);
                    }
                }
                nsca[i] = va >> (8 * lhi);
                nscb[i] = vb >> (8 * lhi);
            }
        }
    };

    v16f acc[NB][NB];   // [n block][m block]
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = (v16f){};

    auto mfma = [&](int i, int j, const v8i* fa, const v8i* fb, int ks) {
        if constexpr (MX) {
            if (ks == 0)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[i], fa[j], acc[i][j], 0, 0, 0,
                                                                          (int)scb[i], 0, (int)sca[j]);
            else
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[i], fa[j], acc[i][j], 0, 0, 2,
                                                                          (int)scb[i], 2, (int)sca[j]);
        } else {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[i], fa[j], acc[i][j], 0, 0, 0, 127, 0,
                                                                      127);
        }
    };

    // One fill item q (0..15) = one 16-byte chunk of A (q even) or B (q odd):
    // write its register to LDS, then reload the register for a later stage.
    auto store_item = [&](int buf, int st, int q) {
        uint8_t* dst = smem + buf * STAGE_BYTES + lds_w + (q & 1) * TILE_BYTES + (q >> 1) * (32 * BK);
        v4u v = (q & 1) ? rb[q >> 1] : ra[q >> 1];
        if constexpr (KTAIL) v &= ((st * BK + (tid & 7) * 16) < K) ? 0xFFFFFFFFu : 0u;   // chunks past K
        *reinterpret_cast<v4u*>(dst) = v;
    };
    auto load_item = [&](int st, int q) {
        const uint32_t so = (uint32_t)st * BK + (uint32_t)(q >> 1) * row_step;
        if (q & 1)
            rb[q >> 1] = __builtin_amdgcn_raw_buffer_load_b128(rsB, voff, so, 0);
        else
            ra[q >> 1] = __builtin_amdgcn_raw_buffer_load_b128(rsA, voff, so, 0);
    };

    v8i f0a[NB], f0b[NB], f1a[NB], f1b[NB];
    if (nk > 0) {
        // prologue: stage 0 -> LDS buffer 0; stage 1 (or 0 again) in flight to registers
        gload(0);
        sload(0);
        lstore(0, 0);
        gload(min(1, nk - 1));
        __syncthreads();
        read_frags(0, 0, f0a, f0b);

        // Loop invariant at the top of stage s: LDS buffer s&1 holds stage s, its
        // k-step-0 fragments are in f0a/f0b, and stage s+1 is in flight to ra/rb.
        // Stages past the end are clamped to the last one: the extra loads and
        // LDS writes are never read, and the body needs no branch.
        // Memory traffic is spread evenly over the 32 matrix-core steps: each
        // fill item is written to LDS and reloaded at the same point of every
        // stage, so each load has exactly one stage to land.
        for (int s = 0; s < nk; ++s) {
            const int cur = s & 1, nxt = cur ^ 1;
            const int st1 = min(s + 1, nk - 1), st2 = min(s + 2, nk - 1);
            if constexpr (MX) {
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    sca[i] = nsca[i];
                    scb[i] = nscb[i];
                }
                sload(st1);
            }
            // steps 0-15 (k-step 0): k-step-1 fragments from LDS; fill items 0-7
            read_frags(cur, 1, f1a, f1b);
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j) mfma(i, j, f0a, f0b, 0);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                store_item(nxt, st1, q);
                load_item(st2, q);
            }
            // steps 16-23 (k-step 1): fill items 8-15
#pragma unroll
            for (int t = 0; t < 8; ++t) mfma(t / NB, t % NB, f1a, f1b, 1);
#pragma unroll
            for (int q = 8; q < 16; ++q) {
                store_item(nxt, st1, q);
                load_item(st2, q);
            }
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_DS_WRITE, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
            }
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_DS_WRITE, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
            }
            __syncthreads();
            // steps 24-31: the next stage's k-step-0 fragments load behind them
            read_frags(nxt, 0, f0a, f0b);
#pragma unroll
            for (int t = 8; t < 16; ++t) mfma(t / NB, t % NB, f1a, f1b, 1);
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
            }
        }
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

template <bool MX, bool OUT_F32, bool KTAIL>
static hipError_t launch_one(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                             const float* sa, const float* sb, const uint8_t* ea, const uint8_t* eb, void* D,
                             hipStream_t stream) {
    auto kern = gemm_fp8_kernel<MX, OUT_F32, KTAIL>;
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

template <bool MX>
static hipError_t launch_mode(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                              const float* sa, const float* sb, const uint8_t* ea, const uint8_t* eb, void* D,
                              int out_f32, hipStream_t stream) {
    const bool tail = (k % BK) != 0;
    if (out_f32)
        return tail ? launch_one<MX, true, true>(m, n, k, A, B, sa, sb, ea, eb, D, stream)
                    : launch_one<MX, true, false>(m, n, k, A, B, sa, sb, ea, eb, D, stream);
    return tail ? launch_one<MX, false, true>(m, n, k, A, B, sa, sb, ea, eb, D, stream)
                : launch_one<MX, false, false>(m, n, k, A, B, sa, sb, ea, eb, D, stream);
}

// 32-bit buffer offsets: a 256-row panel of K bytes must stay below 2^32.
static bool fits(int64_t m, int64_t n, int64_t k) {
    const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
    return m < (1LL << 31) && n < (1LL << 31) && k < (1LL << 24) && tiles < (1LL << 31);
}

hipError_t launch_gemm_scaled(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                              const float* sa, const float* sb, void* D, int out_f32, hipStream_t stream) {
    if (!fits(m, n, k)) return hipErrorInvalidValue;
    return launch_mode<false>(m, n, k, A, B, sa, sb, nullptr, nullptr, D, out_f32, stream);
}

hipError_t launch_gemm_mx(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                          const uint8_t* ea, const uint8_t* eb, void* D, int out_f32, hipStream_t stream) {
    if (!fits(m, n, k)) return hipErrorInvalidValue;
    return launch_mode<true>(m, n, k, A, B, nullptr, nullptr, ea, eb, D, out_f32, stream);
}

}  // namespace fp8g
