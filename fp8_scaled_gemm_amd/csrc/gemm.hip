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
// Tiling: a 256-thread workgroup (4 waves, 2x2) owns a 256x256 output tile;
// each wave owns 128x128 = 4x4 blocks of the 32x32 matrix-core tile (256 fp32
// accumulators per lane).  K is walked in 64-byte stages, one
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 per block per stage; mode (a) passes the
// neutral scale code 127 (2^0) and applies sa, sb in the epilogue, mode (b)
// passes the operands' block scales.
//
// Persistent workgroups: one per CU, each walking a list of tiles.  Its stages
// form one continuous stream across its tiles, so the loads of the next tile
// are in flight while the current tile's epilogue runs.
//
// Operand staging: direct global -> LDS loads (buffer_load_dwordx4 ... lds;
// lane L of a wave writes LDS bytes [M0 + 16L, M0 + 16L + 16)), four LDS stage
// buffers, issued three stages ahead.  No registers hold staged data and no
// LDS-write instructions are needed.  The compiler cannot track these loads
// (it would wait for all of them before every LDS read), so they are issued
// from inline assembly (they write LDS only, no registers) and the kernel
// waits for them itself: before the barrier of stage g it waits until only the
// loads issued after stage g+1's remain (vector-memory loads complete in
// order, so a count of outstanding loads identifies the stage).
//
// LDS layout per stage: A then B, 256 rows of 64 bytes (four 16-byte chunks);
// logical chunk c of row r sits in slot c ^ ((r >> 2) & 3).  A 128-bit read
// serves 16 lanes per LDS cycle (64 banks): 16 consecutive rows at one
// logical chunk hit 16 distinct 16-byte bank groups.  The swizzle is applied
// on the global side: lane L of a load fills slot L % 4 of row L / 4 and so
// fetches chunk (L % 4) ^ ((L / 16) & 3) of that row.  Mode (b) adds one
// dword of scales (4 blocks, a stage pair) per row and operand.
//
// The matrix core reads a lane's 32 operand bytes as two 16-byte halves:
// bytes 0-15 belong to K block 0 of the 64-wide step and bytes 16-31 to block
// 1; lanes 32-63 hold the upper 16 of each block.  So a lane takes chunks lhi
// and 2 + lhi of its row, and the scale of block 0 / 1 of the step comes from
// lanes 0-31 / 32-63.
//
// Operand roles: the matrix-core "A" operand is fed from B's rows (n) and the
// "B" operand from A's rows (m), so each lane's accumulator block holds one m
// and four consecutive n per group of registers: 8-byte (bf16) or 16-byte
// (fp32) row-contiguous stores in the epilogue.
//
// Tile order: workgroup b runs on XCD b % 8; each XCD gets a contiguous run of
// tiles, walked in groups of GROUP_M tile-rows, so the tiles an XCD runs
// together share A and B panels in its own L2.
//
// Matrix-core results must never be consumed under a lane-divergent branch:
// the compiler may then move the instruction into that branch, where it runs
// with a partial EXEC mask yet still writes every lane.  Here they feed only
// the accumulators and the epilogue, under uniform control flow.

#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace fp8g {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int BM = 256;        // tile rows (m)
constexpr int BN = 256;        // tile cols (n)
constexpr int BK = 64;         // bytes of K per stage (one matrix-core step)
constexpr int NTHREADS = 256;
constexpr int WT = 128;        // wave tile edge
constexpr int NB = WT / 32;    // 32x32 blocks per wave-tile edge
constexpr int NUM_XCD = 8;
constexpr int GROUP_M = 8;
constexpr int NSTAGE = 4;      // LDS stage buffers; loads run NSTAGE-1 stages ahead

constexpr int OP_BYTES = BM * BK;                 // 16 KB: one operand, one stage
constexpr int SCALE_BYTES = BM * 4;               // MX: one dword (4 blocks) per row, per operand
constexpr int STAGE_BYTES = 2 * OP_BYTES + 2 * SCALE_BYTES;   // 34 KB
constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;   // 136 KB
constexpr int DMA_PER_OP = OP_BYTES / 1024 / 4;   // 1 KB per wave instruction, 4 waves: 4

constexpr int BUF_DW3 = 0x00020000;   // raw (untyped) buffer descriptor word 3, 32-bit data format

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ __amdgpu_buffer_rsrc_t panel(const void* p, uint32_t bytes) {
    // buffer over `bytes` bytes at p: loads at or past the end return 0
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, BUF_DW3);
}

// 16 bytes per lane from buffer rs at (voff + soff) into LDS at lds_addr + 16 * lane.
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, __amdgpu_buffer_rsrc_t rs, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff)
                 : "memory", "m0");
}
// 4 bytes per lane into LDS at lds_addr + 4 * lane.
__device__ __forceinline__ void dma4(uint32_t lds_addr, uint32_t voff, __amdgpu_buffer_rsrc_t rs, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff)
                 : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

struct TileCoord {
    int tm, tn;
};

// Tile id -> tile coordinates: groups of GROUP_M tile-rows, columns inside a group.
__device__ __forceinline__ TileCoord tile_coord(int t, int tiles_m, int tiles_n) {
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

// ---------------------------------------------------------------- kernel

template <bool MX, bool OUT_F32, bool KTAIL>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_fp8_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
    const float* __restrict__ sa, const float* __restrict__ sb, const uint8_t* __restrict__ ea,
    const uint8_t* __restrict__ eb, void* __restrict__ Dv) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int l32 = lane & 31, lhi = lane >> 5;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int total = tiles_m * tiles_n;
    const int nk = (K + BK - 1) / BK;            // stages per tile
    const int nblk = K / 32;                     // MX scale bytes per row

    // ---- this workgroup's tiles: XCD x = b % 8 owns a contiguous run of tiles;
    // its W_x workgroups take every W_x-th tile of the run.
    const int G = gridDim.x, b = blockIdx.x;
    const int xcd = b % NUM_XCD, slot = b / NUM_XCD;
    const int wx = (G - xcd + NUM_XCD - 1) / NUM_XCD;                 // workgroups on this XCD
    const int q = total / NUM_XCD, r = total % NUM_XCD;
    const int run0 = xcd * q + min(xcd, r), runn = q + (xcd < r ? 1 : 0);
    const int my_tiles = (slot < runn) ? (runn - slot + wx - 1) / wx : 0;
    const int NS = my_tiles * nk;                                      // stages in this workgroup's stream
    auto tile_of = [&](int j) __attribute__((always_inline)) { return tile_coord(run0 + slot + j * wx, tiles_m, tiles_n); };

    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;   // LDS byte address of the stage buffers

    // ---- loads of the stream's stages, in order, into LDS buffer g % NSTAGE,
    // NSTAGE stages ahead of the stage being computed.  A cursor (tile, stage)
    // walks the stream; descriptors change once per tile.  Past the end of the
    // stream the last stage is loaded again into a free buffer (never read), so
    // every stage issues the same number of loads.
    // lane L of wave w fills row 16*(4p + w) + L/4, slot L%4, for p = 0..3
    const uint32_t dma_row = (uint32_t)(16 * wave + (lane >> 2));
    const uint32_t dma_voff = dma_row * (uint32_t)K + (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) * 16);
    // MX scales: dword DMA, lane L of wave w fills row 64*w + L (4 blocks = one stage pair)
    const uint32_t sdma_voff = (uint32_t)(64 * wave + lane) * (uint32_t)nblk;
    int ij = 0, is = 0, ig = 0;                        // cursor: tile, stage in tile, stream stage
    __amdgpu_buffer_rsrc_t rsA, rsB, rsEA, rsEB;
    auto cursor_tile = [&]() __attribute__((always_inline)) {
        const TileCoord tc = tile_of(min(ij, my_tiles - 1));
        const int m0 = tc.tm * BM, n0 = tc.tn * BN;
        const uint32_t rows_a = (uint32_t)min(BM, M - m0), rows_b = (uint32_t)min(BN, N - n0);
        rsA = panel(A + (int64_t)m0 * K, rows_a * (uint32_t)K);
        rsB = panel(B + (int64_t)n0 * K, rows_b * (uint32_t)K);
        if constexpr (MX) {
            rsEA = panel(ea + (int64_t)m0 * nblk, rows_a * (uint32_t)nblk);
            rsEB = panel(eb + (int64_t)n0 * nblk, rows_b * (uint32_t)nblk);
        }
    };
    // load q of the cursor's stage: q = 2p (+1) is row group p of A (B); in mode
    // (b) q = 8 (9) is the scale dword of A (B) for the stage's pair, which every
    // stage of the pair loads into its own buffer
    auto dma_item = [&](int q) __attribute__((always_inline)) {
        const int s_ld = ig < NS ? is : nk - 1;        // past the end: reload the last stage
        const uint32_t sbuf = lds0 + (uint32_t)((ig % NSTAGE) * STAGE_BYTES);
        if (q < 2 * DMA_PER_OP) {
            const int p = q >> 1;
            const uint32_t so = uniform((uint32_t)(s_ld * BK) + (uint32_t)(64 * p) * (uint32_t)K);
            dma16(uniform(sbuf + (uint32_t)((q & 1) * OP_BYTES + p * 4096 + wave * 1024)), dma_voff,
                  (q & 1) ? rsB : rsA, so);
        } else if constexpr (MX && !KTAIL) {
            const uint32_t so = uniform((uint32_t)(2 * (s_ld & ~1)));
            dma4(uniform(sbuf + (uint32_t)(2 * OP_BYTES + (q & 1) * SCALE_BYTES + wave * 256)), sdma_voff,
                 (q & 1) ? rsEB : rsEA, so);
        }
    };
    auto advance = [&]() __attribute__((always_inline)) {
        ++ig;
        if (++is == nk) {
            is = 0;
            ++ij;
            cursor_tile();
        }
    };

    // loads per stage
    constexpr int LOADS = 2 * DMA_PER_OP + ((MX && !KTAIL) ? 2 : 0);

    // ---- fragment reads (stage buffer, this lane's rows, chunks lhi and 2+lhi)
    const uint32_t key = (uint32_t)((l32 >> 2) & 3);
    const uint32_t frag_a0 = (uint32_t)((wm * WT + l32) * BK) + (((uint32_t)lhi ^ key) << 4);
    const uint32_t frag_a1 = (uint32_t)((wm * WT + l32) * BK) + (((uint32_t)(2 + lhi) ^ key) << 4);
    const uint32_t frag_b0 = frag_a0 - (uint32_t)(wm * WT * BK) + (uint32_t)(OP_BYTES + wn * WT * BK);
    const uint32_t frag_b1 = frag_a1 - (uint32_t)(wm * WT * BK) + (uint32_t)(OP_BYTES + wn * WT * BK);
    auto frag = [&](int g, uint32_t off0, uint32_t off1, int i) __attribute__((always_inline)) -> v8i {
        const uint8_t* sbuf = smem + (g % NSTAGE) * STAGE_BYTES;
        const v4u x0 = *reinterpret_cast<const v4u*>(sbuf + off0 + i * 32 * BK);
        const v4u x1 = *reinterpret_cast<const v4u*>(sbuf + off1 + i * 32 * BK);
        return (v8i){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    };

    // ---- MX scales for stage g: per lane and row block, the scale byte of this
    // lane half's block in byte 0 (so the matrix core always reads byte 0).
    // Non-tail: one dword (blocks 4p..4p+3, a stage pair) per row in the LDS
    // scale area of the stage.  Tail (rows of nblk bytes, not a
    // multiple of 4): bytes from global, 2^0 past the row end.  Rows past M / N
    // read 0 (their data is zero too).
    auto read_scales = [&](int g, int s, uint32_t* xa, uint32_t* xb) __attribute__((always_inline)) {
        if constexpr (MX) {
            const uint32_t sh = (uint32_t)(8 * (2 * (s & 1) + lhi));
            if constexpr (!KTAIL) {
                const uint8_t* sc = smem + (g % NSTAGE) * STAGE_BYTES + 2 * OP_BYTES;
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    xa[i] = *reinterpret_cast<const uint32_t*>(sc + (wm * WT + i * 32 + l32) * 4) >> sh;
                    xb[i] = *reinterpret_cast<const uint32_t*>(sc + SCALE_BYTES + (wn * WT + i * 32 + l32) * 4) >> sh;
                }
            } else {
                // unconditional buffer loads (no lane-divergent branch near the
                // matrix-core steps); rows past M / N read 0 from past the panel
                const TileCoord tc = tile_of(g / nk);
                const int m0 = tc.tm * BM, n0 = tc.tn * BN;
                const __amdgpu_buffer_rsrc_t pa = panel(ea + (int64_t)m0 * nblk, (uint32_t)min(BM, M - m0) * (uint32_t)nblk);
                const __amdgpu_buffer_rsrc_t pb = panel(eb + (int64_t)n0 * nblk, (uint32_t)min(BN, N - n0) * (uint32_t)nblk);
                const int kb = 2 * s + lhi;                 // this lane half's block of stage s
                const bool in = kb < nblk;
                const uint32_t kc = (uint32_t)min(kb, nblk - 1);
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    const uint32_t va = __builtin_amdgcn_raw_buffer_load_b8(
                        pa, (uint32_t)(wm * WT + i * 32 + l32) * (uint32_t)nblk + kc, 0, 0);
                    const uint32_t vb = __builtin_amdgcn_raw_buffer_load_b8(
                        pb, (uint32_t)(wn * WT + i * 32 + l32) * (uint32_t)nblk + kc, 0, 0);
                    xa[i] = in ? va : 127u;
                    xb[i] = in ? vb : 127u;
                }
            }
        }
    };

    // ---- K tail: the last stage of a tile holds chunks past K (the next row's
    // bytes, or zeros past the panel): zero them in LDS once the stage landed.
    auto fix_tail = [&](int g) __attribute__((always_inline)) {
        if constexpr (KTAIL) {
            const int s = g % nk;
            if (s == nk - 1) {
                uint8_t* sbuf = smem + (g % NSTAGE) * STAGE_BYTES;
                // 512 rows (A then B) x 4 chunks; thread tid handles chunk tid & 3 of rows tid/4 + 64 i
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int row = (tid >> 2) + 64 * i;         // 0..511
                    const int c = tid & 3;
                    if (s * BK + c * 16 >= K) {
                        const int rr = row & 255;
                        *reinterpret_cast<v4u*>(sbuf + (row >> 8) * OP_BYTES + rr * BK +
                                                ((c ^ ((rr >> 2) & 3)) << 4)) = (v4u){0u, 0u, 0u, 0u};
                    }
                }
            }
        }
    };

    // The empty asm after each step pins it where it is written: the builtin has
    // no side effects, so without it the optimizer may sink whole stages of
    // steps past later barriers, leaving the matrix core idle in between.
    auto mfma = [&](v16f& c, const v8i& fbi, const v8i& faj, uint32_t sbi, uint32_t saj) __attribute__((always_inline)) {
        if constexpr (MX)
            c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fbi, faj, c, 0, 0, 0, (int)sbi, 0, (int)saj);
        else
            c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fbi, faj, c, 0, 0, 0, 127, 0, 127);
        asm volatile("" : "+a"(c));
    };

    // ---- epilogue of stream tile j: lane holds m = .. + l32 and n = .. + 8g + 4*lhi + t
    // (t = 0..3) in acc[.][.][4g+t].  Buffer loads / stores over the tile's rows of
    // D, sa, sb: out-of-range lanes get an offset past the end, which the hardware
    // drops (stores) or reads as 0.  All scale loads are issued before the first
    // store: the vector-memory counter also counts stores, so a load waited for
    // after stores would wait for those stores too.
    constexpr int ESZ = OUT_F32 ? 4 : 2;
    auto epilogue = [&](int j, v16f (&acc)[NB][NB]) __attribute__((always_inline)) {
        const TileCoord tc = tile_of(j);
        const int m0 = tc.tm * BM, n0 = tc.tn * BN;
        const uint32_t rows = (uint32_t)min(BM, M - m0);
        const __amdgpu_buffer_rsrc_t rsD =
            panel(reinterpret_cast<uint8_t*>(Dv) + (int64_t)m0 * N * ESZ, rows * (uint32_t)N * ESZ);
        constexpr uint32_t OOB = 0x80000000u;   // beyond any panel (panels are < 2^31 bytes)
        float smv[NB], snv[NB][4][4];
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
            smv[jb] = 1.0f;
            if constexpr (!MX) {
                const int mr = wm * WT + jb * 32 + l32;
                smv[jb] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                        panel(sa + m0, rows * 4u), m0 + mr < M ? (uint32_t)mr * 4u : OOB, 0, 0));
            }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    snv[i][gq][t] = 1.0f;
                    // dword loads (the backend merges them): extracting the elements of
                    // a 128-bit buffer-load builtin one by one is folded to element 0
                    // by this compiler at -O3
                    if constexpr (!MX) {
                        const int n = n0 + wn * WT + i * 32 + 8 * gq + 4 * lhi + t;
                        snv[i][gq][t] = __builtin_bit_cast(
                            float, __builtin_amdgcn_raw_buffer_load_b32(panel(sb, (uint32_t)N * 4u), (uint32_t)n * 4u, 0, 0));
                    }
                }
        __builtin_amdgcn_sched_barrier(0);
        const bool vec_ok = (N % 4) == 0;
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
            const int mr = wm * WT + jb * 32 + l32;          // row inside the tile
            const bool mok = m0 + mr < M;
            const uint32_t rowoff = (uint32_t)mr * (uint32_t)N;
#pragma unroll
            for (int i = 0; i < NB; ++i) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int n = n0 + wn * WT + i * 32 + 8 * gq + 4 * lhi;
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        float x = acc[i][jb][4 * gq + t];
                        if constexpr (!MX) x = x * smv[jb] * snv[i][gq][t];
                        v[t] = x;
                    }
                    if (vec_ok) {
                        // n % 4 == 0 and N % 4 == 0: the 4 values are all in or all out
                        const uint32_t off = (mok && n < N) ? (rowoff + (uint32_t)n) * ESZ : OOB;
                        if constexpr (OUT_F32) {
                            const v4u w4 = {__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                                            __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3])};
                            __builtin_amdgcn_raw_buffer_store_b128(w4, rsD, off, 0, 0);
                        } else {
                            typedef unsigned int v2u __attribute__((ext_vector_type(2)));
                            const v2u w2 = {bf16_bits(v[0]) | (bf16_bits(v[1]) << 16),
                                            bf16_bits(v[2]) | (bf16_bits(v[3]) << 16)};
                            __builtin_amdgcn_raw_buffer_store_b64(w2, rsD, off, 0, 0);
                        }
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const uint32_t off = (mok && n + t < N) ? (rowoff + (uint32_t)(n + t)) * ESZ : OOB;
                            if constexpr (OUT_F32)
                                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v[t]), rsD, off, 0, 0);
                            else
                                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)bf16_bits(v[t]), rsD, off, 0, 0);
                        }
                    }
                }
            }
        }
    };

    if (nk == 0) {   // K == 0: every tile is the empty sum
        for (int j = 0; j < my_tiles; ++j) {
            v16f acc[NB][NB];
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int jb = 0; jb < NB; ++jb) acc[i][jb] = (v16f){};
            epilogue(j, acc);
        }
        return;
    }
    if (NS == 0) return;

    // ---- prologue: stages 0..NSTAGE-1 in flight; stage 0 landed and its fragments read
    cursor_tile();
    for (int g = 0; g < NSTAGE; ++g) {
#pragma unroll
        for (int q = 0; q < LOADS; ++q) dma_item(q);
        advance();
    }
    wait_vmcnt<(NSTAGE - 1) * LOADS>();
    __syncthreads();
    fix_tail(0);
    if constexpr (KTAIL) __syncthreads();

    // Fragment registers are double-buffered: stage g computes from one set
    // while the other receives stage g+1's fragments.
    v8i fa0[NB], fb0[NB], fa1[NB], fb1[NB];
    uint32_t xa[NB] = {}, xb[NB] = {};
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        fa0[i] = frag(0, frag_a0, frag_a1, i);
        fb0[i] = frag(0, frag_b0, frag_b1, i);
    }
    read_scales(0, 0, xa, xb);

    // ---- the stream.  Stage g (fragments and scales in registers):
    //   the 4 matrix-core steps of row block 0;
    //   wait until stage g+1 landed (g+2, g+3 may be in flight) and sync: its
    //   loads landed everywhere, and every wave's reads of buffer g % NSTAGE
    //   (stage g's fragments, read during stage g-1) are done (the barrier
    //   waits for outstanding LDS reads);
    //   12 slots, each one matrix-core step plus one load of stage g+NSTAGE
    //   into buffer g % NSTAGE and two 16-byte LDS reads of stage g+1's
    //   fragments into the other register set.  Spreading the loads keeps the
    //   address unit from blocking the matrix-core steps behind a burst of
    //   loads from all four waves.
    auto stage = [&](v16f (&acc)[NB][NB], int g, int s, const v8i* fa, const v8i* fb, v8i* na,
                     v8i* nbf) __attribute__((always_inline)) {
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) mfma(acc[0][jb], fb[0], fa[jb], xb[0], xa[jb]);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(NSTAGE - 2) * LOADS>();
        __syncthreads();
        if constexpr (KTAIL) {
            fix_tail(g + 1);
            __syncthreads();
        }
        __builtin_amdgcn_sched_barrier(0);
        const int g1 = g + 1;
        const int s1 = (s + 1 == nk) ? 0 : s + 1;
        uint32_t nxa[NB], nxb[NB];
#pragma unroll
        for (int k = 0; k < 12; ++k) {
            const int i = 1 + k / 4, jb = k % 4;
            mfma(acc[i][jb], fb[i], fa[jb], xb[i], xa[jb]);
            if (k < LOADS) dma_item(k);
            // reads in order of first use: row block 0 of B, the four of A, then B 1..3
            if (k == 0) nbf[0] = frag(g1, frag_b0, frag_b1, 0);
            if (k >= 1 && k <= 4) na[k - 1] = frag(g1, frag_a0, frag_a1, k - 1);
            if (k >= 5 && k <= 7) nbf[k - 4] = frag(g1, frag_b0, frag_b1, k - 4);
            if (k == 8) read_scales(g1, s1, nxa, nxb);
            __builtin_amdgcn_sched_barrier(0);
        }
        advance();
        // keep this stage's operand registers allocated to its end
#pragma unroll
        for (int i = 0; i < NB; ++i) asm volatile("" : : "v"(fa[i]), "v"(fb[i]));
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            xa[i] = nxa[i];
            xb[i] = nxb[i];
        }
    };

    int g = 0;
    for (int j = 0; j < my_tiles; ++j) {
        v16f acc[NB][NB];   // [n block][m block]
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) acc[i][jb] = (v16f){};
        int s = 0;
        for (; s + 1 < nk; s += 2, g += 2) {
            stage(acc, g, s, fa0, fb0, fa1, fb1);
            stage(acc, g + 1, s + 1, fa1, fb1, fa0, fb0);
        }
        if (s < nk) {   // odd stage count: the last stage alone, then realign the register sets
            stage(acc, g, s, fa0, fb0, fa1, fb1);
            ++g;
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                fa0[i] = fa1[i];
                fb0[i] = fb1[i];
            }
        }
        epilogue(j, acc);
    }
    wait_vmcnt<0>();   // the past-the-end loads must land before the workgroup exits
}

template <bool MX, bool OUT_F32, bool KTAIL>
static hipError_t launch_one(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                             const float* sa, const float* sb, const uint8_t* ea, const uint8_t* eb, void* D,
                             hipStream_t stream) {
    auto kern = gemm_fp8_kernel<MX, OUT_F32, KTAIL>;
    // 136 KB of dynamic LDS is above the default launch limit; raise it once.
    static std::once_flag once;
    static hipError_t attr_status = hipSuccess;
    std::call_once(once, [&] {
        attr_status = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    });
    if (attr_status != hipSuccess) return attr_status;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
    const int64_t grid = tiles < cus ? tiles : cus;   // persistent: at most one workgroup per CU
    kern<<<dim3((unsigned)grid), dim3(NTHREADS), LDS_BYTES, stream>>>((int)m, (int)n, (int)k, A, B, sa, sb, ea,
                                                                      eb, D);
    return hipGetLastError();
}

template <bool MX>
static hipError_t launch_mode(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                              const float* sa, const float* sb, const uint8_t* ea, const uint8_t* eb, void* D,
                              int out_f32, hipStream_t stream) {
    // mode (a) needs whole 64-byte stages; mode (b) also needs whole 4-byte scale dwords per stage pair
    const bool tail = MX ? (k % (2 * BK)) != 0 : (k % BK) != 0;
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
