// FP8 scaled GEMM on the gfx950 matrix cores, two scaling modes, each operand
// E4M3 or E5M2.
//
//   mode (a)  D[m,n] = sa[m] sb[n] sum_k A[m,k] B[n,k]
//             per-token / per-channel fp32 scales, as the DeepGEMM call on the
//             page "FP8 推理基础设施（五）：从 DeepGEMM 到 vLLM".
//   mode (b)  D[m,n] = sum_j 2^(ea[m,j]-127) 2^(eb[n,j]-127) sum_{t<32} A[m,32j+t] B[n,32j+t]
//             MXFP8: one UE8M0 scale per 32 K elements of every row, as on the
//             page "[sglang] FlashInfer v0.6.7 MXFP8 Gemm 통합", sections 1-2.
//
// Operand formats: the matrix-core instruction takes a format per operand
// (E4M3 = "fp8", E5M2 = "bf8"), so each of A and B may be either; the format
// pair is a template parameter and changes nothing else (a zero byte is +0 in
// both, so the zero-filled K tail is the same).
//
// Both operands are K-major bytes (A [M,K], B [N,K]).  The work is a dense
// contraction (2MNK flops at arithmetic intensity in the thousands), so it is
// bound by the matrix cores, not HBM.
//
// Tiling: a 256-thread workgroup (4 waves, 2x2) owns a 256x256 output tile;
// each wave owns 128x128 = 4x4 blocks of the 32x32 matrix-core tile (256 fp32
// accumulators per lane).  Problems with at most half as many 256x256 tiles as
// CUs use 128x128 tiles instead (waves of 64x64 = 2x2 blocks): four times the
// workgroups, each moving twice the operand bytes per flop, which the idle
// CUs more than pay for.  In mode (a), problems whose 128x128 tiles would
// still fill at most half of the CUs (2048 x 1024: 128 tiles for 256 CUs) use
// 64x128 tiles (waves of 32x64 = 1x2 blocks), unless splitting the 128x128
// tiles over K is predicted faster.  In both modes, 256x128 tiles (waves of
// 128x64 = 4x2 blocks) replace 256x256 ones where those leave a last round
// of workgroups partly empty.
//
// K is walked in 64-byte steps, one V_MFMA_SCALE_F32_32X32X64_F8F6F4 per block
// per step; mode (a) passes the neutral scale code 127 (2^0) and applies sa,
// sb in the epilogue, mode (b) passes the operands' block scales.
//
// Persistent workgroups: one per CU, each walking a list of tiles.  Its
// stages (128 bytes of K, two steps) form one stream across its tiles, so the
// loads of the next tile are in flight while the current tile's epilogue runs.
//
// Operand staging: direct global -> LDS loads (buffer_load_dwordx4 ... lds;
// lane L of a wave writes LDS bytes [M0 + 16L, M0 + 16L + 16)).  A stage moves
// 128 bytes of every row: whole 128-byte lines, which the memory system serves
// at twice the rate of 64-byte pieces of rows (measured: 66 vs 33 bytes per
// clock per CU from L2 for rows 8 KB apart).  Each operand of a stage (256 rows
// x 128 B = 32 KB) is one "item" in a ring of NSLOT LDS slots (5 x 32 KB =
// 160 KB; mode (b) with whole scale dwords uses 4 slots, beside its scales).  One item
// is loaded per K step, its 8 loads spread over that step's matrix-core
// instructions, NSLOT-1 items ahead.  The compiler cannot track these loads
// (it would wait for all of them before every LDS read), so they are issued
// from inline assembly and the kernel waits for them itself; vector-memory
// loads complete in order, so a count of outstanding loads identifies the
// item.  Loads past the end of a panel (rows past M or N, bytes past K) read 0
// (buffer range check on voffset + soffset).
//
// LDS layout of a slot: 256 rows of 128 bytes (eight 16-byte chunks); logical
// chunk c of row r sits in slot c ^ ((r >> 1) & 7).  A 128-bit read serves 16
// lanes per LDS cycle (64 banks, 256 bytes): 16 consecutive rows at one logical
// chunk fall in 16 distinct 16-byte bank groups.  A load instruction fills 8
// rows: lane L takes slot L % 8 of row L / 8 and fetches the chunk stored there.
//
// The matrix core reads a lane's 32 operand bytes as two 16-byte halves:
// bytes 0-15 belong to K block 0 of the 64-wide step and bytes 16-31 to block
// 1; lanes 32-63 hold the upper 16 of each block.  So for step h of a stage a
// lane takes chunks 4h + lhi and 4h + 2 + lhi of its row, and the scale of
// block 0 / 1 of the step comes from lanes 0-31 / 32-63.
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

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace fp8g {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BK = 128;        // bytes of K per stage (two matrix-core steps)
constexpr int KSTEP = 64;      // bytes of K per matrix-core step
constexpr int NTHREADS = 256;
constexpr int NUM_XCD = 8;
constexpr int GROUP_M = 8;

// Tile geometry: a BM x BN output tile per workgroup (BM rows of A, BN rows of
// B), 4 waves in 2x2, each wave WTM x WTN = NBM x NBN blocks of 32x32.  TILE
// names the shape: 256 (256x256), 128 (128x128, for problems with few
// tiles), TILE_64x128 (mode (a), for problems whose 128x128 tiles would leave
// at least half of the CUs idle) or TILE_256x128 (for problems whose 256x256
// tiles leave a last round partly empty).
constexpr int TILE_64x128 = 64128, TILE_256x128 = 256128;
template <int TILE>
struct Geo {
    static constexpr int BM = TILE > 1000 ? TILE / 1000 : TILE, BN = TILE > 1000 ? TILE % 1000 : TILE;
    static constexpr int WTM = BM / 2, WTN = BN / 2;           // wave tile
    static constexpr int NBM = WTM / 32, NBN = WTN / 32;       // blocks per wave tile: 4x4, 2x2, 1x2 or 4x2
    // one operand of one stage (an "item"), and its loads per wave (1 KB per
    // wave instruction, 4 waves)
    static constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
    static constexpr int LA = A_BYTES / 1024 / 4, LB = B_BYTES / 1024 / 4;
};

// Ring geometry per kernel variant.  256-row items: 5 slots of 32 KB fill the
// LDS, so mode (b) with whole scale dwords (scale groups beside the ring)
// fits only 4 slots.  128-row items: mode (a) 8 slots of 16 KB, loads 7 items
// ahead (against 5 slots: 7-10% faster at 2048x1024x4096 and the other
// 128-tile shapes measured; 6 or 7 slots: the same within 2%); mode (b) 5
// (8 slots ran 5% slower there).  64x128 tiles (A items of 8 KB in slots of
// 16 KB): 6 slots, loads 5 items ahead (at 2048x1024x4096: 13.0 us, against
// 16.8 us with 5 slots, 15.0 us with 8 and 16.4 us with 10 slots of 24 KB
// pairs).  256x128 tiles: 3 pairs of a 32 KB A slot and a 16 KB B slot (6
// slots, loads 5 items ahead), in mode (b) and 12 KB of scale groups; the
// epilogue borrows the B slot that is free then.
template <bool MX, bool KTAIL, int TILE>
struct Ring {
    using G = Geo<TILE>;
    static constexpr bool SCALES = MX && !KTAIL;
    static constexpr int NSLOT =
        TILE == 256 ? (SCALES ? 4 : 5) : (TILE == TILE_64x128 || TILE == TILE_256x128) ? 6 : (MX ? 5 : 8);
    // slot k holds items of index k modulo NSLOT; with slots of two sizes
    // (COMPACT: even slots A items, odd ones B items, NSLOT even) each pair is
    // A_BYTES + B_BYTES, otherwise every slot has the larger item's size
    static constexpr bool COMPACT = TILE == TILE_256x128;
    static_assert(!COMPACT || NSLOT % 2 == 0, "ring");
    static constexpr int SLOT = G::B_BYTES > G::A_BYTES ? G::B_BYTES : G::A_BYTES;
    static constexpr int LDS = COMPACT ? NSLOT / 2 * (G::A_BYTES + G::B_BYTES) : NSLOT * SLOT;
    static constexpr int LA = G::LA, LB = G::LB;   // load instructions per item and wave, A and B
    // 4 slots hold two stages: stage g+2 can be loaded only once stage g's
    // slots are free (its step 1), so both its items are issued in that step
    // (none in step 0) to give them the longest lead.  5 or more slots: one
    // item per step, NSLOT-1 items ahead.
    static constexpr bool PAIRED = NSLOT == 4;
    // mode (b) scale groups after the ring: 2 buffers of BM rows of A and BN
    // rows of B x 16 bytes (the scales of SC_GROUP stages)
    static constexpr int SC_GROUP = 4;
    static constexpr int SC_AREA = LDS;
    static constexpr int SC_A = G::BM * 16, SC_B = G::BN * 16;
    static constexpr int SC_BYTES = SCALES ? 2 * (SC_A + SC_B) : 0;
    // epilogue staging (16 KB; in mode (a) also the tile's sa, sb at
    // +16 KB): with 5 slots of 32 KB, or the 16 KB B slots of 256x128 tiles,
    // the slot that is free during the epilogue is borrowed; otherwise
    // (paired, or 16 KB slots) a region of its own.  Mode (a) on 256x128
    // tiles keeps the tile's sa, sb in 2 KB of their own after the ring
    // (TS_SEPARATE, at TS_AREA), since the borrowed B slot holds only the
    // 16 KB of staging.
    static constexpr bool OWN_STAGE = PAIRED || (TILE != 256 && TILE != TILE_256x128);
    static constexpr int STAGE_AREA = LDS + SC_BYTES;
    static constexpr bool TS_SEPARATE = !MX && TILE == TILE_256x128;
    static constexpr int TS_AREA = STAGE_AREA;
    static constexpr int LDS_TOTAL = STAGE_AREA + (OWN_STAGE ? (MX ? 16 : 18) * 1024 : 0) + (TS_SEPARATE ? 2048 : 0);
};
static_assert(Ring<false, false, 256>::LDS_TOTAL <= 160 * 1024 && Ring<true, false, 256>::LDS_TOTAL <= 160 * 1024 &&
                  Ring<true, false, 128>::LDS_TOTAL <= 160 * 1024 && Ring<false, false, 128>::LDS_TOTAL <= 160 * 1024 &&
                  Ring<false, false, TILE_64x128>::LDS_TOTAL <= 160 * 1024 &&
                  Ring<true, false, TILE_256x128>::LDS_TOTAL <= 160 * 1024 &&
                  Ring<false, false, TILE_256x128>::LDS_TOTAL <= 160 * 1024,
              "LDS");

// The share of n items that slot k of s slots takes: one per slot while they
// last when s >= n, else an even split.
__host__ __device__ constexpr int share_lo(int k, int n, int s) { return s >= n ? (k < n ? k : n) : k * n / s; }
__host__ __device__ constexpr int share_hi(int k, int n, int s) { return s >= n ? (k < n ? k + 1 : n) : (k + 1) * n / s; }

constexpr int BUF_DW3 = 0x00020000;   // raw (untyped) buffer descriptor word 3, 32-bit data format
// Cache policy of the staged epilogues' D stores (each store instruction
// writes 8 rows x 128 contiguous bytes): non-temporal.  Every workgroup writes
// its finished tile at about the same time, 4 MB per XCD for a round of
// 256x256 bf16 tiles.  Measured at 8192x22016x8192: 1.4-2% faster in mode
// (a), 3% in mode (b); at N = 22008 (rows not whole lines) still 0.8%
// (write-through, sc0 sc1: no gain).  The L2 miss traffic of the operand loads
// is unchanged (FETCH_SIZE), so the gain is in how the writes drain, not in the
// operands' reuse.  The epilogue from registers (16 bytes or less in each of
// 32 rows per store) keeps the default policy: non-temporal, it ran 30-50%
// slower.
constexpr int ST_NT = 2;

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

// The lane index, computed afresh (v_mbcnt) inside an opaque statement.  Code
// that runs once per tile (epilogues, the tile's scale loads) derives its
// lane-dependent values from this rather than from the kernel's own lane index:
// the compiler then cannot hoist them to the kernel start, where they would
// stay live through the main loop and be spilled.  Each spill reload is a
// scratch load, and the compiler waits for it with a count that does not know
// about the operand loads issued from inline assembly, so it waited for all of
// them too (measured: two such waits per tile).
__device__ __forceinline__ int fresh_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

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

// FA, FB: format code of A and of B (0 = E4M3, 1 = E5M2, as the instruction's
// format fields).  SPLIT (mode (a), K a multiple of 128): the tiles past
// tiles_whole (the last, at most half-full round of tiles) are split over K
// into `split` equal ranges of stages, one work item each; see the split
// reduction below.  ws: the items' fp32 partial tiles, cnt: one arrival
// counter per split tile (zero between launches).
template <bool MX, bool OUT_F32, bool KTAIL, int FA, int FB, int TILE, bool SPLIT>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_fp8_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
    const float* __restrict__ sa, const float* __restrict__ sb, const uint8_t* __restrict__ ea,
    const uint8_t* __restrict__ eb, void* __restrict__ Dv, int tiles_whole, int split, float* __restrict__ ws,
    int* __restrict__ cnt) {
    static_assert(!SPLIT || (!MX && !KTAIL && TILE == 128), "K splits: mode (a), whole stages, 128x128 tiles");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using GEO = Geo<TILE>;
    constexpr int BM = GEO::BM, BN = GEO::BN, WTM = GEO::WTM, WTN = GEO::WTN, NBM = GEO::NBM, NBN = GEO::NBN;
    constexpr int NBX = NBM > NBN ? NBM : NBN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: kept in scalar registers
    const int wm = wave & 1, wn = wave >> 1;
    const int l32 = lane & 31, lhi = lane >> 5;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int total = tiles_m * tiles_n;
    const int nk = (K + BK - 1) / BK;            // stages per tile
    const int nblk = K / 32;                     // MX scale bytes per row

    // ---- this workgroup's work items: XCD x = b % 8 owns a contiguous run of
    // tiles; its W_x workgroups take every W_x-th tile of the run.  SPLIT: only
    // the first tiles_whole tiles are walked so; the split items of the
    // remaining tiles (tile tiles_whole + u, K range s of `split`, item u *
    // split + s) are distributed over the XCDs the same way, at most one per
    // workgroup, after its whole tiles.
    const int G = gridDim.x, b = blockIdx.x;
    const int xcd = b % NUM_XCD, slot = b / NUM_XCD;
    const int wx = (G - xcd + NUM_XCD - 1) / NUM_XCD;                 // workgroups on this XCD
    const int n_whole = SPLIT ? tiles_whole : total;
    const int q = n_whole / NUM_XCD, r = n_whole % NUM_XCD;
    const int run0 = xcd * q + min(xcd, r), runn = q + (xcd < r ? 1 : 0);
    const int my_whole = (slot < runn) ? (runn - slot + wx - 1) / wx : 0;
    int my_split = -1;                                                 // this workgroup's split item, if any
    if constexpr (SPLIT) {
        const int ns = (total - tiles_whole) * split;
        const int q2 = ns / NUM_XCD, r2 = ns % NUM_XCD;
        if (slot < q2 + (xcd < r2 ? 1 : 0)) my_split = xcd * q2 + min(xcd, r2) + slot;
    }
    const int my_tiles = my_whole + (my_split >= 0 ? 1 : 0);          // work items
    const int nks = SPLIT ? nk / split : nk;                           // stages of a split item
    const int NS = my_whole * nk + (my_split >= 0 ? nks : 0);          // stages in this workgroup's stream
    // item j: its tile, first stage (kb) and stages (ns)
    struct Item {
        TileCoord tc;
        int kb, ns;
    };
    auto item_of = [&](int j) __attribute__((always_inline)) -> Item {
        Item it;
        if (!SPLIT || j < my_whole) {
            it.tc = tile_coord(run0 + slot + j * wx, tiles_m, tiles_n);
            it.kb = 0;
            it.ns = nk;
        } else {
            it.tc = tile_coord(tiles_whole + my_split / split, tiles_m, tiles_n);
            it.kb = (my_split % split) * nks;
            it.ns = nks;
        }
        return it;
    };
    auto tile_of = [&](int j) __attribute__((always_inline)) { return item_of(j).tc; };

    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;   // LDS byte address of the stage buffers

    // ---- loads.  Item i of the stream is operand i & 1 (A, B) of stream stage
    // i >> 1; it goes to LDS slot i % NSLOT.  A cursor (tile, stage, operand)
    // walks the items; descriptors change once per tile.  Past the end of the
    // stream the last stage is loaded again (never read), so every K step
    // issues the same number of loads.
    using R = Ring<MX, KTAIL, TILE>;
    constexpr int NSLOT = R::NSLOT, SLOT = R::SLOT, LA = R::LA, LB = R::LB;
    static_assert(!R::PAIRED || LA == LB, "paired ring: square tiles");
    // loads of n consecutive items that start with an A item
    auto loads_of = [](int n) constexpr { return (n + 1) / 2 * LA + n / 2 * LB; };
    // LDS byte offset of ring slot k
    auto slot_off = [&](int k) __attribute__((always_inline)) -> uint32_t {
        if constexpr (!R::COMPACT) return (uint32_t)(k * SLOT);
        else return (uint32_t)((k >> 1) * (GEO::A_BYTES + GEO::B_BYTES) + (k & 1) * GEO::A_BYTES);
    };
    // lane L of wave w, instruction p fills row 32p + 8w + L/8, slot L%8, which
    // holds logical chunk (L%8) ^ ((row >> 1) & 7) = (L%8) ^ ((4w + L/16) & 7)
    const uint32_t dma_chunk = (uint32_t)((lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7));
    const uint32_t dma_voff = (uint32_t)(8 * wave + (lane >> 3)) * (uint32_t)K + dma_chunk * 16u;
    constexpr uint32_t OOB_OFF = 0x80000000u;   // past any panel (panels are < 2^31 bytes)
    int ij = 0, is = 0, iop = 0, ii = 0, islot = 0;   // cursor: work item, stage in it, operand, load item, its slot
    int ikb = 0, ins = nk;                            // the cursor work item's first stage and stages
    __amdgpu_buffer_rsrc_t rsA, rsB;
    auto cursor_tile = [&]() __attribute__((always_inline)) {
        const Item it = item_of(min(ij, my_tiles - 1));
        const TileCoord tc = it.tc;
        ikb = it.kb;
        ins = it.ns;
        const int m0 = tc.tm * BM, n0 = tc.tn * BN;
        const uint32_t rows_a = (uint32_t)min(BM, M - m0), rows_b = (uint32_t)min(BN, N - n0);
        rsA = panel(A + (int64_t)m0 * K, rows_a * (uint32_t)K);
        rsB = panel(B + (int64_t)n0 * K, rows_b * (uint32_t)K);
    };
    // load q (0..LA-1 or 0..LB-1) of the cursor's item
    auto dma_item = [&](int q) __attribute__((always_inline)) {
        const int s_ld = (ii < 2 * NS) ? is : ins - 1;   // past the end: reload the last stage
        const uint32_t sbuf = lds0 + slot_off(islot);
        const uint32_t k0 = (uint32_t)((ikb + s_ld) * BK);
        uint32_t voff = dma_voff;
        if constexpr (KTAIL) {
            // bytes past K (the next row's, or past the panel) must read as 0
            if (k0 + dma_chunk * 16u >= (uint32_t)K) voff = OOB_OFF;
        }
        const uint32_t so = uniform(k0 + (uint32_t)(32 * q) * (uint32_t)K);
        dma16(uniform(sbuf + (uint32_t)((4 * q + wave) * 1024)), voff, iop ? rsB : rsA, so);
    };

    // ---- mode (b) scale groups (whole scale dwords, K % 128 == 0).  Group gi
    // of a tile covers its stages 4gi .. 4gi+3: bytes 16gi .. 16gi+15 of every
    // scale row.  Stream group number u (tile j: u = j * ngt + gi) goes to
    // buffer u & 1 at SC_AREA + (u & 1) (SC_A + SC_B), A's rows first, then
    // B's (sc_area): row r in the 16 bytes at 16 r, the dword of group stage t at position
    // (t + (r >> 3)) & 3 (rotated so that the 32 rows of one scale read fall in
    // distinct banks).  Load p of an operand fills rows 16p .. 16p+15, lane L
    // row 16p + L/4 at position L % 4: 16 bytes of a row in one or two lines,
    // where loading each stage's dword alone touches a line per row per stage.
    // Wave w issues loads p = w, w+4, ... of both operands: SC_LA of A, then
    // SC_LB of B.
    constexpr int SC_LA = R::SCALES ? BM / 16 / 4 : 0, SC_LB = R::SCALES ? BN / 16 / 4 : 0;
    constexpr int SC_LOADS = SC_LA + SC_LB;   // per wave and group: 8, 4 or 6
    // LDS byte offset of buffer ub's scale rows of operand o
    auto sc_area = [](int ub, int o) constexpr -> int {
        if constexpr (R::SC_A == R::SC_B) return R::SC_AREA + 2 * ub * R::SC_A + o * R::SC_A;
        else return R::SC_AREA + ub * (R::SC_A + R::SC_B) + o * R::SC_A;
    };
    const int ngt = (nk + R::SC_GROUP - 1) / R::SC_GROUP;            // groups per tile
    const uint32_t sc_voff = (uint32_t)(16 * wave + (lane >> 2)) * (uint32_t)nblk +
                             4u * (((uint32_t)(lane & 3) - (uint32_t)(2 * wave + (lane >> 5))) & 3u);
    __amdgpu_buffer_rsrc_t rsEA, rsEB;   // scale panels of the tile of the group loaded last
    auto sc_tile = [&](int j) __attribute__((always_inline)) {
        const TileCoord tc = tile_of(j);
        const int m0 = tc.tm * BM, n0 = tc.tn * BN;
        rsEA = panel(ea + (int64_t)m0 * nblk, (uint32_t)min(BM, M - m0) * (uint32_t)nblk);
        rsEB = panel(eb + (int64_t)n0 * nblk, (uint32_t)min(BN, N - n0) * (uint32_t)nblk);
    };
    // load q (0 .. SC_LOADS-1) of group gi (of the tile of rsEA, rsEB) into buffer ub
    auto sc_load = [&](int q, int gi, int ub) __attribute__((always_inline)) {
        if constexpr (R::SCALES) {
            if constexpr (R::SC_A == R::SC_B) {
                constexpr int PER_OP = SC_LOADS / 2;
                const int o = q / PER_OP, p = wave + 4 * (q % PER_OP);
                const uint32_t dst = lds0 + (uint32_t)(R::SC_AREA + (2 * ub + o) * R::SC_A + 256 * p);
                dma4(uniform(dst), sc_voff, o ? rsEB : rsEA,
                     uniform((uint32_t)(16 * gi) + (uint32_t)(64 * (q % PER_OP)) * (uint32_t)nblk));
            } else {
                const int o = q < SC_LA ? 0 : 1, idx = o ? q - SC_LA : q, p = wave + 4 * idx;
                const uint32_t dst = lds0 + (uint32_t)(sc_area(ub, o) + 256 * p);
                dma4(uniform(dst), sc_voff, o ? rsEB : rsEA,
                     uniform((uint32_t)(16 * gi) + (uint32_t)(64 * idx) * (uint32_t)nblk));
            }
        }
    };
    auto advance = [&]() __attribute__((always_inline)) {
        ++ii;
        islot = (islot + 1 == NSLOT) ? 0 : islot + 1;
        if (++iop == 2) {
            iop = 0;
            if (++is == ins) {
                is = 0;
                ++ij;
                cursor_tile();
            }
        }
    };

    // ---- fragment reads: step h of the stage whose items sit in LDS slots
    // sa_off (A) and sb_off (B); this lane's rows, chunks 4h + lhi and 4h + 2 + lhi
    const uint32_t key = (uint32_t)((l32 >> 1) & 7);
    const uint32_t frag_a = (uint32_t)((wm * WTM + l32) * BK);
    const uint32_t frag_b = (uint32_t)((wn * WTN + l32) * BK);
    const uint32_t c0 = ((uint32_t)lhi ^ key) << 4, c1 = ((uint32_t)(2 + lhi) ^ key) << 4;
    auto frag = [&](uint32_t slot_off, uint32_t row_off, int h, int i) __attribute__((always_inline)) -> v8i {
        const uint8_t* p = smem + slot_off + row_off + i * 32 * BK;
        const v4u x0 = *reinterpret_cast<const v4u*>(p + (c0 ^ (uint32_t)(64 * h)));
        const v4u x1 = *reinterpret_cast<const v4u*>(p + (c1 ^ (uint32_t)(64 * h)));
        return (v8i){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    };
    // slot index + k, modulo NSLOT (k < NSLOT)
    auto slot_add = [&](int slot, int k) __attribute__((always_inline)) -> int {
        return (slot + k >= NSLOT) ? slot + k - NSLOT : slot + k;
    };

    // ---- mode (b) scales for step h of stage s of stream tile j: per lane and
    // row block, the scale byte of this lane half's block in byte 0 (the matrix
    // core reads byte 0).  With whole scale dwords: the stage's dword (blocks
    // 4s .. 4s+3) from the LDS scale group.  Otherwise (rows of nblk bytes, not
    // a multiple of 4): unconditional byte loads from global, 2^0 past the row
    // end; rows past M / N read 0 (their data is zero too).  j < my_tiles.
    auto read_scales = [&](int j, int s, int h, uint32_t* xa, uint32_t* xb) __attribute__((always_inline)) {
        if constexpr (MX) {
            if constexpr (R::SCALES) {
                // the stage's dword holds the scales of its 4 blocks; shifted by
                // this lane half, byte 2h is step h's block (selected in the
                // matrix-core instruction), so one read serves both steps.  The
                // lane-dependent parts come from a fresh lane index: kept live
                // from the kernel start they were spilled.
                const int ln = fresh_lane();
                const int l32s = ln & 31;
                const uint32_t sh = (uint32_t)(8 * (ln >> 5));
                const int ub = (j * ngt + s / R::SC_GROUP) & 1;
                const uint8_t* sca;
                const uint8_t* scb;
                if constexpr (R::SC_A == R::SC_B) {
                    sca = smem + R::SC_AREA + 2 * ub * R::SC_A;
                    scb = sca + R::SC_A;
                } else {
                    sca = smem + sc_area(ub, 0);
                    scb = smem + sc_area(ub, 1);
                }
                // row wm*WTM + 32i + l32: (row >> 3) & 3 == (l32 >> 3) & 3
                const uint32_t pos = (((uint32_t)(s & 3) + (uint32_t)(l32s >> 3)) & 3u) * 4u;
#pragma unroll
                for (int i = 0; i < NBX; ++i) {
                    if (i < NBM)
                        xa[i] = *reinterpret_cast<const uint32_t*>(sca + (wm * WTM + i * 32 + l32s) * 16 + pos) >> sh;
                    if (i < NBN)
                        xb[i] = *reinterpret_cast<const uint32_t*>(scb + (wn * WTN + i * 32 + l32s) * 16 + pos) >> sh;
                }
            } else {
                const TileCoord tc = tile_of(j);
                const int m0 = tc.tm * BM, n0 = tc.tn * BN;
                const __amdgpu_buffer_rsrc_t pa = panel(ea + (int64_t)m0 * nblk, (uint32_t)min(BM, M - m0) * (uint32_t)nblk);
                const __amdgpu_buffer_rsrc_t pb = panel(eb + (int64_t)n0 * nblk, (uint32_t)min(BN, N - n0) * (uint32_t)nblk);
                const int kb = 4 * s + 2 * h + lhi;   // this lane half's block
                const bool in = kb < nblk;
                const uint32_t kc = (uint32_t)min(kb, nblk - 1);
#pragma unroll
                for (int i = 0; i < NBX; ++i) {
                    if (i < NBM) {
                        const uint32_t va = __builtin_amdgcn_raw_buffer_load_b8(
                            pa, (uint32_t)(wm * WTM + i * 32 + l32) * (uint32_t)nblk + kc, 0, 0);
                        xa[i] = in ? va : 127u;
                    }
                    if (i < NBN) {
                        const uint32_t vb = __builtin_amdgcn_raw_buffer_load_b8(
                            pb, (uint32_t)(wn * WTN + i * 32 + l32) * (uint32_t)nblk + kc, 0, 0);
                        xb[i] = in ? vb : 127u;
                    }
                }
            }
        }
    };

    // The empty asm after each step pins it where it is written: the builtin has
    // no side effects, so without it the optimizer may sink whole stages of
    // steps past later barriers, leaving the matrix core idle in between.
    // The instruction's first operand is fed from B's rows, so its format
    // field is FB and the second one's FA.
    // OPS: the byte of each scale register that holds this lane's block scale
    auto mfma = [&](v16f& c, const v8i& fbi, const v8i& faj, uint32_t sbi, uint32_t saj, auto ops_tag)
                    __attribute__((always_inline)) {
        constexpr int OPS = decltype(ops_tag)::value;
        if constexpr (MX)
            c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fbi, faj, c, FB, FA, OPS, (int)sbi, OPS, (int)saj);
        else
            c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fbi, faj, c, FB, FA, 0, 127, 0, 127);
        asm volatile("" : "+a"(c));
    };

    // ---- epilogue of stream tile j from registers (where no staged epilogue applies):
    // lane holds m = .. + l32 and n = .. + 8g + 4*lhi + t (t = 0..3) in
    // acc[.][.][4g+t].  Stores over the tile's rows of D: out-of-range lanes get
    // an offset past the end, which the hardware drops.  Mode (a) reads the
    // tile's sa, sb from LDS at stage_off + 16 KB / + 17 KB (loaded by
    // tile_scales_to_lds during the tile's last K step, like the staged
    // epilogue): loaded here into registers, the compiler's wait for them would
    // also wait for the next tile's operand loads in flight.
    constexpr int ESZ = OUT_F32 ? 4 : 2;
    constexpr uint32_t SC_OFF = 16384;   // the tile's sa at stage_off + 16 KB, sb at + 17 KB
    // LDS offset of the tile's sa (sb 1 KB after it) for the staging region at stage_off
    auto ts_off = [&](uint32_t stage_off) __attribute__((always_inline)) -> uint32_t {
        if constexpr (R::TS_SEPARATE) return (uint32_t)R::TS_AREA;
        else return stage_off + SC_OFF;
    };
    auto epilogue = [&](int j, v16f (&acc)[NBN][NBM], uint32_t stage_off) __attribute__((always_inline)) {
        const TileCoord tc = tile_of(j);
        const int m0 = tc.tm * BM, n0 = tc.tn * BN;
        const uint32_t rows = (uint32_t)min(BM, M - m0);
        const __amdgpu_buffer_rsrc_t rsD =
            panel(reinterpret_cast<uint8_t*>(Dv) + (int64_t)m0 * N * ESZ, rows * (uint32_t)N * ESZ);
        constexpr uint32_t OOB = 0x80000000u;   // beyond any panel (panels are < 2^31 bytes)
        const int lane_u = fresh_lane();
        const int l32 = lane_u & 31, lhi = lane_u >> 5;
        const float* lsa = reinterpret_cast<const float*>(smem + ts_off(stage_off));
        const float* lsb = reinterpret_cast<const float*>(smem + ts_off(stage_off) + 1024);
        float smv[NBM], snv[NBN][4][4];
#pragma unroll
        for (int jb = 0; jb < NBM; ++jb) {
            smv[jb] = 1.0f;
            if constexpr (!MX) smv[jb] = lsa[wm * WTM + jb * 32 + l32];   // rows past M hold 0 (and are not stored)
        }
#pragma unroll
        for (int i = 0; i < NBN; ++i)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                if constexpr (!MX) {
                    // a float vector: __builtin_bit_cast of an element of an integer
                    // vector reads element 0 whatever the index (clang)
                    const v4f t4 = *reinterpret_cast<const v4f*>(lsb + wn * WTN + i * 32 + 8 * gq + 4 * lhi);
#pragma unroll
                    for (int t = 0; t < 4; ++t) snv[i][gq][t] = t4[t];
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) snv[i][gq][t] = 1.0f;
                }
            }
        __builtin_amdgcn_sched_barrier(0);
        const bool vec_ok = (N % 4) == 0;
#pragma unroll
        for (int jb = 0; jb < NBM; ++jb) {
            const int mr = wm * WTM + jb * 32 + l32;          // row inside the tile
            const bool mok = m0 + mr < M;
            const uint32_t rowoff = (uint32_t)mr * (uint32_t)N;
#pragma unroll
            for (int i = 0; i < NBN; ++i) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int n = n0 + wn * WTN + i * 32 + 8 * gq + 4 * lhi;
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
                            const v2u w2 = {bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3])};
                            __builtin_amdgcn_raw_buffer_store_b64(w2, rsD, off, 0, 0);
                        }
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const uint32_t off = (mok && n + t < N) ? (rowoff + (uint32_t)(n + t)) * ESZ : OOB;
                            if constexpr (OUT_F32)
                                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v[t]), rsD, off, 0, 0);
                            else
                                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)bf16x2_bits(v[t], 0.0f), rsD, off, 0, 0);
                        }
                    }
                }
            }
        }
    };

    // ---- bf16 epilogue through LDS (N % 8 == 0), in a free 32 KB region at
    // stage_off: the tile's sa, sb sit at stage_off + 16 KB / + 17 KB (loaded by
    // tile_scales_to_lds); each wave stages bands of 32 rows x 64 columns (4 KB,
    // one 128-byte line per row) in its own 4 KB, reads them back row-contiguous
    // and stores 16 bytes per lane, 8 rows x 128 bytes (whole lines) per
    // instruction.  A store instruction that touches 32 rows at 16 bytes each
    // runs about 8x slower.  Band layout: 32 rows of 128 bytes, logical 16-byte
    // chunk c of row r in physical chunk c ^ ((r >> 1) & 7), its 8-byte halves
    // swapped when r >= 16: the 8-byte writes of 32 rows and the 16-byte reads of
    // 2 rows per LDS cycle both hit distinct banks.
    auto tile_scales_to_lds = [&](int j, uint32_t stage_off) __attribute__((always_inline)) {
        if constexpr (!MX) {
            const TileCoord tc = tile_of(j);
            const int m0 = tc.tm * BM, n0 = tc.tn * BN;
            const uint32_t v = (uint32_t)(64 * wave + fresh_lane()) * 4u;   // lane L of wave w: element 64w + L
            dma4(uniform(lds0 + ts_off(stage_off) + (uint32_t)(wave * 256)), v,
                 panel(sa + m0, (uint32_t)min(BM, M - m0) * 4u), 0u);
            dma4(uniform(lds0 + ts_off(stage_off) + 1024u + (uint32_t)(wave * 256)), v,
                 panel(sb + n0, (uint32_t)min(BN, N - n0) * 4u), 0u);
        }
    };
    auto epilogue_staged = [&](int j, v16f (&acc)[NBN][NBM], uint32_t stage_off) __attribute__((always_inline)) {
        const TileCoord tc = tile_of(j);
        const int m0 = tc.tm * BM, n0 = tc.tn * BN;
        const uint32_t rows = (uint32_t)min(BM, M - m0);
        const __amdgpu_buffer_rsrc_t rsD =
            panel(reinterpret_cast<uint8_t*>(Dv) + (int64_t)m0 * N * 2, rows * (uint32_t)N * 2u);
        constexpr uint32_t OOB = 0x80000000u;
        const int lane_e = fresh_lane();
        const int l32e = lane_e & 31, lhie = lane_e >> 5;
        uint8_t* st = smem + stage_off + wave * 4096;
        const float* lsa = reinterpret_cast<const float*>(smem + ts_off(stage_off));
        const float* lsb = reinterpret_cast<const float*>(smem + ts_off(stage_off) + 1024);
        const uint32_t wkey = (uint32_t)((l32e >> 1) & 7), whalf = (uint32_t)(lhie ^ (l32e >> 4));
        // rows past M need no check: the descriptor covers exactly the tile's rows
        // of D, and offsets past it are dropped
        const uint32_t rc = (uint32_t)(lane_e & 7);        // read-back: 16-byte chunk of the lane
        const int rr = lane_e >> 3;                          // read-back: row within 8
        const uint32_t rd_off = (uint32_t)(rr * 128) + ((rc ^ (uint32_t)((rr >> 1) & 3)) << 4);
#pragma unroll
        for (int ih = 0; ih < NBN / 2; ++ih) {     // 64-column part of the wave tile: blocks i = 2ih, 2ih+1
            float snv[2][4][4];
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    if constexpr (!MX) {
                        // a float vector: __builtin_bit_cast of an element of an integer
                        // vector reads element 0 whatever the index (clang)
                        const v4f t4 = *reinterpret_cast<const v4f*>(lsb + wn * WTN + (2 * ih + ii) * 32 + 8 * gq + 4 * lhie);
#pragma unroll
                        for (int t = 0; t < 4; ++t) snv[ii][gq][t] = t4[t];
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t) snv[ii][gq][t] = 1.0f;
                    }
                }
#pragma unroll
            for (int jb = 0; jb < NBM; ++jb) {
                float smv = 1.0f;
                if constexpr (!MX) smv = lsa[wm * WTM + jb * 32 + l32e];
#pragma unroll
                for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        float v[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) v[t] = acc[2 * ih + ii][jb][4 * gq + t] * smv * snv[ii][gq][t];
                        typedef unsigned int v2u __attribute__((ext_vector_type(2)));
                        const v2u w2 = {bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3])};
                        const uint32_t pc = (uint32_t)(4 * ii + gq) ^ wkey;
                        *reinterpret_cast<v2u*>(st + l32e * 128 + pc * 16 + whalf * 8) = w2;
                    }
                const int n = n0 + wn * WTN + 64 * ih + 8 * (int)rc;
                // branch-free select (a compare-and-select here becomes a branch)
                uint32_t keep = n < N ? 0xFFFFFFFFu : 0u;
                asm volatile("" : "+v"(keep));
                const uint32_t col_off = (uint32_t)n * 2u;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    // band row r = 8k + rr: (r >> 1) & 7 = 4k + (rr >> 1) (mod 8), so the
                    // physical chunk is rc ^ ((rr >> 1) & 3) ^ 4 (k & 1)
                    v4u d = *reinterpret_cast<const v4u*>(st + k * 1024 + (rd_off ^ (uint32_t)(64 * (k & 1))));
                    if (k >= 2) d = (v4u){d.z, d.w, d.x, d.y};   // rows 16..31: halves swapped
                    const uint32_t mr = (uint32_t)(wm * WTM + jb * 32 + 8 * k + rr);   // row inside the tile
                    const uint32_t off = mr * (uint32_t)N * 2u + col_off;
                    __builtin_amdgcn_raw_buffer_store_b128(d, rsD, (off & keep) | (OOB & ~keep), 0, ST_NT);
                }
            }
        }
    };
    // ---- fp32 epilogue through LDS (mode (a), N % 32 == 0): as the bf16 one, with bands of
    // one 32x32 block (32 rows x 128 bytes, 4 KB per wave).  Lane (l32, lhi)
    // writes the 16-byte chunks 2 gq + lhi (gq = 0..3) of band row l32, logical
    // chunk c of row r at physical chunk c ^ ((r >> 1) & 7): the writes of 16
    // lanes (16 rows, one chunk) and the reads of 16 lanes (2 rows, 8 chunks)
    // both hit 16 distinct 16-byte bank groups.  Read back row-contiguously, 8
    // lanes store one 128-byte row of the band, as whole lines.
    auto epilogue_staged_f32 = [&](int j, v16f (&acc)[NBN][NBM], uint32_t stage_off) __attribute__((always_inline)) {
        const TileCoord tc = tile_of(j);
        const int m0 = tc.tm * BM, n0 = tc.tn * BN;
        const uint32_t rows = (uint32_t)min(BM, M - m0);
        const __amdgpu_buffer_rsrc_t rsD =
            panel(reinterpret_cast<uint8_t*>(Dv) + (int64_t)m0 * N * 4, rows * (uint32_t)N * 4u);
        constexpr uint32_t OOB = 0x80000000u;
        const int lane_e = fresh_lane();
        const int l32e = lane_e & 31, lhie = lane_e >> 5;
        uint8_t* st = smem + stage_off + wave * 4096;
        const float* lsa = reinterpret_cast<const float*>(smem + ts_off(stage_off));
        const float* lsb = reinterpret_cast<const float*>(smem + ts_off(stage_off) + 1024);
        const uint32_t wkey = (uint32_t)((l32e >> 1) & 7);
        // rows past M need no check: the descriptor covers exactly the tile's rows
        // of D, and offsets past it are dropped
        const uint32_t rc = (uint32_t)(lane_e & 7);        // read-back: 16-byte chunk of the lane
        const int rr = lane_e >> 3;                          // read-back: row within 8
        const uint32_t rd_off = (uint32_t)(rr * 128) + ((rc ^ (uint32_t)((rr >> 1) & 3)) << 4);
#pragma unroll
        for (int i = 0; i < NBN; ++i) {     // 32-column block of the wave tile
            float snv[4][4];
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                if constexpr (!MX) {
                    const v4f t4 = *reinterpret_cast<const v4f*>(lsb + wn * WTN + i * 32 + 8 * gq + 4 * lhie);
#pragma unroll
                    for (int t = 0; t < 4; ++t) snv[gq][t] = t4[t];
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) snv[gq][t] = 1.0f;
                }
            }
            const int n = n0 + wn * WTN + 32 * i + 4 * (int)rc;
            // branch-free select (a compare-and-select here becomes a branch)
            uint32_t keep = n < N ? 0xFFFFFFFFu : 0u;
            asm volatile("" : "+v"(keep));
            const uint32_t col_off = (uint32_t)n * 4u;
#pragma unroll
            for (int jb = 0; jb < NBM; ++jb) {
                float smv = 1.0f;
                if constexpr (!MX) smv = lsa[wm * WTM + jb * 32 + l32e];
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    v4f w4;
#pragma unroll
                    for (int t = 0; t < 4; ++t) w4[t] = acc[i][jb][4 * gq + t] * smv * snv[gq][t];
                    const uint32_t pc = (uint32_t)(2 * gq + lhie) ^ wkey;
                    *reinterpret_cast<v4f*>(st + l32e * 128 + pc * 16) = w4;
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    // band row r = 8k + rr: (r >> 1) & 7 = 4k + (rr >> 1) (mod 8), so the
                    // physical chunk is rc ^ ((rr >> 1) & 3) ^ 4 (k & 1)
                    const v4u d = *reinterpret_cast<const v4u*>(st + k * 1024 + (rd_off ^ (uint32_t)(64 * (k & 1))));
                    const uint32_t mr = (uint32_t)(wm * WTM + jb * 32 + 8 * k + rr);   // row inside the tile
                    const uint32_t off = mr * (uint32_t)N * 4u + col_off;
                    __builtin_amdgcn_raw_buffer_store_b128(d, rsD, (off & keep) | (OOB & ~keep), 0, ST_NT);
                }
                // one block at a time: interleaved across blocks, the schedule kept
                // too many values live and spilled
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // Staged epilogues: bf16 for N % 8 == 0; fp32 in mode (a) for N % 32 == 0,
    // rows of whole 128-byte lines (at N = 22012, rows straddling lines, staged
    // fp32 ran 4% slower than from registers; mode (b) with fp32 output staged
    // spilled in its main loop)
    const bool staged = OUT_F32 ? (!MX && (N % 32) == 0) : (N % 8) == 0;
    auto epilogue_staged_any = [&](int j, v16f (&acc)[NBN][NBM], uint32_t stage_off) __attribute__((always_inline)) {
        if constexpr (OUT_F32) epilogue_staged_f32(j, acc, stage_off);
        else epilogue_staged(j, acc, stage_off);
    };

    // ---- split reduction (SPLIT: the workgroup's split item, after its last K
    // step).  Every split item stores its fp32 partial tile to ws (item
    // u * split + s; per wave and block 4 KB: accumulators 4c .. 4c+3 of lane
    // L at 1024 c + 16 L, so that every store covers 1 KB in whole lines) and,
    // once those stores have completed, counts itself
    // in cnt[u].  The item that arrives last (count split - 1) reads the other
    // partials and adds all of them in split order, p0 + p1 + ..., its own
    // from registers, so the sum does not depend on the order of arrival; it
    // resets cnt[u] to zero for the next launch and returns true: its
    // workgroup stores the tile.  No workgroup waits for another.
    // Coherence across the XCDs' separate L2 caches comes from the accesses
    // themselves, not from fences: the partials are stored and loaded with
    // device scope (SC1: written through to, and read from, the level all XCDs
    // share) and the counter is a device-scope atomic.  A device-scope fence
    // would instead write back and invalidate the whole L2 of the XCD, taking
    // every other workgroup's operand panels with it (measured: the 2048 x
    // 1024 x 4096 GEMM ran 3.6x slower so).  The LDS word at stage_off (the
    // epilogue's staging area, free here) passes the count to all waves.
    constexpr int CP_SC1 = 16;   // cache policy of the buffer builtins: device scope
    auto split_reduce = [&](v16f (&acc)[NBN][NBM], uint32_t stage_off) __attribute__((always_inline)) -> bool {
        const int u = my_split / split, sidx = my_split % split;
        const int ln = fresh_lane();
        constexpr uint32_t PART = BM * BN * 4;   // bytes per partial tile
        const __amdgpu_buffer_rsrc_t rw = panel(reinterpret_cast<uint8_t*>(ws) + (size_t)my_split * PART, PART);
#pragma unroll
        for (int i = 0; i < NBN; ++i)
#pragma unroll
            for (int jb = 0; jb < NBM; ++jb) {
                const uint32_t off = (uint32_t)((wave * NBN * NBM + i * NBM + jb) * 4096 + ln * 16);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(v4u, (v4f){acc[i][jb][4 * c], acc[i][jb][4 * c + 1], acc[i][jb][4 * c + 2],
                                                      acc[i][jb][4 * c + 3]}),
                        rw, off + 1024 * c, 0, CP_SC1);
            }
        asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // this wave's partial is visible device-wide
        __syncthreads();
        int* flag = reinterpret_cast<int*>(smem + stage_off);
        if (tid == 0) {
            const int old = __hip_atomic_fetch_add(cnt + u, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *flag = (old == split - 1) ? 1 : 0;
        }
        __syncthreads();
        const bool last = *flag != 0;
        __syncthreads();   // every wave has read the flag before that LDS is used again
        if (!last) return false;
        const __amdgpu_buffer_rsrc_t rr =
            panel(reinterpret_cast<uint8_t*>(ws) + (size_t)(u * split) * PART, PART * (uint32_t)split);
        auto load16 = [&](uint32_t off) __attribute__((always_inline)) -> v16f {
            const v4f a = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, CP_SC1));
            const v4f b4 = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rr, off + 1024, 0, CP_SC1));
            const v4f c = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rr, off + 2048, 0, CP_SC1));
            const v4f d = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rr, off + 3072, 0, CP_SC1));
            return (v16f){a.x, a.y, a.z, a.w, b4.x, b4.y, b4.z, b4.w, c.x, c.y, c.z, c.w, d.x, d.y, d.z, d.w};
        };
        // the split count as a constant, so that every partial's loads of a
        // block are issued together (a runtime loop waited for each in turn)
        auto add_parts = [&](auto s_tag) __attribute__((always_inline)) {
            constexpr int S = decltype(s_tag)::value;
#pragma unroll
            for (int i = 0; i < NBN; ++i)
#pragma unroll
                for (int jb = 0; jb < NBM; ++jb) {
                    const uint32_t off = (uint32_t)((wave * NBN * NBM + i * NBM + jb) * 4096 + ln * 16);
                    v16f p[S];
#pragma unroll
                    for (int s2 = 0; s2 < S; ++s2)
                        if (s2 != sidx) p[s2] = load16(s2 * PART + off);
                    v16f t = sidx == 0 ? acc[i][jb] : p[0];
#pragma unroll
                    for (int s2 = 1; s2 < S; ++s2) t += s2 == sidx ? acc[i][jb] : p[s2];
                    acc[i][jb] = t;
                }
        };
        if (split == 2) add_parts(std::integral_constant<int, 2>{});
        else if (split == 3) add_parts(std::integral_constant<int, 3>{});
        else add_parts(std::integral_constant<int, 4>{});
        if (tid == 0) __hip_atomic_store(cnt + u, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    };

    if (nk == 0) {   // K == 0: every tile is the empty sum
        for (int j = 0; j < my_tiles; ++j) {
            v16f acc[NBN][NBM];
#pragma unroll
            for (int i = 0; i < NBN; ++i)
#pragma unroll
                for (int jb = 0; jb < NBM; ++jb) acc[i][jb] = (v16f){};
            tile_scales_to_lds(j, 0);
            wait_vmcnt<0>();
            __syncthreads();
            if (staged) epilogue_staged_any(j, acc, 0);
            else epilogue(j, acc, 0);
            __syncthreads();
        }
        return;
    }
    if (NS == 0) return;

    // ---- prologue: items 0 .. NSLOT-2 in flight; stage 0 (items 0, 1) and the
    // first scale group (loaded before them) landed, and the fragments and
    // scales of step 0 read
    cursor_tile();
    if constexpr (R::SCALES) {
        sc_tile(0);
#pragma unroll
        for (int q = 0; q < SC_LOADS; ++q) sc_load(q, 0, 0);
    }
    constexpr int PRO_ITEMS = R::PAIRED ? 4 : NSLOT - 1;   // items in flight before step 0
    for (int i = 0; i < PRO_ITEMS; ++i) {
        const int nq = (i & 1) ? LB : LA;   // item i is operand i & 1
#pragma unroll
        for (int q = 0; q < nq; ++q) dma_item(q);
        advance();
    }
    wait_vmcnt<loads_of(PRO_ITEMS - 2)>();
    __syncthreads();

    // Fragment registers are double-buffered: step t computes from one set
    // while the other receives step t+1's fragments.
    v8i fa0[NBM], fb0[NBN], fa1[NBM], fb1[NBN];
    uint32_t xa[NBM] = {}, xb[NBN] = {};
#pragma unroll
    for (int i = 0; i < NBX; ++i) {
        if (i < NBM) fa0[i] = frag(0, frag_a, 0, i);
        if (i < NBN) fb0[i] = frag(slot_off(1), frag_b, 0, i);
    }
    read_scales(0, 0, 0, xa, xb);
    int rslot = 0;   // LDS slot of the current stage's A item (its B item is the next slot)

    // ---- one K step: step h of stage s of stream tile j (fragments and scales
    // in registers).
    //   the NBM matrix-core steps of row block 0 (4 for 256-row tiles);
    //   h == 1 only: wait until the next stage's items landed (items past them
    //   may be in flight) and sync: they landed for every wave, and every wave's
    //   reads of this stage's items (done during step 0) are finished (the
    //   barrier waits for outstanding LDS reads), so their slots may be refilled;
    //   the remaining (NBN-1)·NBM matrix-core steps ("slots": 12 for 256x256
    //   tiles), each with its share of the loads of the item NSLOT-1 ahead
    //   (into the slot of the item just before this step's) and of the next
    //   step's fragment reads (two 16-byte LDS reads each) into the other
    //   register set.  Spreading the loads keeps the address unit from blocking the
    //   matrix-core steps behind a burst of loads from all four waves.
    //   LAST (the tile's last step): no reads of the next step's fragments (they
    //   are read after the epilogue, which then has their registers to itself).
    // matrix-core steps after row block 0: 12 for 256x256 tiles, 4 for
    // 256x128, 2 for 128x128 and 1 for 64x128; the step's loads and the next
    // step's NBM + NBN fragment reads are spread over them.
    // Mode (b) scales from LDS (once per stage, in its step 1, for the next
    // stage) are read first, in slot 0: LDS reads complete in order, so scales
    // read after the fragments would hold the next step's first matrix-core
    // instruction until every fragment read had landed.
    // Scales loaded byte-wise from global memory (K tail) are read after the
    // step's item loads instead.
    // Mode (b) scale groups: step 0 of a group's first stage loads the next
    // group (the tile's next, or the next tile's first) into the other buffer,
    // whose group was last read in step 0 of the stage before, ahead of the
    // barrier of that stage's step 1.  The paired ring spreads the loads over
    // this step, which loads no items; with 5 or more slots they go first,
    // before the item loads, which the next wait may leave in flight.  Either way they
    // have landed at that wait, the earliest point the group is read.
    constexpr int SLOTS = (NBN - 1) * NBM;
    constexpr int NREAD = NBM + NBN;
    static_assert(SLOTS >= 1, "a matrix-core slot after row block 0");
    constexpr int SCALE_SLOT = R::SCALES ? 0 : (SLOTS > NREAD ? NREAD + 1 : SLOTS - 1);
    // With NSLOT >= 5 slots the ring runs NSLOT - 1 items ahead, one item per
    // step, so step h of every stage loads an item of operand (h + NSLOT - 1) & 1
    // (A: LA loads, B: LB).  LI_LAST: the loads of a stage's step 1 (mode (a)).
    constexpr int LI_LAST = (NSLOT & 1) ? LB : LA;
    auto kstep = [&](v16f (&acc)[NBN][NBM], int j, int s, auto h_tag, auto last_tag, const v8i* fa, const v8i* fb,
                     v8i* na, v8i* nbf) __attribute__((always_inline)) {
        constexpr int h = decltype(h_tag)::value;
        constexpr bool LAST = decltype(last_tag)::value;
        using Ops = std::integral_constant<int, R::SCALES ? 2 * h : 0>;
        constexpr int LI_STEP = ((h + NSLOT - 1) & 1) ? LB : LA;   // this step's loads (unpaired ring)
        // whole scale dwords are read once per stage, in its step 1 for the next stage
        constexpr bool READ_SC = !R::SCALES || h == 1;
        bool sc_go = false;
        int sc_gi = 0, sc_ub = 0;
        if constexpr (R::SCALES) {
            if (h == 0 && s % R::SC_GROUP == 0) {
                const bool in_tile = s + R::SC_GROUP < nk;
                if (in_tile || j + 1 < my_tiles) {
                    if (!in_tile) sc_tile(j + 1);
                    sc_go = true;
                    sc_gi = in_tile ? s / R::SC_GROUP + 1 : 0;
                    sc_ub = (j * ngt + s / R::SC_GROUP + 1) & 1;
                }
            }
        }
#pragma unroll
        for (int jb = 0; jb < NBM; ++jb) mfma(acc[0][jb], fb[0], fa[jb], xb[0], xa[jb], Ops{});
        if (h == 1) {
            __builtin_amdgcn_sched_barrier(0);
            // the next stage's items landed: with NSLOT >= 5 slots the NSLOT-4
            // items issued after them may be in flight; with 4 (paired) none
            wait_vmcnt<R::PAIRED ? 0 : loads_of(NSLOT - 4)>();
            __syncthreads();
            // last stage of a tile: the slot of its B item is now free until the
            // next tile's first step; load the tile's scales into it for the
            // epilogue (before this step's item loads, so that waiting for all
            // but those leaves the scales landed)
            if constexpr (!MX && LAST) {
                tile_scales_to_lds(j, R::OWN_STAGE ? (uint32_t)R::STAGE_AREA : slot_off(slot_add(rslot, 1)));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const int sn = h ? s + 1 : s, hn = h ^ 1;
        const int na_slot = h ? slot_add(rslot, 2) : rslot;   // slots of the items read next
        const uint32_t sa_off = slot_off(na_slot), sb_off = slot_off(slot_add(na_slot, 1));
        uint32_t nxa[NBM], nxb[NBN];
#pragma unroll
        for (int k = 0; k < SLOTS; ++k) {
            const int i = 1 + k / NBM, jb = k % NBM;
            mfma(acc[i][jb], fb[i], fa[jb], xb[i], xa[jb], Ops{});
            if constexpr (R::SCALES) {
                if (sc_go) {
                    if constexpr (R::PAIRED) {
#pragma unroll
                        for (int q = share_lo(k, SC_LOADS, SLOTS); q < share_hi(k, SC_LOADS, SLOTS); ++q)
                            sc_load(q, sc_gi, sc_ub);
                    } else if (k == 0) {
#pragma unroll
                        for (int q = 0; q < SC_LOADS; ++q) sc_load(q, sc_gi, sc_ub);
                    }
                }
            }
            if constexpr (!R::PAIRED) {
#pragma unroll
                for (int q = share_lo(k, LI_STEP, SLOTS); q < share_hi(k, LI_STEP, SLOTS); ++q) dma_item(q);
            } else if (h == 1) {
                // the stage's two items: the first over the first half of the slots, the second over the rest
                constexpr int HALF = SLOTS / 2;
                const int kk = k % HALF;
#pragma unroll
                for (int q = kk * LA / HALF; q < (kk + 1) * LA / HALF; ++q) dma_item(q);
                if (k == HALF - 1) advance();
            }
            // reads in order of first use: row block 0 of B, the NBM of A, then the rest of B
            if constexpr (!LAST) {
                if (R::SCALES && READ_SC && k == SCALE_SLOT) read_scales(j, sn, hn, nxa, nxb);
#pragma unroll
                for (int e = share_lo(k, NREAD, SLOTS); e < share_hi(k, NREAD, SLOTS); ++e) {
                    if (e == 0) nbf[0] = frag(sb_off, frag_b, hn, 0);
                    else if (e <= NBM) na[e - 1] = frag(sa_off, frag_a, hn, e - 1);
                    else nbf[e - NBM] = frag(sb_off, frag_b, hn, e - NBM);
                }
                if (!R::SCALES && k == SCALE_SLOT) read_scales(j, sn, hn, nxa, nxb);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (!R::PAIRED || h == 1) advance();
        if (h) rslot = na_slot;
        // keep this step's operand registers allocated to its end
#pragma unroll
        for (int i = 0; i < NBX; ++i) {
            if (i < NBM && i < NBN) asm volatile("" : : "v"(fa[i]), "v"(fb[i]));
            else if (i < NBM) asm volatile("" : : "v"(fa[i]));
            else asm volatile("" : : "v"(fb[i]));
        }
        if constexpr (!LAST && READ_SC) {
#pragma unroll
            for (int i = 0; i < NBX; ++i) {
                if (i < NBM) xa[i] = nxa[i];
                if (i < NBN) xb[i] = nxb[i];
            }
        }
    };
    using Step0 = std::integral_constant<int, 0>;
    using Step1 = std::integral_constant<int, 1>;
    using NotLast = std::integral_constant<bool, false>;
    using Last = std::integral_constant<bool, true>;

    for (int j = 0; j < my_tiles; ++j) {
        v16f acc[NBN][NBM];   // [n block][m block]
#pragma unroll
        for (int i = 0; i < NBN; ++i)
#pragma unroll
            for (int jb = 0; jb < NBM; ++jb) acc[i][jb] = (v16f){};
        const int nsj = SPLIT ? item_of(j).ns : nk;   // stages of this work item
        for (int s = 0; s < nsj - 1; ++s) {
            kstep(acc, j, s, Step0{}, NotLast{}, fa0, fb0, fa1, fb1);
            kstep(acc, j, s, Step1{}, NotLast{}, fa1, fb1, fa0, fb0);
        }
        kstep(acc, j, nsj - 1, Step0{}, NotLast{}, fa0, fb0, fa1, fb1);
        kstep(acc, j, nsj - 1, Step1{}, Last{}, fa1, fb1, fa0, fb0);
        // the slot of the last stage's B item is free until the next K step
        // loads into it (every wave finished reading it before the last barrier)
        const uint32_t stage_off = R::OWN_STAGE ? (uint32_t)R::STAGE_AREA : slot_off(slot_add(rslot, NSLOT - 1));
        if constexpr (SPLIT) {
            // the split item is the workgroup's last: the one that does not add
            // up the tile has no epilogue and nothing after it
            if (j == my_whole && !split_reduce(acc, stage_off)) break;
        }
        if (staged) {
            if constexpr (!MX) wait_vmcnt<LI_LAST>();   // the tile's scales (only the last item's loads may be in flight)
            __syncthreads();
            epilogue_staged_any(j, acc, stage_off);
            __syncthreads();   // staging reads done before that slot is loaded again
        } else {
            if constexpr (!MX) {
                wait_vmcnt<LI_LAST>();
                __syncthreads();
            }
            epilogue(j, acc, stage_off);
            if constexpr (!MX) __syncthreads();   // scale reads done before that slot is loaded again
        }
        // the next stage's step-0 fragments and scales (its items landed before
        // the last barrier; the slots of this stage's items are not refilled
        // before the next barrier).  After the last tile the fragment reads
        // (LDS) are harmless and unused; the scales are read only for a tile
        // that exists (the K-tail path reads them from global memory).
#pragma unroll
        for (int i = 0; i < NBX; ++i) {
            if (i < NBM) fa0[i] = frag(slot_off(rslot), frag_a, 0, i);
            if (i < NBN) fb0[i] = frag(slot_off(slot_add(rslot, 1)), frag_b, 0, i);
        }
        if (j + 1 < my_tiles) read_scales(j + 1, 0, 0, xa, xb);
    }
    wait_vmcnt<0>();   // the past-the-end loads must land before the workgroup exits
}

// ---- split items (mode (a), 128x128 tiles, K a multiple of 128).  When the
// tiles leave a last round at most half full (r = tiles % CUs tiles, 2r <=
// CUs), each of those r tiles may be split over K into S equal ranges of
// stages (S <= min(CUs / r, 4), S dividing the stages, at least 4 stages
// each), one work item per range, so that the last round keeps up to S r CUs
// busy instead of r.  Each item's partial tile then goes through memory (see
// the split reduction in the kernel), so S is chosen by a cost model fitted
// to measurements on MI355X: a stage of a 128x128 tile takes about 0.37 us
// whatever the number of tiles (the loop is latency-bound), and the exchange
// about 1.5 us plus its traffic (every item's 64 KB partial written, S - 1 of
// S read back) at about 4 TB/s.  Measured against unsplit tiles:
// 128x128x4096 16.7 -> 12.2 us (S = 4), 2048x1024x8192 31.2 -> 26.3 us
// (S = 2), 1024x1024x4096 17.1 -> 15.9 us (S = 4); 2048x1024x4096 gained
// nothing (18.2 / 18.4 us: 16 stages saved, 24 MB exchanged) and
// 2048x1024x1024 lost 44%, so neither splits.  (Those two and 1024x1024x4096
// now run on 64x128 tiles; see prefer_tile64.)  The workspace holds the arrival
// counters (one int per split tile, padded to 256 bytes) and the partial
// tiles (S r <= CUs of them).
struct SplitPlan {
    int tiles_whole, split;
};
constexpr double T_STAGE_US = 0.37, T_FIXED_US = 1.5, BYTES_PER_US = 4.0e6;
constexpr double PART_BYTES = 128.0 * 128.0 * 4.0;
// predicted K loop and exchange of r tiles of nk stages split s ways
static double split_us(int64_t r, int s, int64_t nk) {
    const double moved = (double)(s * r) * PART_BYTES * (1.0 + (double)(s - 1) / s);
    return (double)(nk / s) * T_STAGE_US + T_FIXED_US + moved / BYTES_PER_US;
}
static SplitPlan split_plan(int64_t tiles, int cus, int64_t nk) {
    SplitPlan p{(int)tiles, 1};
    const int64_t r = tiles % cus;
    if (r == 0 || 2 * r > cus || nk < 8) return p;
    double best = 0.1 * (double)nk * T_STAGE_US;   // require a predicted gain of 10% at least
    for (int s = 2; s <= 4 && s <= cus / r; ++s) {
        if (nk % s != 0 || nk / s < 4) continue;
        const double gain = (double)nk * T_STAGE_US - split_us(r, s, nk);
        if (gain > best) {
            best = gain;
            p.split = s;
            p.tiles_whole = (int)(tiles - r);
        }
    }
    return p;
}
// 64x128 tiles or 128x128 tiles split over K, for a problem whose 128x128
// tiles fill at most half of the CUs (so its 64x128 tiles fit one round).
// Fitted to measurements on MI355X: one round of 64x128 tiles takes about
// 4.4 us plus 0.26 us per stage, one of 128x128 tiles 5.4 us plus the split
// schedule's predicted loop and exchange; 64x128 tiles are taken when they
// are predicted at least 5% faster.  Measured (split / 64x128 tiles):
// 1024x1024x8192 21.2 / 23.0 us, 512x512x8192 16.0 / 20.8 us, 256x256x16384
// 22.0 / 37.6 us (split taken); 2048x1024x8192 27.1 / 25.2 us, 1024x512x4096
// 13.7 / 12.3 us (64x128 taken).  The model misses the smallest problems by
// a few percent: 128x128x4096 12.9 / 12.1 us and 1024x256x4096 13.0 /
// 12.3 us take the split.
static bool prefer_tile64(int64_t tiles128, int cus, int64_t nk, bool tail) {
    constexpr double T64_FIXED_US = 4.4, T64_STAGE_US = 0.26, T128_FIXED_US = 5.4;
    if (tail) return true;
    const SplitPlan sp = split_plan(tiles128, cus, nk);
    if (sp.split == 1) return true;
    return T64_FIXED_US + (double)nk * T64_STAGE_US <
           0.95 * (T128_FIXED_US + split_us(tiles128 - sp.tiles_whole, sp.split, nk));
}
static int64_t ws_cnt_bytes(int cus) { return ((int64_t)cus * 4 + 255) / 256 * 256; }
// bytes of workspace any split launch on a device with `cus` CUs may use
static int64_t split_ws_bytes(int cus) { return ws_cnt_bytes(cus) + (int64_t)cus * 256 * 256 * 4; }

// Zeroes n ints (the arrival counters of a new split workspace): a kernel
// rather than a memset, so that no memset node can reach a captured graph.
static __global__ __launch_bounds__(256) void clear_counters_kernel(int* __restrict__ p, int n) {
    const int i = (int)(blockIdx.x * 256 + threadIdx.x);
    if (i < n) p[i] = 0;
}

// The calling stream's split workspace (split_ws_bytes), allocated on the
// stream's first split launch and kept for the life of the process; its
// counters are cleared on the stream before the first use.  One workspace per
// (device, stream): launches on one stream run in order, so they never share
// it at the same time, and other streams have their own.  A stream that is
// being captured into a graph gets its workspace if it has one and nullptr
// otherwise (nothing is allocated or cleared during a capture): the launch
// then takes the unsplit schedule.
static hipError_t stream_workspace(int dev, hipStream_t stream, int cus, void** out) {
    static std::mutex mu;
    static std::map<std::pair<int, uintptr_t>, void*> cache;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(dev, reinterpret_cast<uintptr_t>(stream));
    const auto it = cache.find(key);
    if (it != cache.end()) {
        *out = it->second;
        return hipSuccess;
    }
    *out = nullptr;
    if (cs != hipStreamCaptureStatusNone) return hipSuccess;
    void* p = nullptr;
    e = hipMalloc(&p, (size_t)split_ws_bytes(cus));
    if (e != hipSuccess) return e;
    const int nc = (int)(ws_cnt_bytes(cus) / 4);
    clear_counters_kernel<<<dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, stream>>>(reinterpret_cast<int*>(p), nc);
    e = hipGetLastError();
    if (e != hipSuccess) {
        (void)hipFree(p);
        return e;
    }
    cache.emplace(key, p);
    *out = p;
    return hipSuccess;
}

template <bool MX, bool OUT_F32, bool KTAIL, int FA, int FB, int TILE, bool SPLIT>
static hipError_t launch_one(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                             const float* sa, const float* sb, const uint8_t* ea, const uint8_t* eb, void* D,
                             int dev, int cus, const SplitPlan& sp, void* ws, hipStream_t stream) {
    auto kern = gemm_fp8_kernel<MX, OUT_F32, KTAIL, FA, FB, TILE, SPLIT>;
    constexpr int LDS_BYTES = Ring<MX, KTAIL, TILE>::LDS_TOTAL;
    // up to 160 KB of dynamic LDS is above the default launch limit; raise it
    // once per device (the attribute is set for the current device).  Setting
    // it twice from racing threads is harmless.
    static std::atomic<uint64_t> configured{0};
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (!bit || !(configured.load(std::memory_order_acquire) & bit)) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        configured.fetch_or(bit, std::memory_order_release);
    }
    constexpr int BM = Geo<TILE>::BM, BN = Geo<TILE>::BN;
    const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
    const int64_t items = SPLIT ? sp.tiles_whole + (tiles - sp.tiles_whole) * sp.split : tiles;
    const int64_t grid = items < cus ? items : cus;   // persistent: at most one workgroup per CU
    int* cnt = SPLIT ? reinterpret_cast<int*>(ws) : nullptr;
    float* part = SPLIT ? reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + ws_cnt_bytes(cus)) : nullptr;
    kern<<<dim3((unsigned)grid), dim3(NTHREADS), LDS_BYTES, stream>>>((int)m, (int)n, (int)k, A, B, sa, sb, ea,
                                                                      eb, D, sp.tiles_whole, sp.split, part, cnt);
    return hipGetLastError();
}

// The schedule of a launch on a device with `cus` CUs: the tile shape and,
// for 128x128 tiles in mode (a) with K a multiple of 128, the split plan.  The
// launch and fp8g_gemm_schedule both take it from here.
//   128x128 tiles when 256x256 tiles would leave at least half of the CUs
//   idle: four times the tiles, each at a lower matrix-core rate.  Mode (a)
//   also when the 256x256 tiles spill just past one round (at most an eighth
//   of a second one): 4352x4096 (272 tiles) ran 4-14% faster on 128x128 tiles
//   at K = 1024..8192, while at 1.5 and 2 rounds the 256x256 tiles were
//   4-35% faster.
//   64x128 tiles (mode (a)) when 128x128 tiles would leave at least half of
//   the CUs idle and splitting them over K is not predicted faster
//   (prefer_tile64): twice the workgroups, each with half the matrix-core
//   work per stage.
//   256x128 tiles in place of 256x256 ones when they need at most 1.5 times
//   the rounds: a round of 256x128 tiles costs 0.57-0.66 of a round of
//   256x256 tiles in mode (b) and 0.5-0.65 in mode (a) (measured at 132 to
//   896 tiles of 256x256), so they pay where 256x256 tiles leave a last round
//   partly empty and lose where that round is nearly full.  Measured, mode (b)
//   (256x256 / 256x128 tiles): 2600x2900x1024 22.7 / 17.9 us (132 tiles of
//   256x256; 1 round against 1), 4352x4096x640 25.4 / 23.0 us (272; 2 rounds
//   against 3), 4096x6144x2048 55.9 / 55.2 us (384; 2 against 3);
//   3072x4096x1024 18.5 / 21.4 us (192; 1 against 2), 4096x8192x2048 66.4 /
//   76.0 us (512; 2 against 4), 4096x14336x4096 197.9 / 225.0 us (896; 4
//   against 7).  Mode (a): 2600x2900 at K = 1024 / 4096 / 8192 22.1 / 17.6,
//   45.4 / 35.7, 72.9 / 58.4 us (1 round against 1); 4608x4608x1024 31.5 /
//   29.2 us, 4608x4608x8192 153.0 / 151.2 us, 4096x6144x1024 31.9 / 29.6 us,
//   4864x4096x4096 83.1 / 80.4 us (2 against 3); 3072x4096x1024 18.0 /
//   18.1 us (1 against 2: not taken).  The mode (a) spill shapes above keep
//   128x128 tiles: 4352x4096 at K = 1024 ran 29.3 us on them against 30.9 us
//   on 256x128 tiles.
//   Only 128x128 tiles split: the 256x256 split kernel would spill around its
//   last step.
struct Schedule {
    int tile;       // 256, 128, TILE_64x128 or TILE_256x128
    SplitPlan sp;   // split == 1: no split
};
static Schedule gemm_schedule(int64_t m, int64_t n, int64_t k, bool mx, int cus) {
    const bool tail = (k % BK) != 0;
    const int64_t tiles256 = ((m + 255) / 256) * ((n + 255) / 256);
    const bool spill = !mx && tiles256 > cus && 8 * (tiles256 - cus) <= cus;
    if (2 * tiles256 <= cus || spill) {
        const int64_t tiles128 = ((m + 127) / 128) * ((n + 127) / 128);
        if (!mx) {
            if (!spill && 2 * tiles128 <= cus && prefer_tile64(tiles128, cus, k / BK, tail)) {
                const int64_t tiles64 = ((m + 63) / 64) * ((n + 127) / 128);
                return {TILE_64x128, {(int)tiles64, 1}};
            }
            if (!tail) return {128, split_plan(tiles128, cus, k / BK)};
        }
        return {128, {(int)tiles128, 1}};
    }
    const int64_t tiles_h = ((m + 255) / 256) * ((n + 127) / 128);   // 256x128 tiles
    const int64_t rounds = (tiles256 + cus - 1) / cus, rounds_h = (tiles_h + cus - 1) / cus;
    if (2 * rounds_h <= 3 * rounds) return {TILE_256x128, {(int)tiles_h, 1}};
    return {256, {(int)tiles256, 1}};
}

template <bool MX, int FA, int FB, int TILE>
static hipError_t launch_tiled(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B, const float* sa,
                               const float* sb, const uint8_t* ea, const uint8_t* eb, void* D, int out_f32, int dev,
                               int cus, const SplitPlan& sp, void* fixed_ws, hipStream_t stream) {
    // a K tail (k not a multiple of the 128-byte stage) zero-fills the bytes
    // past K and, in mode (b), reads the scales byte by byte from global memory
    const bool tail = (k % BK) != 0;
    constexpr int BM = Geo<TILE>::BM, BN = Geo<TILE>::BN;
    const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
    if constexpr (!MX && TILE == 128) {
        if (!tail && sp.split > 1) {
            void* ws = fixed_ws;   // the caller's fixed workspace (of split_ws_bytes(cus) at least), or the stream's
            if (!ws) {
                const hipError_t e = stream_workspace(dev, stream, cus, &ws);
                if (e != hipSuccess) return e;
            }
            if (ws)   // none: a capture on a stream without a workspace runs unsplit
                return out_f32 ? launch_one<MX, true, false, FA, FB, TILE, true>(m, n, k, A, B, sa, sb, ea, eb, D,
                                                                                 dev, cus, sp, ws, stream)
                               : launch_one<MX, false, false, FA, FB, TILE, true>(m, n, k, A, B, sa, sb, ea, eb, D,
                                                                                  dev, cus, sp, ws, stream);
        }
    }
    const SplitPlan whole{(int)tiles, 1};
    if (out_f32)
        return tail ? launch_one<MX, true, true, FA, FB, TILE, false>(m, n, k, A, B, sa, sb, ea, eb, D, dev, cus, whole,
                                                                      nullptr, stream)
                    : launch_one<MX, true, false, FA, FB, TILE, false>(m, n, k, A, B, sa, sb, ea, eb, D, dev, cus,
                                                                       whole, nullptr, stream);
    return tail ? launch_one<MX, false, true, FA, FB, TILE, false>(m, n, k, A, B, sa, sb, ea, eb, D, dev, cus, whole,
                                                                   nullptr, stream)
                : launch_one<MX, false, false, FA, FB, TILE, false>(m, n, k, A, B, sa, sb, ea, eb, D, dev, cus, whole,
                                                                    nullptr, stream);
}

template <bool MX, int FA, int FB>
hipError_t launch_fmt(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B, const float* sa,
                      const float* sb, const uint8_t* ea, const uint8_t* eb, void* D, int out_f32, void* fixed_ws,
                      hipStream_t stream) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const Schedule sc = gemm_schedule(m, n, k, MX, cus);
    if constexpr (!MX) {
        if (sc.tile == TILE_64x128)
            return launch_tiled<MX, FA, FB, TILE_64x128>(m, n, k, A, B, sa, sb, ea, eb, D, out_f32, dev, cus, sc.sp,
                                                         fixed_ws, stream);
    }
    if (sc.tile == TILE_256x128)
        return launch_tiled<MX, FA, FB, TILE_256x128>(m, n, k, A, B, sa, sb, ea, eb, D, out_f32, dev, cus, sc.sp,
                                                      fixed_ws, stream);
    if (sc.tile == 128)
        return launch_tiled<MX, FA, FB, 128>(m, n, k, A, B, sa, sb, ea, eb, D, out_f32, dev, cus, sc.sp, fixed_ws,
                                             stream);
    return launch_tiled<MX, FA, FB, 256>(m, n, k, A, B, sa, sb, ea, eb, D, out_f32, dev, cus, sc.sp, fixed_ws, stream);
}

// Each operand-format pair's kernels may be compiled in an object of their
// own (FP8G_GEMM_FMT = 2 * FA + FB, set by the library build so that the four
// pairs compile in parallel); the object with FP8G_GEMM_FMT 0 also holds the
// dispatch below.  Without the macro one object holds everything.
#ifndef FP8G_GEMM_FMT
#define FP8G_GEMM_FMT -1
#endif

#define FP8G_FMT_PAIR(KW, FA, FB)                                                                              \
    KW hipError_t launch_fmt<false, FA, FB>(int64_t, int64_t, int64_t, const uint8_t*, const uint8_t*,          \
                                            const float*, const float*, const uint8_t*, const uint8_t*, void*,  \
                                            int, void*, hipStream_t);                                           \
    KW hipError_t launch_fmt<true, FA, FB>(int64_t, int64_t, int64_t, const uint8_t*, const uint8_t*,           \
                                           const float*, const float*, const uint8_t*, const uint8_t*, void*,   \
                                           int, void*, hipStream_t);

#if FP8G_GEMM_FMT >= 0
FP8G_FMT_PAIR(extern template, 0, 0)
FP8G_FMT_PAIR(extern template, 0, 1)
FP8G_FMT_PAIR(extern template, 1, 0)
FP8G_FMT_PAIR(extern template, 1, 1)
#endif
#if FP8G_GEMM_FMT == 0
FP8G_FMT_PAIR(template, 0, 0)
#elif FP8G_GEMM_FMT == 1
FP8G_FMT_PAIR(template, 0, 1)
#elif FP8G_GEMM_FMT == 2
FP8G_FMT_PAIR(template, 1, 0)
#elif FP8G_GEMM_FMT == 3
FP8G_FMT_PAIR(template, 1, 1)
#endif

#if FP8G_GEMM_FMT <= 0
template <bool MX>
static hipError_t launch_mode(int64_t m, int64_t n, int64_t k, const uint8_t* A, int fmt_a, const uint8_t* B,
                              int fmt_b, const float* sa, const float* sb, const uint8_t* ea, const uint8_t* eb,
                              void* D, int out_f32, void* fixed_ws, hipStream_t stream) {
    if ((fmt_a != 0 && fmt_a != 1) || (fmt_b != 0 && fmt_b != 1)) return hipErrorInvalidValue;
    if (fmt_a == 0)
        return fmt_b == 0 ? launch_fmt<MX, 0, 0>(m, n, k, A, B, sa, sb, ea, eb, D, out_f32, fixed_ws, stream)
                          : launch_fmt<MX, 0, 1>(m, n, k, A, B, sa, sb, ea, eb, D, out_f32, fixed_ws, stream);
    return fmt_b == 0 ? launch_fmt<MX, 1, 0>(m, n, k, A, B, sa, sb, ea, eb, D, out_f32, fixed_ws, stream)
                      : launch_fmt<MX, 1, 1>(m, n, k, A, B, sa, sb, ea, eb, D, out_f32, fixed_ws, stream);
}

// 32-bit buffer offsets: a 256-row panel of K bytes stays below 2^31, so the
// out-of-range offset 2^31 plus any scalar offset still fits in 32 bits.
static bool fits(int64_t m, int64_t n, int64_t k) {
    const int64_t tiles = ((m + 127) / 128) * ((n + 127) / 128);
    return m < (1LL << 31) && n < (1LL << 31) && k < (1LL << 23) && tiles < (1LL << 31);
}

hipError_t schedule_gemm(int64_t m, int64_t n, int64_t k, int mx, int cus, int* tile_m, int* tile_n, int* split,
                         int* split_tiles) {
    if (!fits(m, n, k)) return hipErrorInvalidValue;
    const Schedule sc = gemm_schedule(m, n, k, mx != 0, cus);
    *tile_m = sc.tile > 1000 ? sc.tile / 1000 : sc.tile;
    *tile_n = sc.tile > 1000 ? sc.tile % 1000 : sc.tile;
    *split = sc.sp.split;
    const int64_t tiles = ((m + *tile_m - 1) / *tile_m) * ((n + *tile_n - 1) / *tile_n);
    *split_tiles = sc.sp.split > 1 ? (int)(tiles - sc.sp.tiles_whole) : 0;
    return hipSuccess;
}

hipError_t launch_gemm_scaled(int64_t m, int64_t n, int64_t k, const uint8_t* A, int fmt_a, const uint8_t* B,
                              int fmt_b, const float* sa, const float* sb, void* D, int out_f32,
                              hipStream_t stream) {
    if (!fits(m, n, k)) return hipErrorInvalidValue;
    return launch_mode<false>(m, n, k, A, fmt_a, B, fmt_b, sa, sb, nullptr, nullptr, D, out_f32, nullptr, stream);
}

// ---- fixed split workspace, for callers that cannot allocate
// (fp8_gemm_scaled_noalloc).  A file-scope device array, SCRATCH_BYTES =
// split_ws_bytes(256): enough for every split launch on a device of up to 256
// CUs.  It is zero when the library is loaded (its counters must start at
// zero) and every split launch leaves its counters at zero again.  In host
// code the name `scratch` stands for a host-side shadow, not for device
// memory: its address on each device comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is passed
// to kernels.  Every call on a device shares that device's array, so calls
// that overlap on one device race.
constexpr int64_t SCRATCH_BYTES = (int64_t)256 * 256 * 256 * 4 + 1024;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];
static_assert(SCRATCH_BYTES >= (256 * 4 + 255) / 256 * 256 + (int64_t)256 * 256 * 256 * 4, "scratch size");

static hipError_t scratch_address(int dev, void** out) {
    constexpr int MAX_DEV = 64;
    static std::mutex mu;
    static void* addr[MAX_DEV] = {};
    if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

hipError_t launch_gemm_scaled_noalloc(int64_t m, int64_t n, int64_t k, const uint8_t* A, const uint8_t* B,
                                      const float* sa, const float* sb, void* D, int out_f32, hipStream_t stream) {
    if (!fits(m, n, k)) return hipErrorInvalidValue;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (split_ws_bytes(cus) > SCRATCH_BYTES) return hipErrorOutOfMemory;   // a device of more than 256 CUs
    void* ws = nullptr;
    e = scratch_address(dev, &ws);
    if (e != hipSuccess) return e;
    return launch_mode<false>(m, n, k, A, 0, B, 0, sa, sb, nullptr, nullptr, D, out_f32, ws, stream);
}

hipError_t launch_gemm_mx(int64_t m, int64_t n, int64_t k, const uint8_t* A, int fmt_a, const uint8_t* B,
                          int fmt_b, const uint8_t* ea, const uint8_t* eb, void* D, int out_f32,
                          hipStream_t stream) {
    if (!fits(m, n, k)) return hipErrorInvalidValue;
    return launch_mode<true>(m, n, k, A, fmt_a, B, fmt_b, nullptr, nullptr, ea, eb, D, out_f32, nullptr, stream);
}
#endif  // FP8G_GEMM_FMT <= 0

}  // namespace fp8g
