/*
 * fp8g -- FP8 (OCP E4M3FN) scaled GEMM and row-wise quantizer for AMD Instinct
 * MI355X (gfx950).  Plain C ABI: host-side sizes, device pointers, a HIP
 * stream.  No synchronization; the only state and allocation is the split
 * workspace of fp8_gemm_scaled (see there).
 *
 * Operations (definitions in each entry point's comment):
 *   fp8_quantize_rowwise  fp32 [rows, cols] -> E4M3 codes + one fp32 scale per row
 *   fp8_quantize_ex       the same quantizer for fp32 or bf16 input, with one
 *                         scale per row or one per tensor, to E4M3 or E5M2
 *   mxfp8_quantize        fp32 [rows, cols] -> E4M3 codes + one UE8M0 scale per
 *                         32 consecutive elements of a row (MXFP8)
 *   fp8_gemm_scaled       D[m,n] = sa[m] * sb[n] * sum_k A[m,k] * B[n,k]
 *   fp8_gemm_scaled_noalloc  the same, allocating nothing (fixed workspace)
 *   mxfp8_gemm            same product with one power-of-two scale per 32 K
 *                         elements of every row of A and of B (MXFP8)
 *   fp8_gemm_scaled_ex,   the two GEMMs with the format of each operand
 *   mxfp8_gemm_ex         chosen: E4M3 or E5M2
 *   concat_mla_k          MLA key rows: 128 "nope" + 64 "rope" elements of
 *                         1-byte (E4M3 / E5M2) or 2-byte type
 *   fp8g_gemm_schedule    the tile and K split a GEMM launch takes (host only)
 *   fp8g_roof_mfma,       roof probes: the matrix-core rate and the streaming
 *   fp8g_roof_stream      bandwidth the part reaches at the moment
 *
 * Common conventions
 *   - Every array is dense and row-major; the caller owns all memory.  A is
 *     [m, k] and B is [n, k], both with k contiguous ("K-major"); D is
 *     [m, n] with n contiguous.  FP8 operands are passed as their byte codes.
 *   - Device pointers must stay valid until the work queued on `stream`
 *     has run.  `stream` may be 0 (the null stream).
 *   - Every pointer must be 16-byte aligned (else FP8G_ERR_ALIGN), except
 *     that an argument whose array is empty may be NULL.
 *   - Arguments are checked on the host before any HIP call; a failed check
 *     returns its status and queues nothing.  A launch failure returns
 *     FP8G_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *     synchronization, as with any HIP kernel.
 *   - Results are bitwise reproducible run to run: sums run in a fixed
 *     order; the per-tensor amax atomic is a max, which no order changes,
 *     and split GEMM tiles add their K ranges' partials in split order
 *     whichever finishes first.
 *   - Calls are thread-safe.  The one mutable state is fp8_gemm_scaled's
 *     split workspace, kept per (device, stream) so that calls on different
 *     streams never share it.
 */
#ifndef FP8G_H
#define FP8G_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP8G_OUT_BF16 = 0, /* bfloat16, round to nearest even */
    FP8G_OUT_F32 = 1   /* float32 */
} fp8g_out_t;

typedef enum {
    FP8G_IN_F32 = 0,  /* float32 input */
    FP8G_IN_BF16 = 1  /* bfloat16 input (converted to float32 exactly) */
} fp8g_in_t;

typedef enum {
    FP8G_SCALE_PER_ROW = 0,    /* one scale per row: scale [rows] */
    FP8G_SCALE_PER_TENSOR = 1  /* one scale for the whole tensor: scale [1] */
} fp8g_granularity_t;

typedef enum {
    FP8G_FMT_E4M3 = 0, /* OCP E4M3FN: bias 7, largest magnitude 448, no infinities */
    FP8G_FMT_E5M2 = 1  /* OCP E5M2: bias 15, largest finite 57344, IEEE-style Inf/NaN */
} fp8g_fmt_t;

typedef enum {
    FP8G_OK = 0,
    FP8G_ERR_NULL = 1,        /* required pointer is NULL */
    FP8G_ERR_SHAPE = 2,       /* negative extent, or k not a multiple of 32 for MXFP8 */
    FP8G_ERR_ALIGN = 3,       /* pointer not 16-byte aligned */
    FP8G_ERR_DTYPE = 4,       /* unknown out_dtype, operand format, input dtype, granularity or element size */
    FP8G_ERR_OVERLAP = 5,     /* an output overlaps an input or another output */
    FP8G_ERR_UNSUPPORTED = 6, /* valid but outside the library's limits (see each call) */
    FP8G_ERR_HIP = 7          /* the HIP runtime refused the launch */
} fp8g_status_t;

/*
 * fp8_quantize_rowwise -- per-row (per-token / per-channel) E4M3 quantization.
 *
 * Source: the scale rule abs_max / 448 (448 = largest E4M3 magnitude) in
 * `_calibrate_scales` of the hybrid-inference class on the page
 * "FP8 推理基础设施（五）：从 DeepGEMM 到 vLLM", applied per row as the
 * per-token scale_a / per-channel scale_b of the same page's DeepGEMM call;
 * the activation flow of section 2.2 of the RTX 4060 FP8 inference page.
 *
 *   s[r]   = fp32(max_c |x[r,c]| / 448)                  (IEEE division)
 *   q[r,c] = E4M3_RNE_SAT(fp32(x[r,c] / s[r]))           (IEEE division, then
 *            round to nearest even with ties to the even code, magnitudes
 *            above 448 saturate to 448, sign copied from x)
 *   if s[r] == 0 (zero or empty row, or amax/448 underflows): s[r] = 0 and
 *   q[r,c] is +0 or -0 by the sign of x[r,c].
 * The scale is a dequantization multiplier: x ~ decode(q) * s.
 *
 * x      device, fp32 [rows, cols], read only
 * q      device, E4M3 codes [rows, cols], written
 * scale  device, fp32 [rows], written
 * rows, cols >= 0; rows == 0 is a no-op; cols == 0 writes scale = 0.
 * rows >= 2^31 -> ERR_UNSUPPORTED.
 * NaN/Inf in x are outside the contract.  Bit-exact with the definition.
 * Errors: ERR_NULL, ERR_SHAPE (negative), ERR_ALIGN, ERR_OVERLAP,
 * ERR_UNSUPPORTED, ERR_HIP.
 */
int fp8_quantize_rowwise(const float* x, int64_t rows, int64_t cols,
                         uint8_t* q, float* scale, hipStream_t stream);

/*
 * fp8_gemm_scaled -- FP8 GEMM with per-token A scales and per-channel B scales.
 *
 * Source: the DeepGEMM call on the page "FP8 推理基础设施（五）：从 DeepGEMM
 * 到 vLLM" (GEMM-call example): E4M3 A and B, m = tokens, n, k = hidden,
 * scale_a one fp32 per token, scale_b one fp32 per channel; argument order
 * m, n, k, A, B, scale_a, scale_b as there.
 *
 *   D[m,n] = out( sa[m] * sb[n] * sum_k dec(A[m,k]) * dec(B[n,k]) )
 * with the sum accumulated in fp32 on the matrix cores, the two scales
 * applied in fp32, and `out` the conversion to bf16 (round to nearest even)
 * or fp32.
 *
 * Accuracy: |D - exact| <= 1e-5 * W + 1 ulp of the output format + T, with
 *   W = |sa sb| sum_k |dec(A[m,k]) dec(B[n,k])|,
 *   T = |sa sb| sum over runs of 8 consecutive k of the sum, over the run's
 *       products p that are not multiples of 2^(E - 13), of min(|p|, 2^(E - 13)),
 *       E the run's largest exponent sum (exponent fields of the two codes,
 *       zeros and subnormals at the smallest normal exponent).
 * T is the gfx950 FP8 matrix core's own rounding: it sums each run of 8
 * products in fixed point 13 bits below the run's largest exponent sum and
 * drops the lower bits (measured on every gfx950 FP8 matrix-core instruction,
 * the scaled 32x32x64 / 16x16x128 and the older 32x32x16 / 16x16x32 forms; none
 * sums exactly).  Without T ("the plain bound") the result holds where no run
 * mixes magnitudes 2^13 apart: on every output of the N(0,1) raw-cast and the
 * 8192x2048x8192 per-token workloads, both output types.  It does not hold in
 * general: on the 8192x22016x8192 FFN-up workload (x50 activation outliers),
 * 34 of 1453056 checked bf16 outputs and 12598 fp32 outputs exceed it.  The
 * bf16 matrix-core instruction, which represents every E4M3 value exactly,
 * sums within the plain bound but runs at half the FP8 rate (measured 2.33 vs
 * 4.65 PFLOP/s); this library does not use it.
 *
 * A        device, E4M3 codes [m, k]          B   device, E4M3 codes [n, k]
 * scale_a  device, fp32 [m]                   scale_b device, fp32 [n]
 * D        device, [m, n] of out_dtype (fp8g_out_t), written
 * m, n, k >= 0.  m == 0 or n == 0: no-op.  k == 0: D = 0.
 * Split workspace: when the 128x128 output tiles leave a last round of tiles
 * at most half full and K (a multiple of 128) is long enough to pay (and, for
 * problems whose 64x128 tiles fit one round, pays more than those), those
 * tiles are split over K and their partial sums pass through a device
 * workspace (with per-tile counters).  The library allocates it with
 * hipMalloc (64 MB + 1 KB on a 256-CU device) on the first such call on each
 * (device, stream), clears its counters with a small kernel on that stream,
 * and keeps it until the process ends.  Under stream capture nothing is
 * allocated: a stream that already has its workspace uses it (the graph then
 * shares it with that stream's later split calls, so the two must not
 * overlap), and one that has none runs the unsplit schedule, whose D meets
 * the same bound but may differ in rounding from a split call's.  Callers
 * that cannot allocate at all use fp8_gemm_scaled_noalloc.
 * Limits (ERR_UNSUPPORTED): k % 16 != 0 (16-byte rows); k >= 2^23, m >= 2^31,
 * or n >= 2^22 (bf16 output) / 2^21 (fp32 output): the kernels address a
 * 256-row panel of A, B or D with 32-bit offsets below 2^31.  E4M3 NaN codes
 * in A or B are outside the contract.
 * Errors: ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_OVERLAP,
 * ERR_UNSUPPORTED, ERR_HIP.
 */
int fp8_gemm_scaled(int64_t m, int64_t n, int64_t k,
                    const uint8_t* A, const uint8_t* B,
                    const float* scale_a, const float* scale_b,
                    void* D, int out_dtype, hipStream_t stream);

/*
 * fp8_gemm_scaled_noalloc -- fp8_gemm_scaled for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.
 *
 * Same arguments, definition, accuracy, limits and errors as fp8_gemm_scaled,
 * and the same kernels, so the same D bit for bit.  The one difference is the
 * split workspace: instead of a per-stream allocation it uses a fixed device
 * array inside the library (64 MB + 1 KB, zero at load; each device the
 * library runs on holds its own copy until the process ends).  The call
 * allocates nothing, clears nothing on the host side, and only queues work on
 * `stream`; every split launch leaves the array's counters at zero again.
 * All calls on one device share that array: calls that overlap on one device
 * (other streams, other threads) race and must be ordered by the caller.
 * Errors: as fp8_gemm_scaled; ERR_UNSUPPORTED also on a device with more than
 * 256 CUs, which the array does not cover.
 */
int fp8_gemm_scaled_noalloc(int64_t m, int64_t n, int64_t k,
                            const uint8_t* A, const uint8_t* B,
                            const float* scale_a, const float* scale_b,
                            void* D, int out_dtype, hipStream_t stream);

/*
 * fp8_quantize_ex -- FP8 quantization with the scale rule of
 * fp8_quantize_rowwise, for fp32 or bf16 input, per row or per tensor, to E4M3
 * or E5M2 codes.
 *
 * Source: the scale rule abs_max / 448 in `_calibrate_scales` of the
 * hybrid-inference class on the page "FP8 推理基础设施（五）：从 DeepGEMM 到
 * vLLM", which takes abs_max over a whole tensor (per tensor); per row as in
 * fp8_quantize_rowwise.  bf16 is the precision models are usually deployed in
 * (page on FP8 vLLM for AMD Instinct, introduction); each bf16 value is
 * converted to fp32 exactly (its bits shifted up by 16), so the result is that
 * of the fp32 quantizer on the converted tensor.  E5M2 output (the page on
 * FlashInfer's concat_mla_k with FP8 inputs takes E5M2 beside E4M3) uses the
 * same rule with that format's largest finite value: MAX = 448 (E4M3) or
 * 57344 (E5M2).
 *
 *   per row:    s[r] = fp32(max_c |x[r,c]| / MAX),  q[r,c] = RNE_SAT(fp32(x[r,c] / s[r]))
 *   per tensor: s[0] = fp32(max_{r,c} |x[r,c]| / MAX), q[r,c] = RNE_SAT(fp32(x[r,c] / s[0]))
 *   RNE_SAT: round to nearest even in the output format, magnitudes above MAX
 *   saturate to MAX, sign copied; a zero scale gives signed zeros, as in
 *   fp8_quantize_rowwise.
 *
 * x        device, [rows, cols] of in_dtype (FP8G_IN_F32 / FP8G_IN_BF16), read only
 * out_fmt  FP8G_FMT_E4M3 or FP8G_FMT_E5M2
 * q        device, codes of out_fmt [rows, cols], written
 * scale    device, fp32, written: [rows] (FP8G_SCALE_PER_ROW) or [1]
 *          (FP8G_SCALE_PER_TENSOR; it holds an intermediate until the call's
 *          work on the stream has finished)
 * rows, cols >= 0.  Per row: rows == 0 is a no-op; rows >= 2^31 ->
 * ERR_UNSUPPORTED.  Per tensor: the scale is always written (0 for an empty
 * tensor).  Bit-exact with the definition.
 * Errors: ERR_NULL, ERR_SHAPE (negative), ERR_DTYPE (unknown in_dtype,
 * granularity or out_fmt), ERR_ALIGN, ERR_OVERLAP, ERR_UNSUPPORTED (size
 * overflow), ERR_HIP.
 */
int fp8_quantize_ex(const void* x, int in_dtype, int64_t rows, int64_t cols, int granularity,
                    int out_fmt, uint8_t* q, float* scale, hipStream_t stream);

/*
 * mxfp8_quantize -- MXFP8 block quantization (the step before mxfp8_gemm).
 *
 * Source: the page "[sglang] FlashInfer v0.6.7 MXFP8 Gemm 통합", section 1:
 * one unsigned-byte scale per 32 elements along K, the scale tensor shaped
 * (rows, cols // 32).  The byte is UE8M0: code c stands for 2^(c - 127).  For
 * block j of row r (elements 32j .. 32j+31):
 *
 *   amax   = max |x[r, 32j + t]|
 *   e      = the smallest integer with amax <= 448 * 2^e, clamped to
 *            [-127, 127]; e = -127 for an all-zero block
 *   scale[r, j] = e + 127
 *   q[r, 32j + t] = E4M3_RNE(x[r, 32j + t] * 2^-e)   (exact power-of-two
 *            scaling; never above 448, so the cast never saturates; the sign
 *            of zero is kept)
 * so that x ~ decode(q) * 2^(scale - 127).
 *
 * x      device, fp32 [rows, cols], read only
 * q      device, E4M3 codes [rows, cols], written
 * scale  device, UE8M0 codes [rows, cols / 32], written
 * cols % 32 != 0 -> ERR_SHAPE.  rows == 0 or cols == 0: no-op.
 * NaN/Inf in x are outside the contract.  Bit-exact with the definition.
 * Errors: ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_OVERLAP, ERR_UNSUPPORTED
 * (size overflow), ERR_HIP.
 */
int mxfp8_quantize(const float* x, int64_t rows, int64_t cols,
                   uint8_t* q, uint8_t* scale, hipStream_t stream);

/*
 * mxfp8_gemm -- MXFP8 block-scaled GEMM.
 *
 * Source: the page "[sglang] FlashInfer v0.6.7 MXFP8 Gemm 통합", section 1
 * (one uint8 scale per 32 elements of K, scale tensor of shape (n, k // 32))
 * and section 2 (the GEMM takes fp8 activations with their uint8 scales, the
 * fp8 weight with its uint8 scales, and an output dtype).  A scale byte c
 * stands for 2^(c - 127) (UE8M0).
 *
 *   D[m,n] = out( sum_j 2^(ea[m,j]-127) * 2^(eb[n,j]-127)
 *                       * sum_{t<32} dec(A[m,32j+t]) * dec(B[n,32j+t]) )
 * accumulated in fp32 on the scaled matrix-core instructions.  Accuracy as
 * fp8_gemm_scaled, with the block scale factors 2^(ea+eb-254) in W and in T
 * (each run of 8 lies inside one 32-element block) and no sa, sb.  On the
 * 4096x14336x4096 workload (2^u block factors), 3 of 487424 checked bf16
 * outputs and 818 fp32 outputs exceed the plain bound.
 *
 * A        device, E4M3 codes [m, k]          B   device, E4M3 codes [n, k]
 * scale_a  device, UE8M0 codes [m, k/32]      scale_b device, UE8M0 codes [n, k/32]
 * D        device, [m, n] of out_dtype, written
 * k % 32 != 0 -> ERR_SHAPE.  m == 0 or n == 0: no-op.  k == 0: D = 0.
 * Limits as fp8_gemm_scaled: k >= 2^23, m >= 2^31, n >= 2^22 (bf16) / 2^21
 * (fp32) -> ERR_UNSUPPORTED.
 * Performance: k % 128 != 0 takes a slower path (scale bytes read one by one
 * from global memory), about half the rate of k % 128 == 0.
 * Scale code 255 (NaN) and E4M3 NaN codes are outside the contract.
 * Errors: ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_OVERLAP,
 * ERR_UNSUPPORTED, ERR_HIP.
 */
int mxfp8_gemm(int64_t m, int64_t n, int64_t k,
               const uint8_t* A, const uint8_t* B,
               const uint8_t* scale_a, const uint8_t* scale_b,
               void* D, int out_dtype, hipStream_t stream);

/*
 * fp8_gemm_scaled_ex, mxfp8_gemm_ex -- the two GEMMs above with a format per
 * operand.
 *
 * Source: the page on FlashInfer's concat_mla_k with FP8 inputs (sections
 * 1-2) takes FP8 E5M2 beside E4M3; read as the OCP E5M2 format (1 sign, 5
 * exponent bits with bias 15, 2 mantissa bits).  The gfx950 scaled
 * matrix-core instruction takes a format per operand, so every pair is
 * accepted: fmt_a, fmt_b are FP8G_FMT_E4M3 or FP8G_FMT_E5M2 (else ERR_DTYPE).
 *
 * Arguments, definitions, limits and errors as fp8_gemm_scaled / mxfp8_gemm,
 * with dec() the decoding of each operand's own format.  fp8_gemm_scaled and
 * mxfp8_gemm are these calls with both formats E4M3.  Infinity and NaN codes
 * in A or B are outside the contract.  Accuracy: as fp8_gemm_scaled / mxfp8_gemm,
 * with each operand's own exponent field in T (E5M2: bias 15, zeros and
 * subnormals at -14).  With an E5M2 operand the products span 2^-32 .. 2^32,
 * so runs mix magnitudes far apart more often and T is larger.
 */
int fp8_gemm_scaled_ex(int64_t m, int64_t n, int64_t k,
                       const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b,
                       const float* scale_a, const float* scale_b,
                       void* D, int out_dtype, hipStream_t stream);

int mxfp8_gemm_ex(int64_t m, int64_t n, int64_t k,
                  const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b,
                  const uint8_t* scale_a, const uint8_t* scale_b,
                  void* D, int out_dtype, hipStream_t stream);

/*
 * concat_mla_k -- assemble MLA key rows from their nope and rope parts.
 *
 * Source: the page on FlashInfer's concat_mla_k with FP8 (E4M3 / E5M2)
 * inputs, sections 1-3: each key row is 128 nope elements followed by 64
 * rope elements; elements of 1 byte (E4M3, E5M2) or 2 bytes (BF16, FP16) are
 * moved unchanged (bit-exact).
 *
 *   k[t, h, 0:128]   = k_nope[t, h, 0:128]
 *   k[t, h, 128:192] = k_rope[t, (rope_heads == 1 ? 0 : h), 0:64]
 *
 * k       device, [tokens, heads, 192] elements, written
 * k_nope  device, [tokens, heads, 128] elements, read only
 * k_rope  device, [tokens, rope_heads, 64] elements, read only; rope_heads is
 *         1 (one rope part per token, shared by its heads) or heads
 * elem_bytes  1 or 2 (else ERR_DTYPE); all arrays dense, row-major.
 * tokens == 0 or heads == 0: no-op.  Errors: ERR_NULL, ERR_SHAPE (negative
 * extent, rope_heads not 1 or heads), ERR_DTYPE, ERR_ALIGN, ERR_OVERLAP
 * (k overlaps an input), ERR_UNSUPPORTED (size overflow), ERR_HIP.
 */
int concat_mla_k(void* k, const void* k_nope, const void* k_rope,
                 int64_t tokens, int64_t heads, int64_t rope_heads,
                 int elem_bytes, hipStream_t stream);

/*
 * fp8g_roof_mfma, fp8g_roof_stream -- roof probes (measurement helpers, not
 * part of the GEMM path).
 *
 * Source: the page on FP8 inference of a 7B model on an RTX 4060, section
 * 4.1, checks a kernel's core utilisation and memory bandwidth.  These two
 * calls measure what the chip delivers at the moment they run, so that the
 * benchmark can put the hot path's kernels beside a measured roof as well as
 * the nominal one.
 *
 * fp8g_roof_mfma: `blocks` workgroups of 256 threads; every wave runs `iters`
 * rounds of four independent chains of the scaled 32x32x64 FP8 matrix-core
 * instruction the GEMMs use, with no memory traffic: blocks * 4 * iters * 4 *
 * 131072 flops.  sink: device, at least one float (practically never written;
 * it keeps the work).  blocks in [1, 2^31), iters in [1, 2^31), else
 * ERR_SHAPE; sink NULL: ERR_NULL.
 *
 * fp8g_roof_stream: reads `bytes` from src and writes bytes / write_ratio to
 * dst (write_ratio 1: a copy; 4: 16 bytes read per 4 written, the fp32
 * quantizer's mix), one 32 KB chunk per workgroup, non-temporal loads, and
 * write-back (nontemporal_stores 0) or non-temporal (1) stores.  bytes >= 0
 * and a multiple of 16, write_ratio 1 or 4, else ERR_SHAPE;
 * nontemporal_stores not 0 or 1: ERR_DTYPE; NULL with bytes > 0: ERR_NULL;
 * unaligned: ERR_ALIGN; dst overlapping src: ERR_OVERLAP.  dst receives
 * unspecified bytes.
 *
 * Both only queue one kernel on `stream`; the caller times it (HIP events on
 * the same stream).  Errors: as above, ERR_HIP.
 */
int fp8g_roof_mfma(int64_t blocks, int64_t iters, float* sink, hipStream_t stream);

int fp8g_roof_stream(const void* src, int64_t bytes, void* dst, int write_ratio, int nontemporal_stores,
                     hipStream_t stream);

/*
 * fp8g_gemm_schedule -- the schedule fp8_gemm_scaled (mode 0; also the _ex and
 * _noalloc forms) or mxfp8_gemm (mode 1; also mxfp8_gemm_ex) takes for an m x
 * n x k problem on a device with `cus` compute units: the host-side choice the
 * launch itself makes, exposed so that callers (and tests) can see it.
 * Host only: no HIP call, no device needed.
 *
 * tile_m x tile_n  the output tile of a workgroup: 256 x 256; 128 x 128 when
 *                  256 x 256 tiles would leave at least half of the CUs idle
 *                  (mode 0 also when they spill just past one round); in mode
 *                  0, 64 x 128 when 128 x 128 tiles would still leave half of
 *                  the CUs idle and splitting them over K is not predicted
 *                  faster; 256 x 128 in place of 256 x 256 when they need at
 *                  most 1.5 times the rounds of workgroups (both modes).
 * split            1, or the number of K ranges (2..4) each of the last
 *                  round's 128 x 128 tiles is split into (mode 0, k a multiple
 *                  of 128; such launches use the split workspace described at
 *                  fp8_gemm_scaled, and under stream capture on a stream
 *                  without one they run unsplit).
 * split_tiles      the number of split tiles (0 when split == 1).
 * The choice comes from cost models fitted to measurements on MI355X
 * (256 CUs); other CU counts get the same rules.  m, n, k >= 0 and cus >= 1,
 * else ERR_SHAPE; mode not 0 or 1: ERR_DTYPE; a NULL output: ERR_NULL; sizes
 * beyond the GEMMs' limits: ERR_UNSUPPORTED.
 */
int fp8g_gemm_schedule(int64_t m, int64_t n, int64_t k, int mode, int cus, int* tile_m, int* tile_n, int* split,
                       int* split_tiles);

/* Static, human-readable text for a status code (never NULL). */
const char* fp8g_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8G_H */
