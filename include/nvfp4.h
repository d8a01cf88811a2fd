/*
 * nvfp4.h - C ABI of libnvfp4, NVFP4 block quantization for AMD CDNA4 (gfx950).
 *
 * NVFP4: 4-bit e2m1 element codes (sign bit + magnitude grid
 * {0, .5, 1, 1.5, 2, 3, 4, 6}) packed two per byte, one e4m3 scale byte per
 * 16-element block, and an optional fp32 second-level (global) scale derived
 * from a global amax.  Sources: the "fp4-train" kernel card (Method, API,
 * Requirements and limits), the four-over-six pull request "Add NVFP4
 * four-over-six (row-wise) quantization to the training prototype" (What,
 * numeric details, CuTe DSL kernel Design) and "Stable FP4 Training via
 * Transposition-Invariant Block Quantization" (abstract).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are dense row-major [M, K] with K % 16 == 0 ("K a multiple of 16;
 *   float32 or bfloat16 input", fp4-train, Requirements and limits).  Element
 *   (m, k) has the global index i = m*K + k; M*K must not exceed 2^33 so that
 *   the pair index i >> 1 of the random-number generator fits 32 bits.
 * - All pointers are DEVICE pointers, owned by the caller, allocated on the
 *   device that is current when the call is made.  The library allocates no
 *   memory and keeps no state other than the fixed scratch array of
 *   nvfp4_amax_noalloc; calls are asynchronous on `stream` (a
 *   hipStream_t; NULL is the default stream) and return once the kernels are
 *   queued.  Outputs must not overlap inputs, except that nvfp4_qdq may
 *   write `out` over `x` when both have the same dtype.
 * - Alignment: x, residual and out must be 16-byte aligned; packed codes
 *   8-byte aligned; scale bytes and amax pointers need 4-byte alignment
 *   only where stated.
 * - Layouts: packed codes [M, K/2] bytes, byte j of a row holds element 2j in
 *   its low nibble and element 2j+1 in its high nibble; code = sign << 3 |
 *   magnitude index.  Scales [M, K/16] e4m3 bytes (plain row-major, no
 *   tensor-core swizzle).  16x16 tile scales [M/16, K/16].
 * - Errors: every argument is validated on the host before anything is
 *   launched; on error nothing is written and a status other than NVFP4_OK is
 *   returned.  NVFP4_E_HIP reports a failed kernel launch.  Nothing is
 *   printed and nothing aborts.  An empty tensor (M == 0 or K == 0) returns
 *   NVFP4_OK and launches nothing, except that nvfp4_amax writes 0.
 *
 * Signature choices
 * - `stream` is a hipStream_t passed as void*, so that this header needs no
 *   HIP include and plain C callers (ctypes, other languages) can use it.
 * - The second-level scale is chosen by nvfp4_scale_mode (NONE, TENSOR,
 *   ROW): it selects the amax shape for nvfp4_amax, nvfp4_quantize_4over6
 *   and nvfp4_dequantize alike.
 * - Only the per-tensor amax needs device scratch, so its size query is
 *   nvfp4_amax_workspace_bytes (nvfp4_amax_noalloc needs none).
 * - nvfp4_quantize_4over6 computes the row amax in the same pass when
 *   amax_is_input is 0 (the pass holds each row on chip), so it takes a
 *   writable amax pointer; nvfp4_quantize_2d takes the truncation-free flag
 *   of its tile scale; nvfp4_dequantize takes the producer's scale mode and
 *   bound.
 *
 * Numerics (identical on every path; the CPU oracle is the reference)
 * - x' = x + r when a residual r is given (error feedback), one fp32 add.
 * - Block amax a = NaN-dropping max of |x'| (all-NaN block -> 0).
 * - Global scale from amax A and bound B (448, or 256/448 for four-over-six):
 *   D = 6*B, S_enc = min(D / A, FLT_MAX), S_dec = A / D, true fp32 divisions.
 * - e4m3 scale: sigma -> min(sigma, 448) -> round-to-nearest-even, satfinite;
 *   s = decoded scale; encode reciprocal rho = min(1 / (s * S_dec), FLT_MAX).
 * - Element: v = |x'| * rho, rounded to the e2m1 grid (RTN: nearest, ties to
 *   even; SR: up iff u * 2^-16 < f22, u the element's 16-bit draw and f22
 *   the fractional distance between the two grid points truncated to 22
 *   bits, so up with probability within 2^-16 of the fractional distance),
 *   >= 6 saturates, a NaN v encodes +6 (0x7); sign bit from x'.
 * - Draws: pcg(v) is the "pcg" hash of Jarzynski and Olano ("Hash Functions
 *   for GPU Rendering"), key = pcg(seed ^ pcg(step ^ 0x9E3779B9)); the pair
 *   of elements 2p, 2p + 1 (global indices) takes the word w = pcg(p ^ key),
 *   element 2p the draw w & 0xFFFF and element 2p + 1 the draw w >> 16.
 * - Dequantize: x_hat = (val * s) * S_dec in fp32, then bf16 round-to-nearest-
 *   even (NaN -> 0x7FC0) when the output is bf16.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_E_NULL = 1,   /* a required pointer is NULL */
  NVFP4_E_SHAPE = 2,  /* negative size, K % 16 != 0, or M % 16 != 0 where tiles need it */
  NVFP4_E_DTYPE = 3,  /* unknown dtype code */
  NVFP4_E_ALIGN = 4,  /* a pointer misses its required alignment */
  NVFP4_E_ARG = 5,    /* bad enum value, bound, or workspace too small */
  NVFP4_E_RANGE = 6,  /* M*K > 2^33 */
  NVFP4_E_HIP = 7     /* the HIP runtime rejected a launch */
} nvfp4_status;

typedef enum { NVFP4_F32 = 0, NVFP4_BF16 = 1 } nvfp4_dtype;
typedef enum { NVFP4_RTN = 0, NVFP4_SR = 1 } nvfp4_round;
typedef enum { NVFP4_MAE = 0, NVFP4_MSE = 1 } nvfp4_err;
/* Second-level scale: none, one amax for the tensor, or one amax per row. */
typedef enum { NVFP4_SCALE_NONE = 0, NVFP4_SCALE_TENSOR = 1, NVFP4_SCALE_ROW = 2 } nvfp4_scale_mode;

/* Human-readable name of a status (static string, never NULL). */
const char* nvfp4_status_str(nvfp4_status s);

/* Bytes of workspace nvfp4_amax needs for a per-tensor amax of M*K elements. */
size_t nvfp4_amax_workspace_bytes(int64_t M, int64_t K);

/*
 * nvfp4_amax - global amax A = NaN-dropping max of |x'| (x' = x + residual
 * when residual != NULL), over the whole tensor (mode TENSOR: amax_out[0],
 * two passes: per-workgroup partials into `workspace`, then one reduction)
 * or over each row (mode ROW: amax_out[0..M-1], one pass).  Source: the
 * four-over-six pull request, What (scalar global_amax = per-tensor
 * scaling, a (rows,) vector = row-wise) and CuTe DSL kernel Design
 * (NaN-dropping max).  workspace: device buffer of at least
 * nvfp4_amax_workspace_bytes(M, K) bytes (TENSOR only; may be NULL for
 * ROW).  An empty tensor gives 0.
 */
nvfp4_status nvfp4_amax(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                        const float* residual, nvfp4_scale_mode mode, float* amax_out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_amax_noalloc - nvfp4_amax for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same result, bit for bit, with no workspace
 * argument.  The per-tensor pass keeps its per-workgroup partial maxima in a
 * device array owned by the library (8 KiB per GPU, held until the process
 * ends; at most 2048 partials, which every shape with M*K <= 2^33 fits:
 * otherwise NVFP4_E_RANGE).  The array's device address is looked up on the
 * first call on each GPU (hipGetSymbolAddress; a failure returns
 * NVFP4_E_HIP).  The call allocates nothing.  All calls on one GPU share
 * that array, so calls that overlap on one GPU (concurrent streams or host
 * threads) race; serialize them.  Arguments and errors otherwise as
 * nvfp4_amax; mode ROW uses no scratch at all.
 */
nvfp4_status nvfp4_amax_noalloc(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                                const float* residual, nvfp4_scale_mode mode, float* amax_out,
                                void* stream);

/*
 * nvfp4_quantize - NVFP4 quantize on 1x16 blocks (fp4-train, API
 * quantize(x, stochastic, residual, seed, step); Method).
 *   x        [M, K] fp32 or bf16 (dt).
 *   residual NULL, or [M, K] fp32 error-feedback residual updated in place:
 *            x' = x + r, then r <- x' - x_hat with the fp32 dequantized x_hat.
 *   global_amax NULL (block scale = block_absmax / 6, fp4-train Method), or
 *            a device pointer to one fp32 amax A: standard NVFP4 two-level
 *            scaling with bound 448, sigma = a * (S_enc * (1/6)).
 *   rnd, seed, step: NVFP4_RTN, or NVFP4_SR with the counter-based
 *            generator keyed by (seed, step) and the global element index.
 *   packed   [M, K/2] out; scales [M, K/16] out.
 */
nvfp4_status nvfp4_quantize(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                            float* residual, const float* global_amax, nvfp4_round rnd,
                            uint32_t seed, uint32_t step, uint8_t* packed, uint8_t* scales,
                            void* stream);

/*
 * nvfp4_dequantize - NVFP4 -> bf16 or fp32 (fp4-train, API dequantize(packed,
 * scale, M, K) -> bf16).  x_hat = (val * s) * S_dec.
 *   tile16   0: scales [M, K/16] (1x16 blocks); 1: tile scales [M/16, K/16]
 *            (M % 16 == 0).
 *   global_amax, scale_mode, bound: the producer's second-level scale: mode
 *            NONE (global_amax ignored, S_dec = 1), TENSOR (global_amax[0]) or
 *            ROW (global_amax[0..M-1], 1x16 only); bound 448 (standard, 2D) or
 *            256/448 (four-over-six).
 *   out      [M, K] of out_dt.
 */
nvfp4_status nvfp4_dequantize(const uint8_t* packed, const uint8_t* scales, int64_t M,
                              int64_t K, int tile16, const float* global_amax,
                              nvfp4_scale_mode scale_mode, float bound, void* out,
                              nvfp4_dtype out_dt, void* stream);

/*
 * nvfp4_qdq - quantize then dequantize in one pass, "the value the tensor
 * cores use" (fp4-train, API qdq(x, stochastic, residual, seed, step)).
 * Arguments as nvfp4_quantize; out [M, K] of out_dt (bf16 as in the card);
 * packed_opt / scales_opt: NULL, or also receive the codes and scales.
 * With a residual this is one error-feedback step (fp4-train, Method).
 */
nvfp4_status nvfp4_qdq(const void* x, nvfp4_dtype dt, int64_t M, int64_t K, float* residual,
                       const float* global_amax, nvfp4_round rnd, uint32_t seed,
                       uint32_t step, void* out, nvfp4_dtype out_dt, uint8_t* packed_opt,
                       uint8_t* scales_opt, void* stream);

/*
 * nvfp4_quantize_4over6 - four-over-six NVFP4 quantize on 1x16 blocks (the
 * four-over-six pull request, What: four_over_six_quantize(x, global_amax,
 * block, err_mode, e4m3_scale_bound); numeric details; CuTe DSL kernel
 * Design).  Each block is encoded with sigma6 = (a / 6) * S_enc (map-to-6)
 * and sigma4 = sigma6 * 1.5 (map-to-4), RTN only; the candidate whose
 * dequantization error sum_i |x_i - d_i| (MAE) or sum_i (x_i - d_i)^2 (MSE),
 * d_i = ((val_i * s) * A) / (6*bound), accumulated in element order 0..15, is
 * strictly lower is kept; ties and NaN keep map-to-6.
 *   global_amax  mode TENSOR: global_amax[0] is read.  mode ROW: one amax
 *                per row; if amax_is_input != 0 they are read from
 *                global_amax[0..M-1], otherwise the kernel computes each
 *                row's NaN-dropping amax in the same pass and writes it there.
 *   err          NVFP4_MAE or NVFP4_MSE.   bound  256 or 448.
 *   packed [M, K/2], scales [M, K/16] out.
 */
nvfp4_status nvfp4_quantize_4over6(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                                   float* global_amax, nvfp4_scale_mode mode,
                                   int amax_is_input, nvfp4_err err, float bound,
                                   uint8_t* packed, uint8_t* scales, void* stream);

/*
 * nvfp4_quantize_2d - transposition-invariant 2D NVFP4 ("Stable FP4 Training
 * via Transposition-Invariant Block Quantization", abstract: one scale per
 * 16x16 tile shared by the forward and transposed operands, combined with
 * stochastic rounding).  M % 16 == 0.  Every element is encoded once (its
 * random draw keyed by its row-major index in X); the rowwise codes are
 * written to packed_row [M, K/2] and the same codes transposed to
 * packed_col [K, M/2] (NULL to skip), so packed_col is the rowwise packing of
 * Q(X)^T.  Block scale: a/6 without a global scale; with global_amax (one
 * fp32 amax) the standard sigma = a * (S_enc * (1/6)), bound 448.
 * truncation_free: 0 rounds the tile scale to the nearest e4m3 value; 1 takes
 * the smallest e4m3 value >= sigma, so no element exceeds 6 before rounding
 * (the paper's "truncation-free scaling"; this reading is the library's, the
 * abstract gives no formula).
 * tile_scales [M/16, K/16] out.
 */
nvfp4_status nvfp4_quantize_2d(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                               const float* global_amax, nvfp4_round rnd, uint32_t seed,
                               uint32_t step, int truncation_free, uint8_t* packed_row,
                               uint8_t* packed_col, uint8_t* tile_scales, void* stream);

/*
 * nvfp4_quantize_rowcol - the forward (rowwise) and the transposed
 * (columnwise) 1x16 NVFP4 operands of one tensor from a single read of it
 * (the four-over-six pull request, What: the backward pass quantizes the
 * transposed operands; Follow-up fusions: a fused row + column kernel
 * instead of x.t().contiguous() followed by a second quantize).
 * Round-to-nearest, one per-tensor global amax.  M % 16 == 0.
 *   global_amax   device pointer to one fp32 amax A (required).
 *   four_over_six 0: the standard encode, sigma = a * (S_enc * (1/6)); bound
 *                 must be 448 and err is ignored (but must be a valid value).
 *                 1: four-over-six per block (err, bound 256 or 448), as
 *                 nvfp4_quantize_4over6 with mode TENSOR.
 *   packed_row [M, K/2], scales_row [M, K/16]: blocks of 16 along K, equal
 *                 to nvfp4_quantize (RTN) / nvfp4_quantize_4over6 of x.
 *   packed_col [K, M/2], scales_col [K, M/16]: the same quantization of
 *                 X^T (blocks of 16 consecutive rows of one column), laid
 *                 out as the rowwise outputs of X^T.
 */
nvfp4_status nvfp4_quantize_rowcol(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                                   const float* global_amax, int four_over_six, nvfp4_err err,
                                   float bound, uint8_t* packed_row, uint8_t* scales_row,
                                   uint8_t* packed_col, uint8_t* scales_col, void* stream);

/*
 * nvfp4_quantize_4over6_2d - four-over-six on 16x16 tiles with one
 * per-tensor global amax (the four-over-six pull request, What: block
 * "16x16" with a scalar global_amax; CuTe DSL kernel Design: each tile row
 * sums its 16 errors in element order, the 16 row sums are combined by the
 * exact width-16 tree, map-to-4 iff its tile error is strictly lower).  One
 * scale per tile shared by X and X^T (transposition-invariant paper,
 * abstract), so the columnwise codes are the rowwise codes transposed.
 * M % 16 == 0.
 *   global_amax   device pointer to one fp32 amax A (required).
 *   err, bound    NVFP4_MAE / NVFP4_MSE; 256 or 448.
 *   packed_row [M, K/2]; packed_col [K, M/2] or NULL to skip;
 *   tile_scales [M/16, K/16].  Dequantize with nvfp4_dequantize(tile16 = 1,
 *   NVFP4_SCALE_TENSOR, bound).
 */
nvfp4_status nvfp4_quantize_4over6_2d(const void* x, nvfp4_dtype dt, int64_t M, int64_t K,
                                      const float* global_amax, nvfp4_err err, float bound,
                                      uint8_t* packed_row, uint8_t* packed_col,
                                      uint8_t* tile_scales, void* stream);

/*
 * Test support (not part of the quantization path).
 *
 * nvfp4_selftest_scan - exhaustive scan of one of the gfx950 conversions the
 * kernels use, through the same device helpers and operand placement, so a
 * test can compare every input pattern with the CPU oracle (the pages fix
 * what must be matched: satfinite round-to-nearest-even e2m1 and e4m3 casts,
 * four-over-six pull request, CuTe DSL kernel Design; stochastic rounding
 * with probability equal to the fractional distance, fp4-train card, Method).
 *   kind 0  fp32 -> e2m1 round-to-nearest of pattern p, param = SEL | slot << 2
 *           (byte SEL of the word, element a or b; the other element 0, the
 *           other bytes of the word 0xA5): y = the whole 32-bit word.
 *   kind 1  e4m3 scale byte of min(p, 448), param = slot (0 or 1): y = byte.
 *   kind 2  stochastic fp32 -> e2m1, param = u16 | SEL << 16 | slot << 18:
 *           the element in `slot` takes the 16-bit draw u16: y = byte SEL.
 *   kind 3  e2m1 byte p -> fp32 bits of element `half`, param = SEL | half << 2.
 *   kind 4  e4m3 code p -> fp32 bits, param = SEL (0 or 1).
 * Patterns first .. first + count - 1 (first + count <= 2^32; <= 256 for
 * kinds 3 and 4) are cut into chunks of 2^chunk_log2 (chunk_log2 0..24, at
 * most 2^22 chunks); records receives four uint32 per chunk (device memory,
 * 16-byte aligned): {y(first pattern), y(last pattern), number of patterns
 * p of the chunk with y(p) != y(p - 1), the first such p}.  Errors as for
 * the other entry points (NVFP4_E_ARG for a bad kind or chunk size,
 * NVFP4_E_RANGE for a run outside the pattern space).
 */
nvfp4_status nvfp4_selftest_scan(int kind, uint32_t param, uint64_t first, uint64_t count,
                                 int chunk_log2, uint32_t* records, void* stream);

/*
 * nvfp4_selftest_launch_plan - the launch geometry an entry point would use
 * for an [M, K] tensor, computed by the same host functions as the launchers
 * (no device work, no GPU needed), so a host test can check every accepted
 * shape against the dispatch limits.
 *   entry    0 quantize / qdq, 1 dequantize (variant 1: 16x16 tiles),
 *            2 quantize_4over6, 3 quantize_2d, 4 quantize_rowcol (variant 1:
 *            four-over-six), 5 quantize_4over6_2d (variant 1: with the
 *            columnwise output), 6 amax (variant 1: per row;
 *            for per tensor the plan is the partial pass).
 *   in_bf16  input dtype (it selects the four-over-six kernel).
 *   plan     HOST pointer to four int64: {kernel id, launches, workgroups of
 *            the largest launch, lanes per workgroup}.
 * Shapes are validated as by the entry point (NVFP4_E_SHAPE, NVFP4_E_RANGE).
 */
nvfp4_status nvfp4_selftest_launch_plan(int entry, int64_t M, int64_t K, int in_bf16, int variant,
                                        int64_t* plan);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
