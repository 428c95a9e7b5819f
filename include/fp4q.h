/*
 * fp4q.h -- block-scaled FP4 quantization of bf16 tensors on AMD MI355X
 * (gfx950).  C ABI of libfp4q.so.
 *
 * The method (cited by page title and section):
 *  - NVFP4: FP4 E2M1 values, one FP8 E4M3 scale per 16 consecutive values
 *    and one FP32 tensor scale ("Four Over Six: More Accurate NVFP4
 *    Quantization with Adaptive Block Scaling", sec. 2.1, Eq. 1-3; NVIDIA
 *    NVFP4 pretraining article, sec. 1 and sec. 6).
 *  - Four Over Six: per 16-value block, quantize with the block maximum
 *    scaled to 6 and to 4 and keep the one with the smaller error ("Four
 *    Over Six", sec. 1, Fig. 1 and the worked example).
 *  - Variants for the tensors of a training step (NVIDIA NVFP4 article,
 *    sec. 2 and sec. 7): a 16-point random Hadamard rotation and stochastic
 *    rounding for gradients, 16x16 two-dimensional blocks for weights.
 *  - MXFP4: 32 values per power-of-two (UE8M0) scale (NVIDIA NVFP4 article,
 *    sec. 1 and sec. 5), with a fixed 32-point Hadamard rotation (AMD
 *    MI355X MXFP4 pretraining article, sec. 2) and row- and column-wise
 *    outputs.
 *
 * Conventions shared by every call:
 *  - Every tensor pointer is a DEVICE pointer (HIP device memory of the
 *    current device).  The caller allocates every buffer and owns it; the
 *    library allocates nothing and keeps no state between calls (except the
 *    fixed per-device array of nvfp4_quantize_noalloc).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is queued on it asynchronously; the call returns before the GPU
 *    finishes.  Concurrent calls on different streams are safe as long as
 *    they do not share output or workspace buffers.
 *  - Inputs are row-major bf16 bit patterns [rows][cols], 16-byte aligned.
 *  - Packed FP4 codes: two per byte, the even-indexed element in the low
 *    nibble; code = sign << 3 | magnitude index into {0, .5, 1, 1.5, 2, 3,
 *    4, 6}.  Code buffers must be 16-byte aligned.
 *  - Scales are one byte per block in row-major block order; NVFP4 scales
 *    are E4M3 (bias 7, max 448), MXFP4 scales are UE8M0 (2^(code-127)).
 *  - Errors: the return value is an fp4_status.  Argument checks run on the
 *    host before any HIP call, so a rejected call touches no device state.
 *    FP4_E_HIP reports a failed kernel launch (the launch's own return
 *    status; an error left by an earlier, unrelated HIP call is neither
 *    reported nor cleared); faults during execution surface at the caller's
 *    next synchronisation.
 *  - Tensors holding Inf/NaN, or (NVFP4) whose largest magnitude is below
 *    2^-64 without being zero, are outside the method's domain: the call
 *    succeeds and never faults, but codes and scales are unspecified.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP4_OK = 0,
  FP4_E_NULL = -1,      /* a required pointer is NULL                     */
  FP4_E_SHAPE = -2,     /* rows/cols negative, not a block multiple, or
                           rows*cols >= 2^40                              */
  FP4_E_ALIGN = -3,     /* a pointer breaks the alignment rules above     */
  FP4_E_FLAGS = -4,     /* unknown bit or an unsupported combination      */
  FP4_E_WORKSPACE = -5, /* workspace smaller than fp4_workspace_bytes()   */
  FP4_E_HIP = -6        /* kernel launch failed                           */
} fp4_status;

/* Mode flags. */
enum {
  FP4_RTN6 = 0u,               /* NVFP4, block max scaled to 6, nearest-even  */
  FP4_FOUR_OVER_SIX = 1u << 0, /* NVFP4: adaptive choice of 6 or 4 per block  */
  FP4_SR = 1u << 1,            /* NVFP4: stochastic rounding of FP4 values    */
  FP4_RHT16 = 1u << 2,         /* NVFP4: 16-point random Hadamard along rows  */
  FP4_BLOCK2D = 1u << 3,       /* NVFP4: 16x16 tiles instead of 1x16 blocks   */
  FP4_HAD32 = 1u << 4,         /* MXFP4: 32-point Hadamard before quantizing  */
  FP4_ROWWISE = 1u << 5,       /* MXFP4: emit row-wise output                 */
  FP4_COLWISE = 1u << 6,       /* MXFP4: emit column-wise output;
                                  NVFP4 2D: also emit the transpose          */
  FP4_MSEDEN = 1u << 7         /* NVFP4: MS-EDEN -- RTN values, unbiasing
                                  factor, stochastic E4M3 scale (with RHT16) */
};

enum { FP4_FORMAT_NVFP4 = 0, FP4_FORMAT_MXFP4 = 1 };

/* Bytes of device workspace nvfp4_quantize and nvfp4_requantize_t (with
 * amax_in == NULL) and fp4_tensor_amax need for this shape and these
 * flags; 0 if none.  The
 * workspace needs no initialisation and is scratch for the duration of the
 * call (stream order). */
size_t fp4_workspace_bytes(int64_t rows, int64_t cols, uint32_t flags);

/* Largest magnitude of the tensor the NVFP4 quantizer scales by ("Four Over
 * Six" Eq. 1 numerator; NVIDIA NVFP4 article sec. 6 and sec. 9: the extra
 * pass over memory for the global scale).  With FP4_RHT16 it is the
 * largest magnitude after the rotation (seeded by `seed`).  Other NVFP4 flag
 * bits are accepted and ignored; FP4_HAD32 is rejected.
 *   x        [rows][cols] bf16, cols % 16 == 0
 *   amax_out one float (device), written in stream order
 *   ws       fp4_workspace_bytes(rows, cols, flags) bytes (device) */
int fp4_tensor_amax(const uint16_t* x, int64_t rows, int64_t cols,
                    uint32_t flags, uint64_t seed, float* amax_out,
                    void* ws, size_t ws_bytes, void* stream);

/* NVFP4 quantization ("Four Over Six" Eq. 1-3 and sec. 1; NVIDIA NVFP4
 * article sec. 2 and sec. 6).
 *   flags     FP4_RTN6 or any of FOUR_OVER_SIX, SR, RHT16, BLOCK2D
 *             (+ COLWISE with BLOCK2D), or MSEDEN|RHT16.  Rejected:
 *             SR|FOUR_OVER_SIX, BLOCK2D|SR, BLOCK2D|RHT16, HAD32, COLWISE
 *             without BLOCK2D, MSEDEN without RHT16 or with SR,
 *             FOUR_OVER_SIX or BLOCK2D.
 *             MSEDEN (Quartet II / MS-EDEN article, sec. 1: rotation,
 *             round-to-nearest values, randomness only in the 8-bit scale;
 *             the unbiasing factor is EDEN's): per block the values are
 *             rounded to nearest against the unrounded scale Delta_pre,
 *             the scale becomes S * Delta_pre with S = sum t^2 / sum t q
 *             and is rounded stochastically to E4M3 (Philox counter =
 *             (block index lo, hi, 1, 0)); C = 256.
 *   seed      Philox key for SR (counter = row*cols + col) and RHT16 signs.
 *   amax_in   NULL: computed here (one extra read of x, needs `ws`);
 *             else one device float taken as the tensor's largest magnitude.
 *   alpha_out one device float: the FP32 tensor scale amax/(6*C), C = 448,
 *             or 256 with FOUR_OVER_SIX.
 *   codes     [rows][cols/2] bytes.
 *   scales    E4M3, [rows][cols/16] (1D) or [rows/16][cols/16] (BLOCK2D).
 *   choice    NULL or one byte per scale, 1 where the block took M = 4.
 *   codes_t, scales_t  BLOCK2D|COLWISE only (else NULL): the same
 *             quantization laid out for the transpose, [cols][rows/2] and
 *             [cols/16][rows/16].
 *   Shapes: cols % 16 == 0; BLOCK2D also rows % 16 == 0. */
int nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols,
                   uint32_t flags, uint64_t seed, const float* amax_in,
                   float* alpha_out, uint8_t* codes, uint8_t* scales,
                   uint8_t* choice, uint8_t* codes_t, uint8_t* scales_t,
                   void* ws, size_t ws_bytes, void* stream);

/* nvfp4_quantize for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call without a workspace argument.  With amax_in ==
 * NULL the amax pass keeps its per-workgroup partial maxima in a fixed
 * 4 KiB device array of the library (one per device, held until the process
 * ends; its address is looked up once per device on the first call there)
 * instead of caller memory.  The call allocates nothing.
 *   Arguments, results and errors as nvfp4_quantize; FP4_E_WORKSPACE if the
 *   shape and flags would need more than that array (never for the flag
 *   sets nvfp4_quantize accepts).
 *   Every call on one device shares that array: calls that overlap in time
 *   on one device (different streams, or host threads) race and may produce
 *   wrong results; calls in one stream's order are safe.  Nothing in it
 *   needs to start at zero (each call writes every partial it reads). */
int nvfp4_quantize_noalloc(const uint16_t* x, int64_t rows, int64_t cols,
                           uint32_t flags, uint64_t seed, const float* amax_in,
                           float* alpha_out, uint8_t* codes, uint8_t* scales,
                           uint8_t* choice, uint8_t* codes_t, uint8_t* scales_t,
                           void* stream);

/* NVFP4 with one FP32 scale per row, quantized in a single read of x.  The
 * NVIDIA NVFP4 article (sec. 9) names the extra memory pass for the global
 * scale as a cost and proposes finer-grained global scales, per row or per
 * block.  Row r takes alpha_r = amax_r / (6*C) ("Four Over Six" Eq. 1 on
 * the row; C = 448, or 256 with FOUR_OVER_SIX; amax after RHT16 when asked)
 * and is otherwise quantized exactly as nvfp4_quantize would quantize it
 * (Eq. 2-3, 4/6, SR with counter = row*cols + col).  Results differ from
 * nvfp4_quantize wherever rows have different maxima; a consumer decodes
 * row r with alpha_rows[r].
 *   flags      FP4_RTN6 or FOUR_OVER_SIX, SR, RHT16 (SR|FOUR_OVER_SIX
 *              rejected); BLOCK2D, COLWISE, ROWWISE and HAD32 rejected.
 *   alpha_rows [rows] device floats.
 *   codes      [rows][cols/2];  scales [rows][cols/16];  choice NULL or
 *              [rows][cols/16].
 *   Shapes: cols % 16 == 0.  No workspace.
 *   Domain, per row: a row whose largest magnitude (after RHT16) is not
 *   zero but below 2^-64 (e.g. a row of bf16 subnormals) is outside the
 *   method's domain, as a whole tensor with that amax would be: its codes,
 *   scales and choice are unspecified (its alpha_rows entry is still
 *   amax_r / (6*C)).  The other rows are unaffected and the call never
 *   faults. */
int nvfp4_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols,
                        uint32_t flags, uint64_t seed, float* alpha_rows,
                        uint8_t* codes, uint8_t* scales, uint8_t* choice,
                        void* stream);

/* Requantization of a 1D NVFP4 tensor for the transposed operand: the
 * NVFP4 quantization of dequantize(X)^T, with its own tensor scale.  The
 * backward pass quantizes data a second time (Quartet II / MS-EDEN
 * article, sec. 2); the weight gradient contracts over the other
 * dimension, so its operand needs blocks along the other axis (NVIDIA
 * NVFP4 article, sec. 7).  Dequantization is q * (alpha * Delta) in fp32
 * (NVIDIA NVFP4 article, sec. 6); the result equals nvfp4_quantize applied
 * to that fp32 transpose ("Four Over Six" Eq. 1-3), bit for bit.
 *   codes, scales, alpha  the input as a 1D nvfp4_quantize writes it:
 *             codes [rows][cols/2], scales [rows][cols/16] (finite E4M3
 *             codes; the sign bit is ignored, 0x7F is outside the domain),
 *             alpha one device float.
 *   flags     FP4_RTN6 or FOUR_OVER_SIX, SR, RHT16, as for a 1D
 *             nvfp4_quantize (SR|FOUR_OVER_SIX rejected); BLOCK2D, COLWISE,
 *             ROWWISE and HAD32 rejected.
 *   seed      Philox key: SR counter = element index in the output
 *             (out_row * rows + out_col); RHT16 signs as nvfp4_quantize.
 *             The rotation runs along output rows.
 *   amax_in   NULL: the output's largest magnitude (after RHT16 when
 *             asked) is computed here (one extra read of the input, needs
 *             `ws`); else one device float taken as that magnitude.
 *   alpha_out one device float: the output's tensor scale.
 *   codes_t   [cols][rows/2];  scales_t [cols][rows/16];
 *   choice_t  NULL or [cols][rows/16], 1 where the block took M = 4.
 *   ws        fp4_workspace_bytes(rows, cols, flags) bytes (device), or
 *             NULL with amax_in.
 *   Shapes: rows % 16 == 0 and cols % 16 == 0. */
int nvfp4_requantize_t(const uint8_t* codes, const uint8_t* scales, const float* alpha,
                       int64_t rows, int64_t cols, uint32_t flags, uint64_t seed,
                       const float* amax_in, float* alpha_out, uint8_t* codes_t,
                       uint8_t* scales_t, uint8_t* choice_t, void* ws, size_t ws_bytes,
                       void* stream);

/* MXFP4 quantization (NVIDIA NVFP4 article sec. 1 and 5; AMD MI355X MXFP4
 * article sec. 2).  Per 32 values: optional 32-point Hadamard (FP4_HAD32,
 * orthonormal), exponent e = floor(log2(amax)) - 2 (UE8M0 code e + 127,
 * 0 for an all-zero group), values scaled by 2^-e and rounded to nearest
 * even E2M1, saturating at 6.
 *   flags     HAD32 optional; ROWWISE and/or COLWISE (at least one).
 *   codes_r   [rows][cols/2], scales_r [rows][cols/32]   (ROWWISE, cols % 32 == 0)
 *   codes_c   [cols][rows/2], scales_c [cols][rows/32]   (COLWISE, rows % 32 == 0):
 *             the row-wise quantization of the transpose; the rotation and
 *             the 32-value groups run down the columns.
 *   Shapes: cols % 8 == 0 always (16-byte rows), plus the multiples above.
 *   Unused outputs may be NULL. */
int mxfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols,
                   uint32_t flags, uint8_t* codes_r, uint8_t* scales_r,
                   uint8_t* codes_c, uint8_t* scales_c, void* stream);

/* MXFP4 matrix product C = A B, the consumer of the quantized tensors
 * (NVIDIA NVFP4 article sec. 1 and 5: MXFP4, E2M1 values with a UE8M0
 * scale per 32, multiplied directly by block-scaled matrix hardware; AMD
 * MI355X MXFP4 article sec. 2: training with both operands in MXFP4), on
 * gfx950's block-scaled FP4 matrix instructions with fp32 accumulation.
 *   a_codes [M][K/2], a_scales [M][K/32]   A in the row-wise MXFP4 layout
 *                                          (mxfp4_quantize ROWWISE of A)
 *   bt_codes [N][K/2], bt_scales [N][K/32] B^T in the same layout (the
 *                                          COLWISE output of mxfp4_quantize
 *                                          applied to B [K][N])
 *   c  [M][N] fp32, row-major.
 *   With HAD32 on both operands the rotations along K cancel in the product
 *   (the 32-point Hadamard is orthonormal), up to rounding.
 *   Shapes: K % 128 == 0, K < 2^23, N < 2^20, M*N < 2^40; M, N >= 0.  Code
 *   buffers 16-byte aligned, scale buffers and c 4-byte aligned. */
int mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* bt_codes,
               const uint8_t* bt_scales, int64_t M, int64_t N, int64_t K, float* c,
               void* stream);

/* Dequantize to fp32 [rows][cols] (the decode applied by the consumer:
 * NVIDIA NVFP4 article sec. 4 and sec. 6).
 *   format FP4_FORMAT_NVFP4: out = q * (alpha * Delta), alpha = *alpha
 *          (device float); flags FP4_BLOCK2D selects 16x16 tiles.
 *   format FP4_FORMAT_MXFP4: out = q * 2^(code-127); alpha ignored (may be
 *          NULL); pass (cols, rows) of the original to decode COLWISE output.
 *   out    16-byte aligned. */
int fp4_dequantize(int format, const uint8_t* codes, const uint8_t* scales,
                   const float* alpha, int64_t rows, int64_t cols,
                   uint32_t flags, float* out, void* stream);

/* Static description of a status code. */
const char* fp4_status_str(int status);

/* Interface version (bumped on any incompatible change). */
int fp4_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FP4Q_H */
