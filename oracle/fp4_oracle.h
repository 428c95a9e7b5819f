/*
 * fp4_oracle.h -- CPU oracle for block-scaled FP4 quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow reference that the HIP
 * library is checked against.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load it; the product path never does.
 * It shares no code, header, table or constant with the HIP library.
 *
 * Sources (web pages on block-scaled FP4; cited by page title + section):
 *  [4/6]   "Four Over Six: more accurate NVFP4 quantization with adaptive
 *          block scaling" (page 3), sec. 1 (FP4 value set, worked example
 *          [10,20,30,40], Fig. 1) and sec. 2.1 (Eq. 1-3).
 *  [NVFP4] NVIDIA NVFP4 pretraining article (page 2), sec. 1 (16-value blocks,
 *          E4M3 block scale, FP32 tensor scale, MXFP4 = 32 values + UE8M0),
 *          sec. 2 (random Hadamard transform, 2D block scaling, stochastic
 *          rounding for gradients), sec. 6 (global encode scale 6*448/amax,
 *          local encode scale applied per element).
 *  [MXFP4] AMD MI355X MXFP4 pretraining article (page 4), sec. 2
 *          (deterministic Hadamard rotation before MXFP4 quantization).
 *  [QII]   Quartet II / MS-EDEN news article (page 1), sec. 2 (the backward
 *          pass quantizes part of the data again).
 *  [Philox] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *          1, 2, 3", SC'11 (Philox4x32-10).
 *
 * All floating point is IEEE binary32 with round-to-nearest-even, in the
 * operation order written in fp4_oracle.c; the only fused multiply-adds are
 * explicit fmaf() calls.  Build with -ffp-contract=off and no fast-math.
 */
#ifndef FP4_ORACLE_H
#define FP4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Mode flags (same bit values as the public interface; redefined here so the
 * oracle includes nothing of the library). */
#define ORC_FOUR_OVER_SIX (1u << 0)
#define ORC_SR            (1u << 1)
#define ORC_RHT16         (1u << 2)
#define ORC_BLOCK2D       (1u << 3)
#define ORC_HAD32         (1u << 4)
#define ORC_ROWWISE       (1u << 5)
#define ORC_COLWISE       (1u << 6)
#define ORC_MSEDEN        (1u << 7)   /* NVFP4: RTN values, stochastic E4M3 scale (needs RHT16) */

/* ---- number formats ---- */
uint8_t orc_e2m1_encode(float t);                /* 4-bit code, RNE, saturating */
float   orc_e2m1_decode(uint8_t code);
uint8_t orc_e4m3_encode(float x);                /* x >= 0; RNE, saturating at 448 */
float   orc_e4m3_decode(uint8_t code);
float   orc_ue8m0_decode(uint8_t code);          /* 2^(code-127) */
void    orc_e2m1_encode_array(const float* t, int64_t n, uint8_t* out);
void    orc_e4m3_encode_array(const float* x, int64_t n, uint8_t* out);

/* ---- random numbers and rotations ---- */
void     orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t orc_rht16_signs(uint64_t seed);         /* 16 sign bits, bit k set = negate x_k */
void     orc_fwht(float* v, int n);              /* unnormalised, in place, n = 16 or 32 */
void     orc_rotate_rht16(const float* x, uint32_t signs, float* y);  /* 16 values */
void     orc_rotate_had32(const float* x, float* y);                   /* 32 values */
float    orc_had32_norm(void);                   /* fp32 nearest to 1/sqrt(32) */

/* ---- the quantization path ---- */
typedef struct {
  /* optional per-element outputs, rows*cols each (row-major), may be NULL */
  float* t;        /* value handed to the FP4 rounding (chosen candidate)    */
  float* u;        /* SR uniform in [0,1) (SR only)                          */
  float* p;        /* SR round-up probability (SR only)                      */
  /* optional per-block outputs, one per block (layout of `scales`)         */
  float* dpre6;    /* unrounded block scale for M = 6; with MSEDEN the
                      corrected scale Delta' that is stochastically rounded */
  float* dpre4;    /* unrounded block scale for M = 4 (4/6 only)            */
  float* err6;     /* block squared error, M = 6 (4/6 only)                  */
  float* err4;     /* block squared error, M = 4 (4/6 only)                  */
} orc_debug;

/* Largest magnitude of the (optionally RHT16-rotated) tensor. */
float orc_tensor_amax(const uint16_t* x_bf16, int64_t rows, int64_t cols,
                      uint32_t flags, uint64_t seed);

/* NVFP4 quantization; returns 0 on success, a negative number for bad
 * arguments.  codes: [rows][cols/2]; scales: [rows][cols/16] (1D) or
 * [rows/16][cols/16] (2D); choice: same layout as scales (1 = M=4 chosen);
 * codes_t/scales_t: quantization of the transpose (2D only). */
int orc_nvfp4_quantize(const uint16_t* x_bf16, int64_t rows, int64_t cols,
                       uint32_t flags, uint64_t seed, const float* amax_in,
                       float* alpha_out, uint8_t* codes, uint8_t* scales,
                       uint8_t* choice, uint8_t* codes_t, uint8_t* scales_t,
                       orc_debug* dbg);

/* MXFP4 quantization: row-wise (codes_r [rows][cols/2], scales_r
 * [rows][cols/32]) and/or column-wise (codes_c [cols][rows/2], scales_c
 * [cols][rows/32]). t_r / t_c: optional pre-rounding values (row-major of
 * X resp. X^T). */
int orc_mxfp4_quantize(const uint16_t* x_bf16, int64_t rows, int64_t cols,
                       uint32_t flags, uint8_t* codes_r, uint8_t* scales_r,
                       uint8_t* codes_c, uint8_t* scales_c,
                       float* t_r, float* t_c);

/* NVFP4 quantization of an fp32 tensor (1D flags only: RTN6, FOUR_OVER_SIX,
 * SR, RHT16); the same definition as orc_nvfp4_quantize on fp32 values. */
int orc_nvfp4_quantize_f32(const float* x, int64_t rows, int64_t cols, uint32_t flags,
                           uint64_t seed, const float* amax_in, float* alpha_out,
                           uint8_t* codes, uint8_t* scales, uint8_t* choice);

/* NVFP4 (1D flags) with one FP32 scale per row: row r uses alpha_r =
 * amax_r / (6 C) from its own largest magnitude (after RHT16); alpha_rows
 * [rows].  Otherwise identical to orc_nvfp4_quantize. */
int orc_nvfp4_quantize_rows(const uint16_t* x_bf16, int64_t rows, int64_t cols,
                            uint32_t flags, uint64_t seed, float* alpha_rows,
                            uint8_t* codes, uint8_t* scales, uint8_t* choice);

/* The two above (1D flags) on rows row0 .. row0 + rows - 1 of a larger
 * tensor with `cols` columns, passed alone: the random counters (SR element
 * index, MS-EDEN block index) are the whole tensor's, and orc_nvfp4_quantize_at
 * takes the whole tensor's amax (amax_in, required).  row0 = 0 gives the
 * functions above. */
int orc_nvfp4_quantize_at(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t row0,
                          uint32_t flags, uint64_t seed, const float* amax_in,
                          float* alpha_out, uint8_t* codes, uint8_t* scales,
                          uint8_t* choice);
int orc_nvfp4_quantize_rows_at(const uint16_t* x_bf16, int64_t rows, int64_t cols,
                               int64_t row0, uint32_t flags, uint64_t seed,
                               float* alpha_rows, uint8_t* codes, uint8_t* scales,
                               uint8_t* choice);

/* Requantize a 1D NVFP4 tensor X [rows][cols] (codes, scales, alpha) for the
 * transposed operand: NVFP4 (flags as above) of dequantize(X)^T, giving
 * codes_t [cols][rows/2], scales_t [cols][rows/16], choice_t (or NULL).
 * rows % 16 == 0, cols % 16 == 0.  Parity pinned against the bf16 path on
 * inputs whose dequantized values are bf16-exact (see the tests). */
int orc_nvfp4_requantize_t(const uint8_t* codes, const uint8_t* scales, float alpha,
                           int64_t rows, int64_t cols, uint32_t flags, uint64_t seed,
                           float* alpha_out, uint8_t* codes_t, uint8_t* scales_t,
                           uint8_t* choice_t);

/* orc_nvfp4_requantize_t of columns col0 .. col0 + cols - 1 of a larger X
 * (their codes [rows][cols/2] and scales [rows][cols/16], all rows): output
 * rows col0 .. col0 + cols - 1 of the whole transpose, with the whole output
 * tensor's amax (amax_in, required) and its SR element indices. */
int orc_nvfp4_requantize_t_at(const uint8_t* codes, const uint8_t* scales, float alpha,
                              int64_t rows, int64_t cols, int64_t col0, uint32_t flags,
                              uint64_t seed, const float* amax_in, float* alpha_out,
                              uint8_t* codes_t, uint8_t* scales_t, uint8_t* choice_t);

/* Dequantization. format 0 = NVFP4 (alpha used, BLOCK2D selects 16x16
 * tiles), 1 = MXFP4 (row-wise layout; pass the transposed shape for the
 * column-wise outputs). */
int orc_dequantize(int format, const uint8_t* codes, const uint8_t* scales,
                   float alpha, int64_t rows, int64_t cols, uint32_t flags,
                   float* out);

/* Simulated NVFP4 for the error study of [4/6] sec. 2.2 (Fig. 2): the 1D
 * RTN6 quantize-then-dequantize of x [rows][cols] (bf16, cols % 16 == 0)
 * into out (fp32), with one source of error switched off:
 *   ORC_SIM_NVFP4      nothing switched off: out = dequantize(quantize(x))
 *   ORC_SIM_SCALE_HP   the block scale is not rounded to E4M3 (Delta kept
 *                      in fp32)
 *   ORC_SIM_VALUE_HP   the scaled values X/(alpha Delta) are not rounded
 *                      to FP4 (kept in fp32)
 *   ORC_SIM_THRESHOLD  a scaled value t is rounded to FP4 only when
 *                      |t| < thr; the others are kept in fp32
 * Returns 0, or -1 for a bad shape or mode. */
#define ORC_SIM_NVFP4     0
#define ORC_SIM_SCALE_HP  1
#define ORC_SIM_VALUE_HP  2
#define ORC_SIM_THRESHOLD 3
int orc_nvfp4_simulate(const uint16_t* x_bf16, int64_t rows, int64_t cols, int mode,
                       float thr, float* out);

#ifdef __cplusplus
}
#endif
#endif
