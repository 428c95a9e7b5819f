/*
 * fp4_oracle.c -- CPU oracle for block-scaled FP4 quantization.
 *
 * TEST INFRASTRUCTURE ONLY (see fp4_oracle.h): plain, slow, single-threaded
 * C that follows the method step by step.  Every function names the passage
 * it follows.  Where the pages leave a step open, the reading taken is stated
 * next to the code.
 *
 * Parity status of each part:
 *   E2M1 / E4M3 / UE8M0 formats ........ pinned (value set, brute force,
 *                                         Eq. 3 literal form, torch fp8 cast)
 *   Eq. 1-3 + Four Over Six ............. pinned (worked example, Fig. 1
 *                                         invariants, brute force per block)
 *   Hadamard rotations .................. pinned (dense Sylvester matrix,
 *                                         orthogonality, norm, one-hot)
 *   Philox4x32-10 ....................... pinned (published known answers)
 *   stochastic rounding ................. pinned (unbiasedness, P(up) = p,
 *                                         grid points fixed)
 *   2D tiles ............................ pinned (transpose identity)
 *   MXFP4 ............................... pinned (power-of-two scales,
 *                                         scaled block max in [4, 8), hand cases)
 *   requantization for the transpose .... pinned (equals the bf16 path when
 *                                         the dequantized values are bf16-exact)
 *   one scale per row ................... pinned (each row = the per-tensor
 *                                         quantizer on that row alone)
 *   error-study simulation .............. pinned (no switch = dequantize of
 *                                         the quantizer, sweep end points)
 *   row / column bands of a larger tensor  pinned (equal to the whole-tensor
 *                                         results for those rows; a wrong
 *                                         offset changes the random draws)
 *   MS-EDEN ............................. partly pinned: the unbiasing factor
 *                                         is not on the pages (EDEN's is taken);
 *                                         its projection property, nearest
 *                                         values, scale-rounding statistics,
 *                                         removed scale bias, error vs SR
 *   exact fp32 operation order of the 4/6 error sum, the SR word-to-uniform
 *   mapping and the RHT sign source are choices where the pages are silent;
 *   they are fixed here and pinned only by the properties above.
 */
#include "fp4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ===================================================================== */
/* Number formats                                                         */
/* ===================================================================== */

/* FP4 E2M1 magnitudes: the 8 non-negative values of the 16-value set
 * +-{0, 0.5, 1, 1.5, 2, 3, 4, 6} ([4/6] sec. 1). Index = 3-bit magnitude code. */
static const float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

/* Round-to-nearest onto the E2M1 grid ([4/6] Eq. 3).  Eq. 3 rounds 2v, v and
 * v/2 to integers on [0,2), [2,4) and [4,6]; with ties to even (the rounding
 * mode named in [NVFP4] sec. 4) this is exactly round-to-nearest-even on the
 * grid, written here as the midpoints between neighbours.  Midpoints go to
 * the neighbour with the even magnitude code.  Eq. 3 stops at |v| <= 6; larger
 * values saturate to 6 (the worked example scales 40 to 6.15 and keeps 6).
 * The sign bit is kept, so -0 and small negatives encode as 0x8. */
uint8_t orc_e2m1_encode(float t) {
  float a = fabsf(t);
  uint8_t m;
  if (a <= 0.25f)      m = 0;   /* tie 0.25 -> 0   */
  else if (a < 0.75f)  m = 1;   /* tie 0.75 -> 1.0 */
  else if (a <= 1.25f) m = 2;   /* tie 1.25 -> 1.0 */
  else if (a < 1.75f)  m = 3;   /* tie 1.75 -> 2.0 */
  else if (a <= 2.5f)  m = 4;   /* tie 2.5  -> 2.0 */
  else if (a < 3.5f)   m = 5;   /* tie 3.5  -> 4.0 */
  else if (a <= 5.0f)  m = 6;   /* tie 5.0  -> 4.0 */
  else                 m = 7;   /* (5, inf) -> 6, saturating */
  return (uint8_t)((signbit(t) ? 0x8u : 0x0u) | m);
}

float orc_e2m1_decode(uint8_t code) {
  float v = kE2M1[code & 7u];
  return (code & 8u) ? -v : v;
}

void orc_e2m1_encode_array(const float* t, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = orc_e2m1_encode(t[i]);
}

/* FP8 E4M3 (the "FN" variant: exponent bias 7, 3 mantissa bits, largest
 * finite 448, no infinity, 0x7F = NaN) used for NVFP4 block scales
 * ([NVFP4] sec. 1: "E4M3 instead of UE8M0"; [4/6] sec. 2.1: M^FP8 = 448).
 * Rounding: nearest, ties to even; values past 448 saturate to 448. */
uint8_t orc_e4m3_encode(float x) {
  if (!(x > 0.0f)) return 0;                 /* +0, -0 and NaN encode as 0 */
  if (isinf(x)) return 0x7E;
  int e2;
  frexp((double)x, &e2);                     /* x = f * 2^e2, f in [0.5, 1) */
  int E = e2 - 1;                            /* x in [2^E, 2^(E+1))         */
  if (E < -6) E = -6;                        /* subnormals share 2^-6's step */
  double quantum = ldexp(1.0, E - 3);        /* 3 mantissa bits             */
  double n = nearbyint((double)x / quantum); /* exact scaling, RNE          */
  /* n in [0, 16]; code = biased exponent * 8 + (n - 8); n = 16 carries into
   * the next exponent and, at E = -6 with n < 8, gives a subnormal code. */
  long code = ((long)(E + 7) << 3) + (long)n - 8;
  if (code > 0x7E) code = 0x7E;              /* saturate at 448             */
  return (uint8_t)code;
}

float orc_e4m3_decode(uint8_t code) {
  code &= 0x7Fu;
  if (code == 0x7F) return NAN;
  int e = code >> 3, m = code & 7;
  if (e == 0) return (float)ldexp((double)m, -9);
  return (float)ldexp(1.0 + m / 8.0, e - 7);
}

void orc_e4m3_encode_array(const float* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = orc_e4m3_encode(x[i]);
}

/* UE8M0 power-of-two scale of MXFP4 ([NVFP4] sec. 1 and sec. 5). */
float orc_ue8m0_decode(uint8_t code) { return (float)ldexp(1.0, (int)code - 127); }

/* ===================================================================== */
/* Philox4x32-10 (Salmon et al., SC'11)                                    */
/* ===================================================================== */

/* One Philox4x32 round: two 32x32->64 multiplications of counter words 0
 * and 2 by the round multipliers; the high halves are mixed with the other
 * two counter words and the round key; the words are permuted. */
static void philox_round(uint32_t c[4], const uint32_t k[2]) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
  const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  uint32_t n0 = hi1 ^ c[1] ^ k[0];
  uint32_t n1 = lo1;
  uint32_t n2 = hi0 ^ c[3] ^ k[1];
  uint32_t n3 = lo0;
  c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

/* Ten rounds; the key is bumped by the Weyl constants (golden ratio and
 * sqrt(3)-1 in 32-bit fixed point) before every round after the first. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int r = 0; r < 10; r++) {
    if (r > 0) { k[0] += 0x9E3779B9u; k[1] += 0xBB67AE85u; }
    philox_round(c, k);
  }
  out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

/* ===================================================================== */
/* Hadamard rotations ([NVFP4] sec. 2 and 7; [MXFP4] sec. 2)              */
/* ===================================================================== */

/* Sign diagonal of the randomized Hadamard transform.  The pages only say
 * "random Hadamard"; reading: one +-1 vector of length 16 for the whole
 * tensor, taken from bits 0..15 of word 0 of Philox4x32-10 with key = seed
 * and counter = (0, 0, 0, 1); bit k set means x_k is negated. */
uint32_t orc_rht16_signs(uint64_t seed) {
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  const uint32_t ctr[4] = {0u, 0u, 0u, 1u};
  uint32_t w[4];
  orc_philox4x32_10(ctr, key, w);
  return w[0] & 0xFFFFu;
}

/* Fast Walsh-Hadamard transform (Sylvester / natural order), unnormalised:
 * stage h = 1, 2, 4, ... pairs (j, j+h) for every j with bit h clear and
 * replaces them by (sum, difference), each rounded to fp32. */
void orc_fwht(float* v, int n) {
  for (int h = 1; h < n; h <<= 1) {
    for (int j = 0; j < n; j++) {
      if (j & h) continue;
      float a = v[j], b = v[j + h];
      v[j] = a + b;
      v[j + h] = a - b;
    }
  }
}

/* 16-point randomized Hadamard: y = (1/4) H16 D x (D = sign diagonal,
 * applied first). 1/4 makes the rotation orthonormal and is exact. */
void orc_rotate_rht16(const float* x, uint32_t signs, float* y) {
  float v[16];
  for (int k = 0; k < 16; k++) v[k] = ((signs >> k) & 1u) ? -x[k] : x[k];
  orc_fwht(v, 16);
  for (int k = 0; k < 16; k++) y[k] = v[k] * 0.25f;
}

/* fp32 value nearest to 1/sqrt(32) = 2^-2.5 (bit pattern 0x3E3504F3). */
float orc_had32_norm(void) { return 0x1.6a09e6p-3f; }

/* Deterministic 32-point Hadamard: y = H32 x / sqrt(32), no random signs. */
void orc_rotate_had32(const float* x, float* y) {
  float v[32];
  for (int k = 0; k < 32; k++) v[k] = x[k];
  orc_fwht(v, 32);
  const float s = orc_had32_norm();
  for (int k = 0; k < 32; k++) y[k] = v[k] * s;
}

/* ===================================================================== */
/* Helpers                                                                */
/* ===================================================================== */

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static void put_nibble(uint8_t* row, int64_t j, uint8_t code) {
  /* element 2i in the low nibble of byte i, element 2i+1 in the high one */
  if (j & 1) row[j >> 1] = (uint8_t)((row[j >> 1] & 0x0Fu) | (code << 4));
  else       row[j >> 1] = (uint8_t)((row[j >> 1] & 0xF0u) | (code & 0x0Fu));
}

static uint8_t get_nibble(const uint8_t* row, int64_t j) {
  return (j & 1) ? (uint8_t)(row[j >> 1] >> 4) : (uint8_t)(row[j >> 1] & 0x0Fu);
}

/* Convert the input (bf16 x, or fp32 xf when x is NULL) to fp32 and apply
 * the row rotation the flags ask for (RHT16 on consecutive 16-value groups
 * of each row). */
static float* load_rotated(const uint16_t* x, const float* xf, int64_t rows, int64_t cols,
                           uint32_t flags, uint64_t seed) {
  float* y = (float*)malloc(sizeof(float) * (size_t)(rows * cols > 0 ? rows * cols : 1));
  if (!y) return NULL;
  for (int64_t i = 0; i < rows * cols; i++) y[i] = x ? bf16_to_f32(x[i]) : xf[i];
  if (flags & ORC_RHT16) {
    const uint32_t signs = orc_rht16_signs(seed);
    float g[16];
    for (int64_t r = 0; r < rows; r++)
      for (int64_t c = 0; c < cols; c += 16) {
        orc_rotate_rht16(&y[r * cols + c], signs, g);
        memcpy(&y[r * cols + c], g, sizeof g);
      }
  }
  return y;
}

static int nvfp4_flags_ok(int64_t rows, int64_t cols, uint32_t flags) {
  if (rows < 0 || cols < 0) return 0;
  if (flags & ~(ORC_FOUR_OVER_SIX | ORC_SR | ORC_RHT16 | ORC_BLOCK2D | ORC_ROWWISE | ORC_COLWISE |
                ORC_MSEDEN)) return 0;
  if ((flags & ORC_MSEDEN) &&
      (!(flags & ORC_RHT16) || (flags & (ORC_SR | ORC_FOUR_OVER_SIX | ORC_BLOCK2D)))) return 0;
  if ((flags & ORC_SR) && (flags & ORC_FOUR_OVER_SIX)) return 0;
  if ((flags & ORC_BLOCK2D) && (flags & (ORC_SR | ORC_RHT16))) return 0;
  if ((flags & ORC_COLWISE) && !(flags & ORC_BLOCK2D)) return 0;
  if (cols % 16) return 0;
  if ((flags & ORC_BLOCK2D) && rows % 16) return 0;
  return 1;
}

/* ===================================================================== */
/* Tensor scale ([4/6] Eq. 1; [NVFP4] sec. 6 and sec. 9)                  */
/* ===================================================================== */

float orc_tensor_amax(const uint16_t* x, int64_t rows, int64_t cols,
                      uint32_t flags, uint64_t seed) {
  if (!nvfp4_flags_ok(rows, cols, flags)) return NAN;
  float* y = load_rotated(x, NULL, rows, cols, flags, seed);
  float amax = 0.0f;
  for (int64_t i = 0; i < rows * cols; i++) {
    float a = fabsf(y[i]);
    if (a > amax) amax = a;
  }
  free(y);
  return amax;
}

/* ===================================================================== */
/* NVFP4 quantization ([4/6] Eq. 1-3, sec. 1; [NVFP4] sec. 1, 2, 6)       */
/* ===================================================================== */

/* Stochastic rounding of one scaled value ([NVFP4] sec. 2: unbiased
 * rounding for gradients).  Between the two neighbouring grid magnitudes
 * lo <= a < hi the value rounds up with probability p = (a - lo)/(hi - lo)
 * (exact in fp32: the subtraction is exact and hi - lo is a power of two).
 * The uniform u is the top 24 bits of Philox word 0 for counter =
 * (element index low, high, 0, 0) and key = seed, scaled by 2^-24; round up
 * iff u < p.  Values at or above 6 saturate. */
static uint8_t e2m1_sr(float t, uint64_t seed, uint64_t idx, float* u_out, float* p_out) {
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  const uint32_t ctr[4] = {(uint32_t)idx, (uint32_t)(idx >> 32), 0u, 0u};
  uint32_t w[4];
  orc_philox4x32_10(ctr, key, w);
  const float u = (float)(w[0] >> 8) * 0x1p-24f;
  const float a = fabsf(t);
  uint8_t m;
  float p = 0.0f;
  if (!(a < 6.0f)) {
    m = 7;
  } else {
    int lo = 0;
    while (lo < 7 && kE2M1[lo + 1] <= a) lo++;       /* kE2M1[lo] <= a < kE2M1[lo+1] */
    p = (a - kE2M1[lo]) / (kE2M1[lo + 1] - kE2M1[lo]);
    m = (uint8_t)((u < p) ? lo + 1 : lo);
  }
  if (u_out) *u_out = u;
  if (p_out) *p_out = p;
  return (uint8_t)((signbit(t) ? 0x8u : 0x0u) | m);
}

/* Quantize one block for one target maximum M.
 *   elems: pointers to the block's values in a fixed order; for a 1D block
 *          16 values, for a 2D tile 16 rows of 16 values (row by row).
 *   The block scale follows Eq. 2 with the division by alpha*M carried out as
 *   a multiplication by the per-tensor encode factor k_M ([NVFP4] sec. 6:
 *   block amax over the target maximum, times the global encode scale,
 *   then rounded to E4M3).  The elements are multiplied by the local encode
 *   scale r = 1/(alpha*Delta) and rounded (Eq. 3 / [NVFP4] sec. 6). */
typedef struct {
  uint8_t scale_code;
  float dpre, s, r, err;
} block_result;

static block_result quantize_block(float* const* elems, int n, float amax_b,
                                   float alpha, float k_m, uint32_t flags,
                                   uint64_t seed, const uint64_t* idx,
                                   uint8_t* codes_out, float* t_out,
                                   float* u_out, float* p_out) {
  block_result br;
  br.dpre = amax_b * k_m;                        /* Eq. 2 (encode form)      */
  br.scale_code = orc_e4m3_encode(br.dpre);      /* quantize scale to E4M3   */
  const float delta = orc_e4m3_decode(br.scale_code);
  br.s = alpha * delta;                          /* decode scale alpha*Delta */
  br.r = (br.s == 0.0f) ? 0.0f : 1.0f / br.s;    /* local encode scale       */
  for (int i = 0; i < n; i++) {
    const float y = *elems[i];
    const float t = y * br.r;
    uint8_t c;
    if (flags & ORC_SR) c = e2m1_sr(t, seed, idx[i], u_out ? &u_out[i] : NULL, p_out ? &p_out[i] : NULL);
    else c = orc_e2m1_encode(t);
    codes_out[i] = c;
    if (t_out) t_out[i] = t;
  }
  /* Block error: squared error of the dequantized values q*s against the
   * inputs.  Order: per row of 16, two fma chains over elements 0..7 and
   * 8..15 (each starting at +0), added; for a 2D tile the 16 row sums are
   * added pairwise ((r0+r1)+(r2+r3))+... . */
  float rowsum[16];
  const int nrows = n / 16;
  for (int rr = 0; rr < nrows; rr++) {
    float acc_lo = 0.0f, acc_hi = 0.0f;
    for (int i = 0; i < 8; i++) {
      const int e = rr * 16 + i;
      const float d = fmaf(orc_e2m1_decode(codes_out[e]), br.s, -*elems[e]);
      acc_lo = fmaf(d, d, acc_lo);
    }
    for (int i = 8; i < 16; i++) {
      const int e = rr * 16 + i;
      const float d = fmaf(orc_e2m1_decode(codes_out[e]), br.s, -*elems[e]);
      acc_hi = fmaf(d, d, acc_hi);
    }
    rowsum[rr] = acc_lo + acc_hi;
  }
  for (int width = nrows; width > 1; width /= 2)
    for (int k = 0; k < width / 2; k++) rowsum[k] = rowsum[2 * k] + rowsum[2 * k + 1];
  br.err = rowsum[0];
  return br;
}

/* NVFP4 quantization of x (bf16) or, when x is NULL, of xf (fp32). */
/* Stochastic rounding of a block scale d >= 0 (in E4M3 units) onto the E4M3
 * grid: between neighbouring E4M3 values lo <= d < hi it rounds up with
 * probability p = (d - lo)/(hi - lo) (exact: the spacing is a power of two),
 * using u = (Philox word 0 >> 8) * 2^-24 for key = seed and counter =
 * (block index lo, block index hi, 1, 0), up iff u < p; d >= 448 gives 448.
 * Returns the E4M3 code. */
static uint8_t e4m3_sr(float d, uint64_t seed, uint64_t blk, float* u_out) {
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  const uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), 1u, 0u};
  uint32_t w[4];
  orc_philox4x32_10(ctr, key, w);
  const float u = (float)(w[0] >> 8) * 0x1p-24f;
  if (u_out) *u_out = u;
  if (!(d > 0.0f)) return 0;
  if (d >= 448.0f) return 0x7E;
  int e2;
  frexp((double)d, &e2);
  int E = e2 - 1;
  if (E < -6) E = -6;                          /* subnormals share 2^-6's step */
  const double quantum = ldexp(1.0, E - 3);
  double n = floor((double)d / quantum);       /* lo = n * quantum            */
  const double p = ((double)d - n * quantum) / quantum;
  if ((double)u < p) n += 1.0;
  long code = ((long)(E + 7) << 3) + (long)n - 8;
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)code;
}

/* One MS-EDEN block (reading R26 of the design notes, after [QII] sec. 1:
 * rotation, round-to-nearest FP4 values, randomness only in the 8-bit
 * scale; the unbiasing factor is EDEN's, Vargaftik et al. 2022):
 *   Delta_pre = amax_b * k6 (Eq. 2, unrounded), s = fl(alpha * Delta_pre),
 *   t_k = y_k * fl(1/s), q_k = nearest E2M1 to t_k (saturating),
 *   N = sum t_k^2, D = sum t_k * q_k (each two fma chains over elements
 *   0..7 and 8..15, added), S = N / D (1 when D = 0),
 *   Delta' = fl(S * Delta_pre), scale = E4M3 code of SR(Delta').
 * y holds the 16 rotated values; codes_out gets the 16 codes. */
static uint8_t quantize_block_msed(const float* y, float amax_b, float alpha, float k6,
                                   uint64_t seed, uint64_t blk, uint8_t* codes_out,
                                   float* dprime_out) {
  const float dpre = amax_b * k6;
  const float s = alpha * dpre;
  const float r = (s == 0.0f) ? 0.0f : 1.0f / s;
  float t[16];
  for (int k = 0; k < 16; k++) {
    t[k] = y[k] * r;
    codes_out[k] = orc_e2m1_encode(t[k]);
  }
  float n_lo = 0.0f, n_hi = 0.0f, d_lo = 0.0f, d_hi = 0.0f;
  for (int k = 0; k < 8; k++) {
    n_lo = fmaf(t[k], t[k], n_lo);
    d_lo = fmaf(t[k], orc_e2m1_decode(codes_out[k]), d_lo);
  }
  for (int k = 8; k < 16; k++) {
    n_hi = fmaf(t[k], t[k], n_hi);
    d_hi = fmaf(t[k], orc_e2m1_decode(codes_out[k]), d_hi);
  }
  const float N = n_lo + n_hi, D = d_lo + d_hi;
  const float S = (D > 0.0f) ? N / D : 1.0f;
  const float dprime = S * dpre;
  if (dprime_out) *dprime_out = dprime;
  return e4m3_sr(dprime, seed, blk, NULL);
}

/* Tensor-level constants from an amax: Eq. 1 and the encode factors. */
typedef struct {
  float alpha, k6, k4;
} scale_consts;

static scale_consts consts_from_amax(float amax, int four_six) {
  /* Eq. 1: alpha = amax / (M_FP4 * M_FP8).  Reading: the scale maximum is
   * C = 448 for the 6-only path and C = 256 when 4/6 is on, so that the
   * M = 4 block scale (amax_b * 6*256/(4*amax) <= 384) stays in E4M3 range. */
  const float C = four_six ? 256.0f : 448.0f;
  scale_consts sc;
  sc.alpha = amax / (6.0f * C);
  /* Encode factors k_M = (6*C/M) / amax, i.e. 1/(alpha*M) taken directly
   * from amax ([NVFP4] sec. 6: global encode scale 6*448/amax). */
  sc.k6 = (amax == 0.0f) ? 0.0f : C / amax;
  sc.k4 = (amax == 0.0f) ? 0.0f : (1.5f * C) / amax;
  return sc;
}

/* rowscale != 0: every row takes its own constants from its own amax
 * (alpha_out then holds one value per row); 1D only. */
static int nvfp4_quantize_any(const uint16_t* x, const float* xf, int64_t rows, int64_t cols,
                              uint32_t flags, uint64_t seed, const float* amax_in,
                              float* alpha_out, uint8_t* codes, uint8_t* scales,
                              uint8_t* choice, uint8_t* codes_t, uint8_t* scales_t,
                              orc_debug* dbg, int rowscale, int64_t row0) {
  if (!nvfp4_flags_ok(rows, cols, flags)) return -1;
  if (!codes || !scales || !alpha_out) return -2;
  const int two_d = (flags & ORC_BLOCK2D) != 0;
  const int four_six = (flags & ORC_FOUR_OVER_SIX) != 0;
  const int msed = (flags & ORC_MSEDEN) != 0;
  if (two_d && (flags & ORC_COLWISE) && (!codes_t || !scales_t)) return -2;

  float* y = load_rotated(x, xf, rows, cols, flags, seed);
  if (!y) return -3;

  if (rowscale && (two_d || amax_in)) { free(y); return -1; }
  float amax = 0.0f;
  if (amax_in) {
    amax = *amax_in;
  } else if (!rowscale) {
    for (int64_t i = 0; i < rows * cols; i++) {
      const float a = fabsf(y[i]);
      if (a > amax) amax = a;
    }
  }
  /* MS-EDEN takes C = 256 like 4/6: its corrected scale may exceed the
   * block's unrounded one (by at most ~1.22), and 448/256 leaves room */
  scale_consts sc = consts_from_amax(amax, four_six || msed);
  if (!rowscale) *alpha_out = sc.alpha;

  const int64_t bcols = cols / 16;                        /* blocks per row */
  const int64_t brows = two_d ? rows / 16 : rows;         /* block rows     */
  const int bn = two_d ? 256 : 16;                        /* values/block   */
  memset(codes, 0, (size_t)(rows * cols / 2));
  if (two_d && (flags & ORC_COLWISE)) memset(codes_t, 0, (size_t)(rows * cols / 2));

  float* elems[256];
  uint64_t idx[256];
  uint8_t c6[256], c4[256];
  float t6[256], t4[256], u6[256], p6[256];

  for (int64_t br = 0; br < brows; br++) {
    if (rowscale) {                      /* this row's own amax and constants */
      float amax_r = 0.0f;
      for (int64_t c = 0; c < cols; c++) {
        const float a = fabsf(y[br * cols + c]);
        if (a > amax_r) amax_r = a;
      }
      sc = consts_from_amax(amax_r, four_six || msed);
      alpha_out[br] = sc.alpha;
    }
    for (int64_t bc = 0; bc < bcols; bc++) {
      /* gather the block, row by row */
      float amax_b = 0.0f;
      for (int i = 0; i < bn; i++) {
        const int64_t r = two_d ? br * 16 + i / 16 : br;
        const int64_t c = bc * 16 + (i % 16);
        elems[i] = &y[r * cols + c];
        idx[i] = (uint64_t)((row0 + r) * cols + c);   /* index in the whole tensor */
        const float a = fabsf(*elems[i]);
        if (a > amax_b) amax_b = a;
      }
      if (msed) {                      /* 1D only (flags checked above) */
        float yb[16];
        for (int i = 0; i < 16; i++) yb[i] = *elems[i];
        const int64_t bidx = br * bcols + bc;
        scales[bidx] = quantize_block_msed(yb, amax_b, sc.alpha, sc.k6, seed,
                                           (uint64_t)((row0 + br) * bcols + bc),
                                           c6, dbg && dbg->dpre6 ? &dbg->dpre6[bidx] : NULL);
        if (choice) choice[bidx] = 0;
        for (int i = 0; i < 16; i++) put_nibble(&codes[br * (cols / 2)], bc * 16 + i, c6[i]);
        continue;
      }
      block_result res6 = quantize_block(elems, bn, amax_b, sc.alpha, sc.k6, flags, seed, idx,
                                         c6, t6, u6, p6);
      block_result chosen = res6;
      const uint8_t* cc = c6;
      const float* tt = t6;
      int pick4 = 0;
      block_result res4 = res6;
      if (four_six) {
        res4 = quantize_block(elems, bn, amax_b, sc.alpha, sc.k4, flags, seed, idx, c4, t4,
                              NULL, NULL);
        /* [4/6] sec. 1: keep the candidate with the smaller error; ties keep
         * M = 6. */
        if (res4.err < res6.err) { chosen = res4; cc = c4; tt = t4; pick4 = 1; }
      }
      const int64_t bidx = br * bcols + bc;
      scales[bidx] = chosen.scale_code;
      if (choice) choice[bidx] = (uint8_t)pick4;
      if (two_d && (flags & ORC_COLWISE)) scales_t[bc * brows + br] = chosen.scale_code;
      for (int i = 0; i < bn; i++) {
        const int64_t r = two_d ? br * 16 + i / 16 : br;
        const int64_t c = bc * 16 + (i % 16);
        put_nibble(&codes[r * (cols / 2)], c, cc[i]);
        if (two_d && (flags & ORC_COLWISE)) put_nibble(&codes_t[c * (rows / 2)], r, cc[i]);
        if (dbg && dbg->t) dbg->t[r * cols + c] = tt[i];
        if (dbg && dbg->u && (flags & ORC_SR)) dbg->u[r * cols + c] = u6[i];
        if (dbg && dbg->p && (flags & ORC_SR)) dbg->p[r * cols + c] = p6[i];
      }
      if (dbg) {
        if (dbg->dpre6) dbg->dpre6[bidx] = res6.dpre;
        if (dbg->dpre4 && four_six) dbg->dpre4[bidx] = res4.dpre;
        if (dbg->err6 && four_six) dbg->err6[bidx] = res6.err;
        if (dbg->err4 && four_six) dbg->err4[bidx] = res4.err;
      }
    }
  }
  free(y);
  return 0;
}

int orc_nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols,
                       uint32_t flags, uint64_t seed, const float* amax_in,
                       float* alpha_out, uint8_t* codes, uint8_t* scales,
                       uint8_t* choice, uint8_t* codes_t, uint8_t* scales_t,
                       orc_debug* dbg) {
  if (!x && rows * cols > 0) return -2;
  return nvfp4_quantize_any(x, NULL, rows, cols, flags, seed, amax_in, alpha_out, codes,
                            scales, choice, codes_t, scales_t, dbg, 0, 0);
}

/* orc_nvfp4_quantize (1D flags) of rows row0 .. row0 + rows - 1 of a larger
 * tensor with `cols` columns, given here alone: the random counters (SR:
 * element index; MS-EDEN: block index) are those of the whole tensor, and
 * amax_in must be the whole tensor's.  With row0 = 0 it is
 * orc_nvfp4_quantize. */
int orc_nvfp4_quantize_at(const uint16_t* x, int64_t rows, int64_t cols, int64_t row0,
                          uint32_t flags, uint64_t seed, const float* amax_in,
                          float* alpha_out, uint8_t* codes, uint8_t* scales,
                          uint8_t* choice) {
  if (!x && rows * cols > 0) return -2;
  if (row0 < 0 || !amax_in || (flags & (ORC_BLOCK2D | ORC_COLWISE))) return -1;
  return nvfp4_quantize_any(x, NULL, rows, cols, flags, seed, amax_in, alpha_out, codes,
                            scales, choice, NULL, NULL, NULL, 0, row0);
}

int orc_nvfp4_quantize_f32(const float* x, int64_t rows, int64_t cols, uint32_t flags,
                           uint64_t seed, const float* amax_in, float* alpha_out,
                           uint8_t* codes, uint8_t* scales, uint8_t* choice) {
  if (!x && rows * cols > 0) return -2;
  if (flags & (ORC_BLOCK2D | ORC_COLWISE)) return -1;
  return nvfp4_quantize_any(NULL, x, rows, cols, flags, seed, amax_in, alpha_out, codes,
                            scales, choice, NULL, NULL, NULL, 0, 0);
}

/* NVFP4 with one FP32 scale per row instead of per tensor: the finer
 * global scale [NVFP4] sec. 9 proposes so that the quantizer needs no
 * separate pass over memory for the amax.  Row r is quantized exactly as
 * the per-tensor quantizer would, with alpha_r = amax_r / (6 C) from the
 * row's own largest magnitude (after RHT16 when asked); the SR counter stays
 * the element index in the whole tensor. */
int orc_nvfp4_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags,
                            uint64_t seed, float* alpha_rows, uint8_t* codes,
                            uint8_t* scales, uint8_t* choice) {
  if (!x && rows * cols > 0) return -2;
  if (flags & (ORC_BLOCK2D | ORC_COLWISE)) return -1;
  return nvfp4_quantize_any(x, NULL, rows, cols, flags, seed, NULL, alpha_rows, codes, scales,
                            choice, NULL, NULL, NULL, 1, 0);
}

/* orc_nvfp4_quantize_rows of rows row0 .. row0 + rows - 1 of a larger tensor
 * (each row's scale is its own, so only the SR counters need row0). */
int orc_nvfp4_quantize_rows_at(const uint16_t* x, int64_t rows, int64_t cols, int64_t row0,
                               uint32_t flags, uint64_t seed, float* alpha_rows,
                               uint8_t* codes, uint8_t* scales, uint8_t* choice) {
  if (!x && rows * cols > 0) return -2;
  if (row0 < 0 || (flags & (ORC_BLOCK2D | ORC_COLWISE))) return -1;
  return nvfp4_quantize_any(x, NULL, rows, cols, flags, seed, NULL, alpha_rows, codes, scales,
                            choice, NULL, NULL, NULL, 1, row0);
}

/* Requantization for the transposed operand of the backward pass ([QII]
 * sec. 2: part of the data is quantized again; [NVFP4] sec. 7: the weight
 * gradient contracts over the other dimension).  The input is a 1D NVFP4
 * quantization of X [rows][cols]; the output is the NVFP4 quantization
 * (flags: RTN6, FOUR_OVER_SIX, SR, RHT16) of the transpose of its
 * dequantized values: quantize((dequantize(X))^T), blocks of 16 running
 * along the original columns.  Output: codes_t [cols][rows/2], scales_t
 * [cols][rows/16], choice_t likewise (may be NULL). */
static int requantize_t_any(const uint8_t* codes, const uint8_t* scales, float alpha,
                            int64_t rows, int64_t cols, int64_t col0, uint32_t flags,
                            uint64_t seed, const float* amax_in, float* alpha_out,
                            uint8_t* codes_t, uint8_t* scales_t, uint8_t* choice_t) {
  if (rows < 0 || cols < 0 || rows % 16 || cols % 16 || col0 < 0) return -1;
  if (flags & (ORC_BLOCK2D | ORC_COLWISE)) return -1;
  const size_t n = (size_t)(rows * cols > 0 ? rows * cols : 1);
  float* xd = (float*)malloc(sizeof(float) * n);
  float* xt = (float*)malloc(sizeof(float) * n);
  if (!xd || !xt) { free(xd); free(xt); return -3; }
  int rc = orc_dequantize(0, codes, scales, alpha, rows, cols, 0, xd);
  if (rc == 0) {
    for (int64_t r = 0; r < rows; r++)
      for (int64_t c = 0; c < cols; c++) xt[c * rows + r] = xd[r * cols + c];
    rc = nvfp4_quantize_any(NULL, xt, cols, rows, flags, seed, amax_in, alpha_out, codes_t,
                            scales_t, choice_t, NULL, NULL, NULL, 0, col0);
  }
  free(xd);
  free(xt);
  return rc;
}

int orc_nvfp4_requantize_t(const uint8_t* codes, const uint8_t* scales, float alpha,
                           int64_t rows, int64_t cols, uint32_t flags, uint64_t seed,
                           float* alpha_out, uint8_t* codes_t, uint8_t* scales_t,
                           uint8_t* choice_t) {
  return requantize_t_any(codes, scales, alpha, rows, cols, 0, flags, seed, NULL, alpha_out,
                          codes_t, scales_t, choice_t);
}

/* orc_nvfp4_requantize_t of columns col0 .. col0 + cols - 1 of a larger X
 * (codes and scales of those columns, all rows): output rows col0 .. of the
 * whole transpose, whose amax (amax_in, required) and SR element indices
 * are the whole output tensor's. */
int orc_nvfp4_requantize_t_at(const uint8_t* codes, const uint8_t* scales, float alpha,
                              int64_t rows, int64_t cols, int64_t col0, uint32_t flags,
                              uint64_t seed, const float* amax_in, float* alpha_out,
                              uint8_t* codes_t, uint8_t* scales_t, uint8_t* choice_t) {
  if (!amax_in) return -1;
  return requantize_t_any(codes, scales, alpha, rows, cols, col0, flags, seed, amax_in,
                          alpha_out, codes_t, scales_t, choice_t);
}

/* ===================================================================== */
/* Error study ([4/6] sec. 2.2, Fig. 2)                                    */
/* ===================================================================== */

/* [4/6] sec. 2.1 names two sources of NVFP4 error, the E4M3 rounding of the
 * block scale and the FP4 rounding of the scaled values; sec. 2.2 (Fig. 2)
 * removes one at a time, and then rounds only the scaled values below a
 * threshold.  Each step below is the plain RTN6 quantizer of this file
 * (Eq. 1-3 with the encode factors of R5) with the named rounding left
 * out. */
int orc_nvfp4_simulate(const uint16_t* x, int64_t rows, int64_t cols, int mode,
                       float thr, float* out) {
  if (rows < 0 || cols < 0 || cols % 16) return -1;
  if (mode < ORC_SIM_NVFP4 || mode > ORC_SIM_THRESHOLD) return -1;
  if (rows * cols > 0 && (!x || !out)) return -1;
  float amax = 0.0f;
  for (int64_t i = 0; i < rows * cols; i++) {
    const float a = fabsf(bf16_to_f32(x[i]));
    if (a > amax) amax = a;
  }
  const float alpha = amax / (6.0f * 448.0f);           /* Eq. 1, M = 6 only */
  const float k6 = (amax == 0.0f) ? 0.0f : 448.0f / amax;
  for (int64_t r = 0; r < rows; r++) {
    for (int64_t c0 = 0; c0 < cols; c0 += 16) {
      float y[16], amax_b = 0.0f;
      for (int k = 0; k < 16; k++) {
        y[k] = bf16_to_f32(x[r * cols + c0 + k]);
        if (fabsf(y[k]) > amax_b) amax_b = fabsf(y[k]);
      }
      const float dpre = amax_b * k6;                    /* Eq. 2, unrounded */
      const float delta = (mode == ORC_SIM_SCALE_HP) ? dpre
                                                     : orc_e4m3_decode(orc_e4m3_encode(dpre));
      const float s = alpha * delta;
      const float rcp = (s == 0.0f) ? 0.0f : 1.0f / s;
      for (int k = 0; k < 16; k++) {
        const float t = y[k] * rcp;                      /* scaled value     */
        int round_it = 1;
        if (mode == ORC_SIM_VALUE_HP) round_it = 0;
        if (mode == ORC_SIM_THRESHOLD) round_it = fabsf(t) < thr;
        const float q = round_it ? orc_e2m1_decode(orc_e2m1_encode(t)) : t;
        out[r * cols + c0 + k] = q * s;
      }
    }
  }
  return 0;
}

/* ===================================================================== */
/* MXFP4 ([NVFP4] sec. 1 and 5; [MXFP4] sec. 2)                           */
/* ===================================================================== */

/* Row-wise MXFP4 of a (rows x cols) fp32 matrix already in memory.
 * Per 32-value group: optional deterministic Hadamard; shared exponent
 * e = floor(log2(amax)) - 2 (the largest E2M1 exponent), so the group
 * maximum scales into [4, 8); UE8M0 code e + 127, clamped to [0, 254]; an
 * all-zero group takes code 0.  Values are scaled by 2^-e and rounded to
 * E2M1 (nearest-even, saturating: scaled values in (6, 8) become 6). */
static void mx_rowwise(const float* y, int64_t rows, int64_t cols, uint32_t flags,
                       uint8_t* codes, uint8_t* scales, float* t_out) {
  memset(codes, 0, (size_t)(rows * cols / 2));
  float g[32];
  for (int64_t r = 0; r < rows; r++) {
    for (int64_t c0 = 0; c0 < cols; c0 += 32) {
      if (flags & ORC_HAD32) orc_rotate_had32(&y[r * cols + c0], g);
      else memcpy(g, &y[r * cols + c0], sizeof g);
      float amax_b = 0.0f;
      for (int k = 0; k < 32; k++) {
        const float a = fabsf(g[k]);
        if (a > amax_b) amax_b = a;
      }
      int e;
      if (amax_b == 0.0f) {
        e = -127;
      } else {
        int e2;
        frexp((double)amax_b, &e2);            /* floor(log2 amax) = e2 - 1 */
        e = (e2 - 1) - 2;
        if (e < -127) e = -127;
        if (e > 127) e = 127;
      }
      scales[r * (cols / 32) + c0 / 32] = (uint8_t)(e + 127);
      for (int k = 0; k < 32; k++) {
        const float t = ldexpf(g[k], -e);
        put_nibble(&codes[r * (cols / 2)], c0 + k, orc_e2m1_encode(t));
        if (t_out) t_out[r * cols + c0 + k] = t;
      }
    }
  }
}

int orc_mxfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols,
                       uint32_t flags, uint8_t* codes_r, uint8_t* scales_r,
                       uint8_t* codes_c, uint8_t* scales_c,
                       float* t_r, float* t_c) {
  if (rows < 0 || cols < 0) return -1;
  if (flags & ~(ORC_HAD32 | ORC_ROWWISE | ORC_COLWISE)) return -1;
  if (!(flags & (ORC_ROWWISE | ORC_COLWISE))) return -1;
  if ((flags & ORC_ROWWISE) && (cols % 32 || !codes_r || !scales_r)) return -1;
  if ((flags & ORC_COLWISE) && (rows % 32 || !codes_c || !scales_c)) return -1;
  const size_t n = (size_t)(rows * cols > 0 ? rows * cols : 1);
  float* y = (float*)malloc(sizeof(float) * n);
  if (!y) return -3;
  for (int64_t i = 0; i < rows * cols; i++) y[i] = bf16_to_f32(x[i]);
  if (flags & ORC_ROWWISE) mx_rowwise(y, rows, cols, flags, codes_r, scales_r, t_r);
  if (flags & ORC_COLWISE) {
    /* Column-wise = row-wise of the transpose: the rotation and the 32-value
     * groups run down each column (the reduction dimension of the product
     * that uses the transposed operand, [NVFP4] sec. 2). */
    float* yt = (float*)malloc(sizeof(float) * n);
    if (!yt) { free(y); return -3; }
    for (int64_t r = 0; r < rows; r++)
      for (int64_t c = 0; c < cols; c++) yt[c * rows + r] = y[r * cols + c];
    mx_rowwise(yt, cols, rows, flags, codes_c, scales_c, t_c);
    free(yt);
  }
  free(y);
  return 0;
}

/* ===================================================================== */
/* Dequantization ([NVFP4] sec. 4 and 6: decode scales applied to codes)   */
/* ===================================================================== */

int orc_dequantize(int format, const uint8_t* codes, const uint8_t* scales,
                   float alpha, int64_t rows, int64_t cols, uint32_t flags,
                   float* out) {
  if (rows < 0 || cols < 0) return -1;
  if (format == 0) {
    const int two_d = (flags & ORC_BLOCK2D) != 0;
    if (cols % 16 || (two_d && rows % 16)) return -1;
    for (int64_t r = 0; r < rows; r++)
      for (int64_t c = 0; c < cols; c++) {
        const int64_t b = two_d ? (r / 16) * (cols / 16) + c / 16 : r * (cols / 16) + c / 16;
        const float s = alpha * orc_e4m3_decode(scales[b]);
        out[r * cols + c] = orc_e2m1_decode(get_nibble(&codes[r * (cols / 2)], c)) * s;
      }
    return 0;
  }
  if (format == 1) {
    if (cols % 32) return -1;
    for (int64_t r = 0; r < rows; r++)
      for (int64_t c = 0; c < cols; c++) {
        const int e = (int)scales[r * (cols / 32) + c / 32] - 127;
        out[r * cols + c] = ldexpf(orc_e2m1_decode(get_nibble(&codes[r * (cols / 2)], c)), e);
      }
    return 0;
  }
  return -1;
}
