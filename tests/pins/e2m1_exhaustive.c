/*
 * Exhaustive pin of the oracle's E2M1 encoder (test code, CPU only).
 *
 * For every fp32 bit pattern with |t| <= 16 (plus +-inf) the oracle's code
 * must equal
 *   (a) a brute-force nearest search over the 8 magnitudes of the FP4 value
 *       set +-{0,0.5,1,1.5,2,3,4,6} ("Four Over Six" page, sec. 1), ties to
 *       the even magnitude code, values past 6 clamped to 6;
 *   (b) Eq. 3 of the same page written literally: 1/2*round(2v) below 2,
 *       round(v) below 4, 2*round(v/2) up to 6, with round-half-even
 *       integers, and 6 beyond.
 * Prints "OK <count>" or the first mismatch.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint8_t orc_e2m1_encode(float t);

static const double kMag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

static int brute_force(float t) {
  double a = fabs((double)t);
  int best = 0;
  double bestd = INFINITY;
  for (int m = 0; m < 8; m++) {
    double d = fabs(a - kMag[m]);
    if (d < bestd || (d == bestd && (m % 2) == 0)) { best = m; bestd = d; }
  }
  if (a > 6.0) best = 7;
  return (signbit(t) ? 8 : 0) | best;
}

static int mag_index(double v) {
  for (int m = 0; m < 8; m++) if (v == kMag[m]) return m;
  return -1;
}

static int eq3_literal(float t) {
  double v = fabs((double)t), q;
  if (v < 2.0)       q = 0.5 * nearbyint(2.0 * v);
  else if (v < 4.0)  q = nearbyint(v);
  else if (v <= 6.0) q = 2.0 * nearbyint(v / 2.0);
  else               q = 6.0;
  return (signbit(t) ? 8 : 0) | mag_index(q);
}

int main(void) {
  const uint32_t lim = 0x41800000u;   /* 16.0f */
  uint64_t count = 0;
  for (int s = 0; s < 2; s++) {
    for (uint32_t b = 0; b <= lim + 1; b++) {
      uint32_t bits = (b == lim + 1) ? 0x7F800000u : b;   /* last one: inf */
      bits |= (uint32_t)s << 31;
      float t;
      memcpy(&t, &bits, 4);
      int o = orc_e2m1_encode(t);
      int bf = brute_force(t);
      int e3 = eq3_literal(t);
      if (o != bf || o != e3) {
        printf("MISMATCH t=%a oracle=%d brute=%d eq3=%d\n", (double)t, o, bf, e3);
        return 1;
      }
      count++;
    }
  }
  printf("OK %llu\n", (unsigned long long)count);
  return 0;
}
