/*
 * E4M3FN codec and correctly rounded 2^x for the oracle.  TEST INFRASTRUCTURE
 * ONLY (see oracle.h).
 *
 * Format (attention-numerics, "See the vectors and the arithmetic"): one sign
 * bit, four exponent bits with bias 7, three mantissa bits; no infinities;
 * 0x7F/0xFF are NaN; the largest finite magnitude is 448 (0x7E).  Conversion
 * rounds to nearest with ties to even and saturates at +-448.  Subnormals are
 * m * 2^-9, so the smallest non-zero magnitude is 2^-9 and anything at or
 * below 2^-10 rounds to zero (the round-to-zero threshold the P-cast summary
 * uses in its collapse formula, Methodologie, Theoretisch Kader).
 */
#include <math.h>
#include <stdint.h>
#include <float.h>
#include "oracle.h"

uint8_t orc_e4m3_encode(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return sign | 0x7F;
  double a = fabs((double)x);
  if (a == 0.0) return sign;
  if (isinf(a)) return sign | 0x7E; /* saturation */
  int e2;
  (void)frexp(a, &e2);      /* a = f * 2^e2, f in [0.5, 1) */
  int E = e2 - 1;           /* floor(log2 a) */
  if (E < -6) E = -6;       /* subnormal range shares the quantum of 2^-6 */
  double quantum = ldexp(1.0, E - 3);
  double n = nearbyint(a / quantum); /* exact scaling; default mode is to-nearest-even */
  double r = n * quantum;
  if (r > 448.0) r = 448.0; /* saturation: a rounded magnitude above the largest finite value */
  if (r == 0.0) return sign;
  (void)frexp(r, &e2);
  E = e2 - 1;
  if (E < -6) {
    int m = (int)(r / ldexp(1.0, -9));
    return sign | (uint8_t)m;
  }
  int m = (int)(r / ldexp(1.0, E - 3)) - 8;
  return sign | (uint8_t)(((E + 7) << 3) | m);
}

float orc_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return (float)(s ? -v : v);
}

void orc_e4m3_encode_n(const float* x, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(x[i]);
}

void orc_e4m3_decode_n(const uint8_t* c, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(c[i]);
}

/* RN32(2^x).  The binary64 exp2 is within one binary64 ulp, so its rounding to
 * binary32 is the correctly rounded result unless 2^x lies within about
 * 2^-52 (relative) of a point half-way between two binary32 values; that case
 * is re-decided with the x87 extended-precision exp2l. */
float orc_exp2_rn32(float x) {
  if (isnan(x)) return x;
  double r = exp2((double)x);
  float f = (float)r;
  if (r == 0.0 || isinf(r) || f == 0.0f || isinf(f)) return f;
  float lo = (double)f <= r ? f : nextafterf(f, -INFINITY);
  float hi = nextafterf(lo, INFINITY);
  double mid = 0.5 * ((double)lo + (double)hi);
  if (fabs(r - mid) <= fabs(r) * 0x1p-44) {
    long double rl = exp2l((long double)x);
    if (rl > (long double)mid) return hi;
    if (rl < (long double)mid) return lo;
  }
  return f;
}

void orc_exp2_rn32_n(const float* x, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_exp2_rn32(x[i]);
}
