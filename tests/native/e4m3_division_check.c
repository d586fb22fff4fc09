/* Host check of the division the e4m3 encoders use in place of an IEEE
 * division (E4m3Divider in the quantiser source): for every positive finite
 * bf16 maximum a, the scale s = RN(a / 448) and every bf16 x with |x| <= a,
 * the e4m3 code of
 *     x1 = x 2^-e, s1 = s 2^-e in [1/2, 1), y1 = RN(1 / s1),
 *     q0 = RN(x1 y1), r = fma(-q0, s1, x1), q = copysign(fma(r, y1, q0), x)
 * equals the e4m3 code of the correctly rounded quotient RN(x / s), and q
 * itself equals RN(x / s) wherever |x / s| >= 2^-100 (below, the residual may
 * underflow; such quotients have a zero code).  Codes are
 * round-to-nearest-even after clamping to +-448, the sign bit kept for
 * zeros.  Usage: e4m3_division_check PART NPARTS (maxima a with
 * (bits(a) - 1) % NPARTS == PART).  Prints the counts; exit status 1 on any
 * difference. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float mag[127]; /* e4m3 magnitudes of the codes 0 .. 126 */

static float from_bf16(uint32_t b) {
  const uint32_t u = b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static int e4m3_code(float q) {
  const int neg = signbit(q) != 0;
  const float a = fminf(fabsf(q), 448.f);
  int lo = 0, hi = 126; /* largest code whose magnitude is <= a */
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (mag[mid] <= a) lo = mid; else hi = mid - 1;
  }
  int c = lo;
  if (lo < 126 && a > mag[lo]) {
    const double half = ((double)mag[lo] + (double)mag[lo + 1]) / 2;
    if (a > half || (a == half && (lo & 1))) c = lo + 1;
  }
  return c | (neg ? 0x80 : 0);
}

int main(int argc, char** argv) {
  if (argc != 3) return 2;
  const int part = atoi(argv[1]), nparts = atoi(argv[2]);
  for (int c = 0; c < 127; ++c) {
    const int e = c >> 3, m = c & 7;
    mag[c] = e == 0 ? ldexpf((float)m, -9) : ldexpf(1.f + m / 8.f, e - 7);
  }
  long long pairs = 0, bad = 0;
  for (uint32_t ab = 1 + part; ab < 0x7f80; ab += nparts) {
    const float a = from_bf16(ab), s = a / 448.f;
    int e;
    const float s1 = frexpf(s, &e), y1 = 1.f / s1;
    for (uint32_t xb = 0; xb < 0x10000; ++xb) {
      const float x = from_bf16(xb);
      if (!(fabsf(x) <= a)) continue;
      const float x1 = ldexpf(x, -e), q0 = x1 * y1, r = fmaf(-q0, s1, x1);
      const float q = copysignf(fmaf(r, y1, q0), x);
      const float ref = x / s;
      ++pairs;
      if (e4m3_code(q) != e4m3_code(ref) || (fabsf(ref) >= 0x1p-100f && memcmp(&q, &ref, 4) != 0)) {
        if (bad < 5) printf("differs: a=%a x=%a\n", a, x);
        ++bad;
      }
    }
  }
  printf("%lld %lld\n", pairs, bad);
  return bad != 0;
}
