/* The two identities the FP4 epilogue of the kernels relies on to form its quotients without a
 * division sequence, checked in binary32 on the host (C's float division and fmaf are correctly
 * rounded):
 *   div6   p * RN(1/6), corrected once by its FMA residual, equals RN(p / 6) for every binary32
 *          significand: all p in [1, 4), which holds both binades of the quotient.
 *   scale  RN(gs / d) == RN(gs / M) * 2^-e for every positive finite e4m3 value d = M * 2^e
 *          (M = 1 + j/8) and a sample of gs over the normal range where the quotient is normal,
 *          and for quotients that overflow.
 * Prints "ok" and exits 0, or prints the first mismatches and exits 1. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint32_t lcg(uint64_t* s) {
  *s = *s * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(*s >> 33);
}

int main(void) {
  long bad = 0;
  const float sixth = 1.0f / 6.0f;
  for (uint32_t u = 0x3f800000u; u < 0x40800000u; ++u) {
    const float p = from_bits(u);
    const volatile float pv = p;
    const float q0 = p * sixth;
    const float got = fmaf(fmaf(-q0, 6.0f, p), sixth, q0);
    const float want = pv / 6.0f;
    if (got != want && bad++ < 5) printf("div6 p=%a got %a want %a\n", p, got, want);
  }
  /* every positive finite e4m3 value: codes 1..126 (exponent field 0 = subnormal, bias 7) */
  uint64_t seed = 12345;
  for (int code = 1; code <= 126; ++code) {
    const int ef = code >> 3, mf = code & 7;
    const double dv = ef == 0 ? ldexp(mf, -9) : ldexp(1.0 + mf / 8.0, ef - 7);
    const float d = (float)dv;
    int e;
    const float M = 2.0f * frexpf(d, &e);  /* d = M * 2^(e-1), M in [1, 2) */
    for (int i = 0; i < 200000; ++i) {
      /* gs over binades 2^-100 .. 2^127 */
      const uint32_t ex = 27u + lcg(&seed) % 227u, man = lcg(&seed) & 0x7FFFFFu;
      const float gs = from_bits((ex << 23) | man);
      const volatile float gv = gs;
      const float want = gv / d;
      const float got = ldexpf(gv / M, -(e - 1));
      if (got != want && bad++ < 5) printf("scale gs=%a d=%a got %a want %a\n", gs, d, got, want);
    }
  }
  if (bad) {
    printf("%ld mismatches\n", bad);
    return 1;
  }
  printf("ok\n");
  return 0;
}
