/* The identity the per-group FP8 epilogue of the kernels relies on to form absmax / 448 without a
 * division sequence, checked in binary32 on the host (C's float division and fmaf are correctly
 * rounded):
 *   m * RN(1/448), corrected once by its FMA residual, equals RN(m / 448) for every m >= 2^-120.
 * Checked exhaustively where an intermediate can be subnormal (m in [2^-120, 2^-100)), over two
 * whole binades of ordinary values (m in [1, 4), which holds both binades of the quotient) and at
 * the top of the range (m in [2^126, 2^128)); between those, every intermediate is a normal
 * number and the three operations scale exactly by powers of two, so the [1, 4) result carries
 * over (below 2^-120 the kernels divide).
 * Prints "ok" and exits 0, or the first mismatches and exits 1. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static long check(uint32_t lo, uint32_t hi) {
  const float c = 1.0f / 448.0f;
  long bad = 0;
  for (uint32_t u = lo; u < hi; ++u) {
    const float m = from_bits(u);
    const volatile float mv = m;
    const float want = mv / 448.0f;
    const float q0 = m * c;
    const float got = fmaf(fmaf(-q0, 448.0f, m), c, q0);
    if (got != want && bad++ < 5) printf("m=%a got %a want %a\n", m, got, want);
  }
  return bad;
}

int main(void) {
  long bad = 0;
  bad += check(0x03800000u, 0x0d800000u); /* [2^-120, 2^-100) */
  bad += check(0x3f800000u, 0x40800000u); /* [1, 4) */
  bad += check(0x7e800000u, 0x7f800000u); /* [2^126, 2^128) */
  if (bad) {
    printf("%ld mismatches\n", bad);
    return 1;
  }
  printf("ok\n");
  return 0;
}
