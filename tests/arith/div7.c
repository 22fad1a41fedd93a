// Exhaustive check of the quotient kernel 1 uses for the INT4 group scale: for every
// non-negative finite fp32 a, q0 = a * fp32(1/7) corrected by one fma with the exact
// residual, fma(fma(-q0, 7, a), fp32(1/7), q0), equals the correctly rounded a / 7.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

int main(void) {
  const float c = 1.0f / 7.0f;
  uint64_t bad = 0;
  for (uint32_t u = 0; u < 0x7F800000u; ++u) {
    float a;
    memcpy(&a, &u, 4);
    const float q0 = a * c;
    const float q1 = fmaf(fmaf(-q0, 7.0f, a), c, q0);
    if (q1 != a / 7.0f) {
      if (bad < 5) printf("mismatch at %a\n", a);
      ++bad;
    }
  }
  printf("%llu mismatches\n", (unsigned long long)bad);
  return bad != 0;
}
