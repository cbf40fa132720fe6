/* Checks the two arithmetic identities the GPU quantiser uses in place of IEEE divisions (host C, IEEE fp32
 * with round-to-nearest-even and subnormals, no contraction):
 *   (1) for L = 3, 15, 255 and c = fp32(1/L): q0 = x * c, r = fma(-q0, L, x), q1 = fma(r, c, q0) equals x / L
 *       for every non-negative finite fp32 x visited (every STRIDE-th bit pattern, STRIDE = argv[1]);
 *   (2) for every positive finite fp16 value s and every start r0 within two ulps of 1 / s:
 *       fma(fma(-s, r0, 1), r0, r0) equals 1 / s (a hardware reciprocal within one ulp is such a start).
 * Prints the mismatch counts and exits non-zero if any. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bits_f(uint32_t u) {
  float x;
  memcpy(&x, &u, 4);
  return x;
}

static float half_value(uint32_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  return e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), e - 25);
}

int main(int argc, char** argv) {
  const long stride = argc > 1 ? atol(argv[1]) : 1;
  const float Ls[3] = {3.0f, 15.0f, 255.0f};
  long bad = 0;
  for (int k = 0; k < 3; ++k) {
    const float L = Ls[k];
    const float c = 1.0f / L;
    long n = 0, miss = 0;
#pragma omp parallel for reduction(+ : n, miss) schedule(static)
    for (long u = 0; u < 0x7F800000L; u += stride) {
      const float x = bits_f((uint32_t)u);
      volatile float q0 = x * c;
      const float r = fmaf(-q0, L, x);
      const float q1 = fmaf(r, c, q0);
      miss += q1 != x / L;
      n++;
    }
    printf("division by %g (c = %a): %ld values, %ld mismatches\n", L, c, n, miss);
    bad += miss;
  }
  long n = 0, miss = 0;
  for (uint32_t h = 1; h < 0x7C00; ++h) {
    const float s = half_value(h), ref = 1.0f / s;
    float r0[5];
    r0[2] = ref;
    r0[1] = nextafterf(ref, 0.0f);
    r0[0] = nextafterf(r0[1], 0.0f);
    r0[3] = nextafterf(ref, INFINITY);
    r0[4] = nextafterf(r0[3], INFINITY);
    for (int i = 0; i < 5; ++i) {
      const float e = fmaf(-s, r0[i], 1.0f);
      miss += fmaf(e, r0[i], r0[i]) != ref;
      n++;
    }
  }
  printf("reciprocal of fp16 scales: %ld (value, start) pairs, %ld mismatches\n", n, miss);
  bad += miss;
  return bad != 0;
}
