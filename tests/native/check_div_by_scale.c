/*
 * Exhaustive check of the q-quantisation division used by the GPU kernels.
 *
 * For a tile with largest magnitude amax (a bf16 value) the kernels use the
 * scale s = RN32(amax / 448) and, when amax >= 2^-60, compute each quotient
 * x / s of a bf16 element |x| <= amax as
 *     r = RN32(1 / s);  y = RN(x * r);  e = fma(-y, s, x);
 *     z = copysign(fma(e, r, y), x)
 * instead of an IEEE division (tiles below 2^-60 use the IEEE division).  What
 * must agree is the OCP e4m3 code that round-to-nearest-even gives for z and
 * for RN32(x / s): this holds when z and the IEEE quotient are the same fp32
 * value, or when both have magnitude <= 2^-10 (half the smallest e4m3
 * subnormal; such values round to a signed zero) and the same sign.
 * Every positive finite bf16 amax >= 2^-60 and every bf16 x (both signs, both
 * zeros) with |x| <= amax is checked.  Exit status 1 on any violation.
 * Build: gcc -O2 -fopenmp -ffp-contract=off -mfma ... -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16f(uint32_t bits) { uint32_t w = bits << 16; float f; memcpy(&f, &w, 4); return f; }

int main(void) {
  long long bad = 0, checked = 0, fp32_diff = 0;
  const float tiny = ldexpf(1.0f, -10);
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : bad, checked, fp32_diff)
  for (uint32_t ab = 1; ab < 0x7F80; ++ab) {          /* positive finite bf16 amax */
    const float amax = bf16f(ab);
    if (amax < ldexpf(1.0f, -60)) continue;            /* those tiles divide exactly */
    const float s = amax / 448.0f;
    const float r = 1.0f / s;
    for (uint32_t xm = 0; xm <= ab; ++xm) {
      for (int sign = 0; sign < 2; ++sign) {
        const float x = bf16f(xm | (sign ? 0x8000u : 0u));
        volatile float y = x * r;
        const float e = fmaf(-y, s, x);
        const float z = copysignf(fmaf(e, r, y), x);
        const float ref = x / s;
        uint32_t zi, ri;
        memcpy(&zi, &z, 4);
        memcpy(&ri, &ref, 4);
        checked += 1;
        if (zi == ri) continue;
        fp32_diff += 1;
        if (fabsf(z) <= tiny && fabsf(ref) <= tiny && signbit(z) == signbit(ref)) continue;
        bad += 1;
      }
    }
  }
  printf("checked %lld (amax, x) pairs: %lld differ in fp32 below 2^-10, %lld give different e4m3 codes\n",
         checked, fp32_diff, bad);
  return bad != 0;
}
