/*
 * Exhaustive host-side check of the quantizer's fp32 quotient.
 *
 * The group quantizer needs t = RN32(x / s) for bf16 x with |x| <= amax and
 * s = RN32(max(amax, 1e-10) / 448), amax itself a bf16 value (the group
 * maximum of bf16 inputs).  The GPU kernels compute it without a per-element
 * division: r = RN32(1/s) once per group, y = RN32(x*r), e = fma(y, s, -x)
 * (the exact negated residual), t = fma(-e, r, y).  This program enumerates
 * every (amax, x) pair of that finite domain, both signs of x (and -0), and
 * checks
 * that the FMA sequence returns the bits of the IEEE quotient wherever it can
 * matter.  The FMA residual is exact only while x and y*s stay out of the
 * fp32 subnormal range, so the two may differ when x is tiny; every such pair must
 * have both quotients below 2^-10, where E4M3 rounding gives zero (of the same
 * sign) either way.  The program reports the pairs that differ (and how many
 * had a normal x) and fails if any differing pair reaches 2^-10.
 *
 * Build: gcc -O2 -mfma -ffp-contract=off -fopenmp; exit status 0 = pass.
 * (x86-64 only: the negations are pinned with an empty asm barrier.)
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16_to_f32(uint32_t b) {
  uint32_t u = b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Hide a value from the optimizer: gcc otherwise rewrites fma(-fma(a, b, -c), ...)
 * as fma(fma(-a, b, c), ...), which differs in the sign of a zero result. */
static inline float opaque(float v) {
  __asm__("" : "+x"(v));
  return v;
}

static uint32_t bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

int main(void) {
  const volatile float floor_ = 1e-10f, fmax = 448.0f;
  unsigned long long pairs = 0, differ = 0, differ_normal_x = 0, fatal = 0;
  const float tiny = 0x1p-10f;
  /* every non-negative finite bf16 amax: patterns 0x0000 .. 0x7F7F */
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, differ, differ_normal_x, fatal)
  for (uint32_t ab = 0; ab <= 0x7F7F; ++ab) {
    const float amax = bf16_to_f32(ab);
    const float a = amax > floor_ ? amax : floor_;
    const float s = a / fmax;
    const float r = 1.0f / s;
    for (uint32_t xb = 0; xb <= ab; ++xb) { /* all bf16 |x| <= amax, both signs */
      for (uint32_t sign = 0; sign < 2; ++sign) {
        const float x = bf16_to_f32(xb | (sign << 15));
        const float ref = x / s;
        const float y = x * r;
        const float e = opaque(fmaf(y, s, opaque(-x)));
        const float t = fmaf(opaque(-e), r, y);
        ++pairs;
        if (bits(t) != bits(ref)) {
          ++differ;
          if (fabsf(x) >= 0x1p-126f) ++differ_normal_x;
          /* must encode alike: both below 2^-10 (E4M3 zero) with x's sign */
          if (fabsf(ref) >= tiny || fabsf(t) >= tiny || signbit(t) != signbit(x)) {
            ++fatal;
            printf("FATAL amax=%a x=%a ref=%a got=%a\n", amax, x, ref, t);
          }
        }
      }
    }
  }
  printf("pairs=%llu differ=%llu differ_with_normal_x=%llu fatal=%llu\n", pairs, differ,
         differ_normal_x, fatal);
  return fatal != 0;
}
