/* Check of the INT2 encoder's division: the code of a value x in a group with
 * fp16 offset z and fp16 step s is u = clip(rint(RN(d / s)), 0, 3),
 * d = RN(x - z) in fp32, and the encoder forms the quotient as
 *
 *     r  = RN(1 / s)                      (once per group; exact for every
 *                                          fp16 s, see check_scale_div.c)
 *     q0 = RN(d * r)
 *     q  = fma(-fma(q0, s, -d), r, q0)    (one correction)
 *
 * For every fp16 step s in [2^-24, 65504] this checks q == RN(d / s) bit for
 * bit:
 *   - for every fp32 d within 4,096 units in the last place of each point
 *     t * s, t = 0.5, 1.5, 2.5, 3.5 (where rint changes its decision; d
 *     anywhere near a boundary is an fp32 value of that window);
 *   - for 512 dividends spread over [0, 3.6 s] per step.
 * The codes clip(rint(q), 0, 3) are compared as well.
 *
 * The reference RN(d / s) is (float)((double)d / (double)s): d has 24
 * significant bits and s 11, so a quotient that is not an fp32 midpoint lies
 * at least 2^-35 of itself away from every midpoint, and rounding to double
 * first cannot move it onto one.
 *
 * Prints "affine2_div <mismatches> affine2_code <mismatches>"; exit status 1
 * if any. Plain C, IEEE single precision with subnormals, no contraction. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bits_f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float half_to_float(uint16_t h) {
  const uint32_t exp = (h >> 10) & 31, man = h & 1023;
  if (exp == 0) return ldexpf((float)man, -24); /* positive subnormal or zero, exact */
  return bits_f(((exp + 112) << 23) | (man << 13));
}

static float recip_div(float d, float s, float r) {
  volatile float q0 = d * r; /* RN(d * r), not fused */
  return fmaf(-fmaf(q0, s, -d), r, q0);
}

static int code_of(float q) {
  float c = rintf(q);
  if (!(c >= 0.0f)) c = 0.0f;
  if (c > 3.0f) c = 3.0f;
  return (int)c;
}

static long long div_bad = 0, code_bad = 0;

static void check(float d, float s, float r) {
  const float q = recip_div(d, s, r);
  const float ref = (float)((double)d / (double)s);
  if (f_bits(q) != f_bits(ref)) {
#pragma omp atomic
    ++div_bad;
  }
  if (code_of(q) != code_of(ref)) {
#pragma omp atomic
    ++code_bad;
  }
}

int main(void) {
#pragma omp parallel for schedule(dynamic, 64)
  for (int h = 1; h <= 0x7BFF; ++h) {
    const float s = half_to_float((uint16_t)h);
    const float r = (float)(1.0 / (double)s); /* RN(1 / s) */
    static const float ts[4] = {0.5f, 1.5f, 2.5f, 3.5f};
    for (int k = 0; k < 4; ++k) {
      const float c = (float)((double)ts[k] * (double)s);
      const int32_t cb = (int32_t)f_bits(c);
      for (int32_t o = -4096; o <= 4096; ++o) {
        const int32_t b = cb + o;
        if (b < 0) continue;
        check(bits_f((uint32_t)b), s, r);
      }
    }
    uint32_t state = 0x9E3779B9u ^ (uint32_t)h;
    for (int i = 0; i < 512; ++i) {
      state = state * 1664525u + 1013904223u;
      const float d = (float)((double)(state >> 8) * (3.6 / 16777216.0) * (double)s);
      check(d, s, r);
    }
  }
  printf("affine2_div %lld affine2_code %lld\n", div_bad, code_bad);
  return div_bad || code_bad ? 1 : 0;
}
