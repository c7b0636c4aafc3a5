/* Exhaustive check of the two divisions the page encoder makes per INT group:
 *
 *   scale:      s = RN(m / qmax) for the group's absmax m, computed as
 *                 R  = RN(1 / qmax)                 (a compile-time constant)
 *                 q0 = RN(m * R)
 *                 s  = fma(-fma(q0, qmax, -m), R, q0)
 *               must equal the correctly rounded quotient bit for bit, for
 *               every positive finite m of fp16 and of bf16 and qmax 127, 7
 *               (and 448, the FP8 block divisor).
 *   reciprocal: r = RN(1 / s) for the stored fp16 scale s in [2^-24, 65504],
 *               computed from the hardware reciprocal estimate r0 (within one
 *               unit in the last place of 1 / s) by one Newton step
 *                 r = fma(r0, fma(-s, r0, 1), r0)
 *               must equal the correctly rounded reciprocal for every fp16 s
 *               and every r0 within two units in the last place of RN(1 / s)
 *               (a margin over the estimate's documented accuracy).
 *
 * Prints the mismatches per part; exit status 1 if any. Plain C, IEEE single
 * precision with subnormals, no fast-math, as on the device. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bits_f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float half_to_float(uint16_t h) {  /* finite, positive codes only */
  const uint32_t exp = (h >> 10) & 31, man = h & 1023;
  if (exp == 0) return ldexpf((float)man, -24);
  return bits_f(((exp + 112) << 23) | (man << 13));
}
static float bf16_to_float(uint16_t b) { return bits_f((uint32_t)b << 16); }

static float scale_div(float m, float qmax, float r) {
  const float q0 = m * r;
  return fmaf(-fmaf(q0, qmax, -m), r, q0);
}

int main(void) {
  long long bad_scale = 0, bad_recip = 0;
  const float qmaxs[3] = {127.0f, 7.0f, 448.0f};
  for (int iq = 0; iq < 3; ++iq) {
    const float qmax = qmaxs[iq], r = 1.0f / qmax;
    for (int k = 1; k < 0x7C00; ++k) {  /* fp16 positive finite */
      const float m = half_to_float((uint16_t)k);
      bad_scale += f_bits(scale_div(m, qmax, r)) != f_bits(m / qmax);
    }
    for (int k = 1; k < 0x7F80; ++k) {  /* bf16 positive finite */
      const float m = bf16_to_float((uint16_t)k);
      bad_scale += f_bits(scale_div(m, qmax, r)) != f_bits(m / qmax);
    }
  }
  for (int k = 1; k < 0x7C00; ++k) {
    const float s = half_to_float((uint16_t)k), exact = 1.0f / s;
    for (int d = -2; d <= 2; ++d) {
      const float r0 = bits_f(f_bits(exact) + (uint32_t)d);
      const float r = fmaf(r0, fmaf(-s, r0, 1.0f), r0);
      bad_recip += f_bits(r) != f_bits(exact);
    }
  }
  printf("scale_div %lld recip_fp16 %lld\n", bad_scale, bad_recip);
  return (bad_scale || bad_recip) ? 1 : 0;
}
