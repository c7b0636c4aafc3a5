/* Exhaustive check of the page encoder's division: q = x / s computed as
 *
 *     r  = RN(1 / s)                      (once per block or group)
 *     q0 = RN(x * r)
 *     q  = fma(-fma(q0, s, -x), r, q0)    (one correction; the residual is exact)
 *
 * decides every stored code exactly as the correctly rounded RN(x / s) does,
 * for every input the encoder can meet (a block or group whose absmax is m
 * holds only values with |x| <= m):
 *
 *   fp8: s = RN(m / 448) for every positive finite source value m (fp16; bf16
 *        with s >= 2^-100, smaller scales taking the correctly rounded
 *        division), x every value of the same format with |x| <= m. q2 must
 *        equal RN(x / s) bit for bit where |RN(x / s)| >= 2^-11; below, both
 *        round to the e4m3 code +-0, so q must have the same sign and
 *        |q| < 2^-10.
 *   int: s = fp16(RN(m / qmax)) kept inside [2^-24, 65504], qmax 127 and 7,
 *        for every positive finite m of either format, x every value of that
 *        format with |x| <= m: the codes clip(rint(q), -qmax, qmax) must agree.
 *
 * Prints the mismatches per domain; exit status 1 if any. Plain C, IEEE
 * single precision with subnormals (no fast-math), as on the device (fp32
 * denormals preserved, IEEE mode). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bits_f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float half_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31, exp = (h >> 10) & 31, man = h & 1023;
  if (exp == 0) {  /* zero or subnormal: man * 2^-24, exact */
    float v = ldexpf((float)man, -24);
    return sign ? -v : v;
  }
  if (exp == 31) return bits_f(sign | 0x7f800000u | (man << 13));
  return bits_f(sign | ((exp + 112) << 23) | (man << 13));
}
static float bf16_to_float(uint16_t b) { return bits_f((uint32_t)b << 16); }

static float recip_div(float x, float s, float r) {
  const float q0 = x * r;
  return fmaf(-fmaf(q0, s, -x), r, q0);
}

static int code_of(float q, float qmax) {
  float c = rintf(q);
  if (!(c >= -qmax)) c = -qmax; /* NaN cannot occur: s > 0 finite, x finite */
  if (c > qmax) c = qmax;
  return (int)c;
}

static uint16_t float_to_half_rne(float f) {  /* finite, positive */
  /* nearest fp16 by comparison with its neighbours: exact and simple */
  int lo = 0, hi = 31744;  /* codes 0 .. 0x7BFF are the finite positives, ascending */
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (half_to_float((uint16_t)mid) <= f) lo = mid; else hi = mid;
  }
  if (lo == 31743) {  /* at or above 65504: infinity if at least 65520 */
    return f >= 65520.0f ? 0x7C00 : 0x7BFF;
  }
  const float a = half_to_float((uint16_t)lo), b = half_to_float((uint16_t)(lo + 1));
  const double da = (double)f - a, db = (double)b - f;
  if (da < db) return (uint16_t)lo;
  if (db < da) return (uint16_t)(lo + 1);
  return (lo & 1) ? (uint16_t)(lo + 1) : (uint16_t)lo;
}

static float int_scale(float m, float qmax) {
  uint16_t h = float_to_half_rne(m / qmax);
  if (h == 0) h = 1;              /* 2^-24 */
  if (h >= 0x7C00) h = 0x7BFF;    /* 65504 */
  return half_to_float(h);
}

int main(void) {
  static float vals[2][32640];
  const int count[2] = {31744, 32640};
  for (int k = 0; k < 31744; ++k) vals[0][k] = half_to_float((uint16_t)k);
  for (int k = 0; k < 32640; ++k) vals[1][k] = bf16_to_float((uint16_t)k);
  long long bad_fp8[2] = {0, 0}, bad_int[2] = {0, 0};
  for (int fmt = 0; fmt < 2; ++fmt) {
    const float* v = vals[fmt];
    long long bf = 0, bi = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : bf, bi)
    for (int im = 1; im < count[fmt]; ++im) {
      const float m = v[im];
      const float s8 = m / 448.0f, r8 = 1.0f / s8;
      const int fp8_fast = s8 >= 0x1p-100f;
      const float s127 = int_scale(m, 127.0f), r127 = 1.0f / s127;
      const float s7 = int_scale(m, 7.0f), r7 = 1.0f / s7;
      for (int ix = 0; ix <= im; ++ix)
        for (int sg = 0; sg < 2; ++sg) {
          const float x = sg ? -v[ix] : v[ix];
          if (fp8_fast) {
            const float qa = recip_div(x, s8, r8), qb = x / s8;
            if (fabsf(qb) >= 0x1p-11f) bf += f_bits(qa) != f_bits(qb);
            else bf += (signbit(qa) != signbit(qb)) || !(fabsf(qa) < 0x1p-10f);
          }
          bi += code_of(recip_div(x, s127, r127), 127.0f) != code_of(x / s127, 127.0f);
          bi += code_of(recip_div(x, s7, r7), 7.0f) != code_of(x / s7, 7.0f);
        }
    }
    bad_fp8[fmt] = bf;
    bad_int[fmt] = bi;
  }
  printf("fp8_fp16 %lld fp8_bf16 %lld int_fp16 %lld int_bf16 %lld\n", bad_fp8[0], bad_fp8[1], bad_int[0],
         bad_int[1]);
  return (bad_fp8[0] || bad_fp8[1] || bad_int[0] || bad_int[1]) ? 1 : 0;
}
