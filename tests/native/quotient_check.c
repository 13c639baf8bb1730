/*
 * Exhaustive check of the per-row quotient used by the quantize kernels.
 *
 * An absmax code is rhaz(fl32(fl32(x*127) / s)) with x an fp16 value and s
 * the row's absmax (also an fp16 value, |x| <= s).  Dividing every element
 * is expensive on the GPU, so the kernels compute r = fl32(1/s) once per row
 * and, per element, n = fl32(x*127), q0 = fl32(n*r), e = fma(-q0, s, n),
 * q = fma(e, r, q0) (a reciprocal-based quotient with one correction step).
 * This program walks every pair of positive fp16 values with x <= s (the
 * operations are symmetric in sign) and reports any pair where q differs
 * from the IEEE quotient fl32(n/s), and any pair where the rounded codes
 * differ.  It also walks every product p = fl32(c * s) of a code c in
 * [-127, 127] and an fp16 scale s (the dequantized outlier weights) and
 * checks the same construction for p / 127 against fl32(p / 127).
 *
 * The kernels round q to the nearest integer, half away from zero, as
 * (int)(fl32(q + copysign(0.5, q))) (truncating conversion).  That is not
 * round-half-away-from-zero for every float (q + 0.5 can itself round up,
 * e.g. for q just below 0.5), so it is also checked here against the exact
 * rule on every quotient the pairs above produce.  A zero scale uses r = 0,
 * which must give code 0 for x = 0 (the only x a zero absmax allows).
 * Exit status 0 iff every count is zero.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float half_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31;
  uint32_t exp = (h >> 10) & 0x1f, man = h & 0x3ff, bits;
  if (exp == 0) {
    if (man == 0) {
      bits = sign;
    } else {  /* subnormal: man * 2^-24 */
      float f = (float)man * 5.9604644775390625e-8f;
      memcpy(&bits, &f, 4);
      bits |= sign;
    }
  } else if (exp == 31) {
    bits = sign | 0x7f800000u | (man << 13);
  } else {
    bits = sign | ((exp - 15 + 127) << 23) | (man << 13);
  }
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

static double rhaz(float v) { return trunc((double)v + copysign(0.5, (double)v)); }

/* the kernels' rounding: fp32 add of +-0.5, then a truncating conversion */
static int gpu_round(float q) {
  const volatile float h = copysignf(0.5f, q);
  const volatile float t = q + h;
  return (int)t;
}

int main(void) {
  long pairs = 0, quot_mismatch = 0, code_mismatch = 0, round_mismatch = 0;
  for (uint32_t hs = 1; hs < 0x7c00; ++hs) {       /* every positive finite s */
    const volatile float s = half_to_float((uint16_t)hs);
    const float r = 1.0f / s;
    for (uint32_t hx = 0; hx <= hs; ++hx) {         /* every x in [0, s] */
      const float x = half_to_float((uint16_t)hx);
      const float n = x * 127.0f;
      const float ref = n / s;
      const float q0 = n * r;
      const float e = fmaf(-q0, s, n);
      const float q = fmaf(e, r, q0);
      ++pairs;
      if (q != ref) ++quot_mismatch;
      if (rhaz(q) != rhaz(ref)) ++code_mismatch;
      if ((double)gpu_round(q) != rhaz(ref) || gpu_round(-q) != -gpu_round(q)) ++round_mismatch;
    }
  }
  {  /* zero scale: r = 0 */
    const volatile float s = 0.0f, r = 0.0f, n = 0.0f * 127.0f;
    const float q0 = n * r, e = fmaf(-q0, s, n), q = fmaf(e, r, q0);
    if (gpu_round(q) != 0) ++round_mismatch;
  }
  long deq = 0, deq_mismatch = 0;
  const volatile float d127 = 127.0f;
  const float r127 = 1.0f / d127;
  for (uint32_t hs = 0; hs < 0x7c00; ++hs) {
    const float s = half_to_float((uint16_t)hs);
    for (int c = -127; c <= 127; ++c) {
      const float p = (float)c * s;
      const float ref = p / d127;
      const float q0 = p * r127;
      const float e = fmaf(-q0, d127, p);
      const float q = fmaf(e, r127, q0);
      ++deq;
      if (q != ref) ++deq_mismatch;
    }
  }
  printf("pairs %ld quotient_mismatch %ld code_mismatch %ld round_mismatch %ld dequant %ld "
         "dequant_mismatch %ld\n",
         pairs, quot_mismatch, code_mismatch, round_mismatch, deq, deq_mismatch);
  return (quot_mismatch == 0 && code_mismatch == 0 && round_mismatch == 0 && deq_mismatch == 0)
             ? 0 : 1;
}
