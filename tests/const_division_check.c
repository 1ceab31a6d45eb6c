/* Check of the shortcut that the WENO kernels use for x / 6 and x / 12:
 * q = x * rd, then q + (x - q * d) * rd with both steps as fused multiply-adds,
 * rd = 1 / d rounded to fp32 (Markstein's division step), against the IEEE
 * quotient x / d.
 *
 * Every positive x of the exponent fields 0 (zero and subnormals) to 27 is
 * tried, and of the fields 100, 200 and 254.  From field 27 on, x * rd, the
 * remainder x - q * d (exact, a nonzero multiple of 2^(field - 153)) and the
 * result are all normal and finite, so scaling x by a power of two scales
 * every step exactly: the outcome for fields 27..254 is that of field 27 (the
 * three later fields are tried as a check of that).  For nonzero x the result
 * for -x is the exact negation (round-to-nearest-even is odd), so this covers
 * every finite nonzero x; of the zeros, +0 is among the patterns tried and -0
 * is tried alone: it gives +0, not the IEEE -0.
 *
 * Prints, per divisor, the number of disagreeing x tried and the exponent
 * field from which all agree; exit status 0 when both agree for zero and for
 * every finite x of exponent field >= 3 (|x| >= 2^-124). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float x; memcpy(&x, &u, sizeof x); return x; }
static uint32_t to_bits(float x) { uint32_t u; memcpy(&u, &x, sizeof u); return u; }

static long disagreements(uint32_t field, float d, float rd) {
  long bad = 0;
  for (uint32_t m = 0; m < (1u << 23); ++m) {
    const float x = from_bits((field << 23) | m);
    const float q0 = x * rd;
    const float q = fmaf(fmaf(-q0, d, x), rd, q0);
    bad += to_bits(q) != to_bits(x / d);
  }
  return bad;
}

int main(void) {
  const float divisors[2] = {6.0f, 12.0f};
  uint32_t fields[31];
  int n = 0;
  for (uint32_t f = 0; f <= 27; ++f) fields[n++] = f;
  fields[n++] = 100, fields[n++] = 200, fields[n++] = 254;
  int status = 0;
  for (int k = 0; k < 2; ++k) {
    const float d = divisors[k];
    const float rd = 1.0f / d;
    long bad_by_field[31] = {0};
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n; ++i) bad_by_field[i] = disagreements(fields[i], d, rd);
    long bad = 0;
    int top_bad = -1;
    for (int i = 0; i < n; ++i) {
      bad += bad_by_field[i];
      if (bad_by_field[i]) top_bad = (int)fields[i];
    }
    printf("d=%g: %ld x disagree, all agree from exponent field %d on\n", d, bad, top_bad + 1);
    if (top_bad >= 3) status = 1;
    const float mz = -0.0f, q0 = mz * rd, q = fmaf(fmaf(-q0, d, mz), rd, q0);
    printf("d=%g: -0 gives %s0 (IEEE %s0)\n", d, signbit(q) ? "-" : "+", signbit(mz / d) ? "-" : "+");
    if (signbit(q) || !signbit(mz / d)) status = 1;  /* the documented +0 */
  }
  return status;
}
