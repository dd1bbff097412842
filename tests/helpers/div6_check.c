/* Exhaustive host check of the quantizer's division of a block amax by 6.
 *
 * The device computes t / 6 as q0 = fl(t * c) with c = fl(1/6), then
 * q1 = fma(fma(-q0, 6, t), c, q0) (one correction step with the exact fma
 * residual, after Markstein).  This program compares q1 with the correctly
 * rounded IEEE quotient t / 6 for every binary32 bit pattern t in
 * [2^-125, FLT_MAX] and prints the number of mismatches (expected 0).  It
 * also prints the mismatch count below 2^-125, where the encode result is
 * the zero scale byte either way. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float q_corrected(float t) {
  const float c = 1.0f / 6.0f;
  const float q0 = t * c;
  return fmaf(fmaf(-q0, 6.0f, t), c, q0);
}

static uint64_t count(uint32_t lo, uint32_t hi) {
  uint64_t bad = 0;
  for (uint32_t b = lo; b < hi; ++b) {
    float t, q, q1;
    memcpy(&t, &b, 4);
    q = t / 6.0f;
    q1 = q_corrected(t);
    bad += memcmp(&q, &q1, 4) != 0;
  }
  return bad;
}

int main(void) {
  const uint64_t normal = count(0x01000000u, 0x7F800000u); /* 2^-125 .. FLT_MAX */
  const uint64_t tiny = count(0u, 0x01000000u);
  printf("%llu %llu\n", (unsigned long long)normal, (unsigned long long)tiny);
  return 0;
}
