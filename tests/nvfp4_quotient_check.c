/* nvfp4_quotient_check.c -- host-side check of the division-free quotient
 * the NVFP4 RoPE insert kernel uses for y = r / S (S a positive E4M3 value).
 *
 * With y0 the hardware fp32 reciprocal of S (within 1 ulp of 1/S), the
 * kernel forms, in fp32 with single roundings,
 *   q0 = r * y0,  e = fma(-q0, S, r)  (exact: at most 6 significant bits),
 *   q  = fma(e, y0, q0),
 * and keeps q when it is a normal float.  Otherwise (a zero, subnormal,
 * infinite or NaN quotient: underflowing residuals, or r too large) it takes
 *   inv_s = fma(y0, fma(-S, y0, 1), y0) * (1 - 2^-50)      (all in fp64),
 *   q     = fp32(fp64(r) * inv_s),
 * and quantises q to E2M1 (nearest, ties to even, saturating at 6, sign bit
 * only for q < 0).  The NVFP4 definition (DeepSeek-V4.1 insert page, NVFP4
 * branch) quantises the correctly rounded fp32 quotient r / S instead.  This
 * program checks that both give the same 4-bit code, and counts the kept
 * quotients of magnitude 2^-100 or more that differ from r / S in any bit
 * (expected: none; below that only the sign reaches the code, and a kept q
 * is normal, nonzero and of the quotient's sign).
 *
 * y0 is unknown beyond its 1-ulp bound, so every float within 2 ulps of 1/S
 * is tried.  Scale invariance: for normal quotients the outcome depends on
 * the significands of r and S only (S's exponent moves y0, inv_s and the
 * quotient by the same power of two), so S runs over the 8 E4M3 significands
 * (1, 1.125, .., 1.875; the E4M3 subnormals m * 2^-9 have these too) and r
 * over every float in [2^-4, 2^4) (quotients from 2^-5 to 16 cover every
 * E2M1 decision and saturation).  Subnormal quotients, where only the sign
 * matters, are swept around the zero/nonzero boundary for every E4M3 S.
 *
 * Usage: nvfp4_quotient_check [stride]  -- stride 1 (default) is every float
 * of the range; a larger stride samples the significands.  Prints the number
 * of cases and mismatches; exits 1 on any mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* E2M1 code of a float by the midpoints 0.25, 0.75, ..., 5 (ties to the even
 * code: ">" where the lower code is even, ">=" where the upper one is). */
static int e2m1(float q) {
  if (q != q) q = 0.0f;
  float a = fabsf(q);
  int m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return (q < 0.0f ? 8 : 0) | m;
}

static double inv_s_of(float S, float y0f) {
  const double sd = S, y0 = y0f;
  return fma(y0, fma(-sd, y0, 1.0), y0) * (1.0 - 0x1p-50);
}

static long long cases, bad, bits;

static void check(float r, float S, float y0) {
  const float truth = r / S;
  const float q0 = r * y0;
  const float e = fmaf(-q0, S, r);
  float q = fmaf(e, y0, q0);
  const int fast = fpclassify(q) == FP_NORMAL;
  if (!fast) q = (float)((double)r * inv_s_of(S, y0));
  ++cases;
  if (fast && fabsf(truth) >= 0x1p-100f && u_of(q) != u_of(truth)) ++bits;
  if (e2m1(truth) != e2m1(q)) {
    if (bad < 10)
      fprintf(stderr, "mismatch r=%a S=%a truth=%a q=%a\n", (double)r, (double)S, (double)truth, (double)q);
    ++bad;
  }
}

/* The reciprocal candidates: floats within 2 ulps of 1/S. */
static int candidates(float S, float out[5]) {
  const float rn = 1.0f / S;
  int k = 0;
  uint32_t u = u_of(rn);
  for (int d = -2; d <= 2; ++d) {
    const float c = f_of(u + (uint32_t)d);
    if (fabs((double)c - 1.0 / (double)S) <= 2.0 * (double)(nextafterf(rn, INFINITY) - rn)) out[k++] = c;
  }
  return k;
}

int main(int argc, char** argv) {
  const uint32_t stride = argc > 1 ? (uint32_t)strtoul(argv[1], NULL, 10) : 1u;
  /* normal quotients: 8 significands x every float of [2^-4, 2^4), both signs */
  const uint32_t lo = u_of(0x1p-4f), hi = u_of(0x1p4f);
  for (int m = 0; m < 8; ++m) {
    const float S = 1.0f + (float)m / 8.0f;
    float c[5];
    const int nc = candidates(S, c);
    for (int k = 0; k < nc; ++k) {
      for (uint32_t u = lo; u < hi; u += stride) {
        check(f_of(u), S, c[k]);
        check(-f_of(u), S, c[k]);
      }
    }
  }
  /* every E4M3 scale the kernel can produce (2^-9 .. 448): specials, the
   * extremes, and subnormal quotients around half the smallest subnormal */
  for (uint32_t s8 = 1; s8 <= 0x7E; ++s8) {
    const uint32_t ef = s8 >> 3, mf = s8 & 7u;
    const float S = ef == 0 ? (float)mf * 0x1p-9f : ldexpf(1.0f + (float)mf / 8.0f, (int)ef - 7);
    float c[5];
    const int nc = candidates(S, c);
    for (int k = 0; k < nc; ++k) {
      const float y0 = c[k];
      const float specials[] = {0.0f, INFINITY, NAN, 3.4028235e38f, 0x1p-149f, 0x1p-126f, 6.0f * S, 6.5f * S,
                                5.0f * S, 0.25f * S};
      for (unsigned i = 0; i < sizeof specials / sizeof specials[0]; ++i) {
        check(specials[i], S, y0);
        check(-specials[i], S, y0);
      }
      /* r near 2^-150 * S (the quotient that rounds to 0 or to 2^-149) */
      const double edge = 0x1p-150 * (double)S;
      const float e = (float)edge;
      for (int d = -4096; d <= 4096; ++d) {
        const float r = f_of(u_of(e) + (uint32_t)d);
        if (!(r > 0.0f)) continue;
        check(r, S, y0);
        check(-r, S, y0);
      }
      /* every subnormal float as r (quotients far below 2^-126) */
      for (uint32_t u = 1; u < 0x00800000u; u += 97u * stride) {
        check(f_of(u), S, y0);
        check(-f_of(u), S, y0);
      }
      /* quotients around the bottom of the normal range (r near S * 2^-126) */
      const float nb = (float)(0x1p-126 * (double)S);
      for (int d = -4096; d <= 4096; ++d) {
        const float r = f_of(u_of(nb) + (uint32_t)d);
        if (!(r > 0.0f)) continue;
        check(r, S, y0);
        check(-r, S, y0);
      }
    }
  }
  printf("cases %lld mismatches %lld quotients_off_by_bits %lld\n", cases, bad, bits);
  return bad || bits ? 1 : 0;
}
