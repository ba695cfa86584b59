/*
 * Exhaustive host check of the quotient the quantisation kernels use.
 *
 * The kernels form x / s for e4m3 quantisation (s = amax / 448 in fp32) not
 * by an IEEE division per value but, once per group, the correctly rounded
 * reciprocal y = 1 / s, and per value
 *     q0 = x * y,  r = fma(-q0, s, x),  q = copysign(fma(r, y, q0), x)
 * -- Markstein's fma-based correction of a reciprocal-based quotient
 * (P. Markstein, "Computation of elementary functions on the IBM RISC
 * System/6000 processor", IBM J. Res. Dev. 34(1), 1990): r is the exact
 * residual of q0 and one fma step moves q0 towards the correctly rounded
 * quotient. The result is not always the correctly rounded quotient, but
 * what matters is the e4m3 code after clamping to +-448 and rounding to
 * nearest-even; the claim is that this code equals the code of the IEEE
 * division for every bf16 x with |x| <= amax, for every bf16 amax >= 2^-96
 * (below that the kernels divide).
 *
 * This program checks exactly that, over every positive finite bf16 amax
 * >= 2^-96 and every bf16 x in [0, amax] (about 5.2e8 pairs); negative x
 * follow by symmetry (every step is odd in x under round-to-nearest), and
 * are checked on every 17th amax anyway. The e4m3 rounding here is written
 * from the OCP 8-bit float definition (bias 7, 3 mantissa bits, subnormals
 * below 2^-6, max 448). Prints the number of pairs checked, the number
 * whose fp32 quotients differ, and the number whose codes differ (must be
 * 0), and exits 1 on a code mismatch.
 *
 * With the argument "encode" it instead reads one hex float per line from
 * stdin and prints the e4m3 code (decimal) of each, so that a test can
 * compare this encoder with an independent one. Built with -DUNCORRECTED
 * the check skips the correction step (q = q0), which must then report code
 * mismatches: the check can fail.
 *
 * The same run checks the quotient the fused GEMM uses instead (its codes
 * feed only the MFMA, so the sign of a zero code does not matter there):
 * y_hi = RN(1 / s), y_lo = RN(RN(1 - s y_hi) y_hi) once per group and
 * q = fma(x, y_hi, RN(x y_lo)) per value, without a clamp. Its code must
 * equal the division's for every x != 0 (x = +-0 may give either zero), and
 * |q| must stay <= 448 (1 + 2^-23), where the hardware conversion still
 * rounds to 448 (it gives the NaN code only above 464). Printed as
 * gemm_code_differs, gemm_zero_sign_differs and gemm_qmax_over.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off quotient_check.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16_value(uint32_t pattern) {
  const uint32_t w = pattern << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return f;
}

/* e4m3fn code of v, |v| <= 448, round to nearest even, sign kept. */
static unsigned e4m3_code(float v) {
  const unsigned sign = signbit(v) ? 0x80u : 0u;
  const float a = fabsf(v);
  unsigned mag;
  if (a < 0x1p-6f) {
    /* subnormal range: the quantum is 2^-9; a * 2^9 is exact */
    mag = (unsigned)nearbyintf(a * 0x1p9f); /* 0..8; 8 is the first normal code */
  } else {
    int e;
    const float f = frexpf(a, &e); /* a = f * 2^e, f in [0.5, 1) */
    const float m = nearbyintf((2.0f * f - 1.0f) * 8.0f); /* 0..8, exact inputs */
    mag = (unsigned)(((e - 1 + 7) << 3) + (int)m);       /* m == 8 carries into the exponent */
  }
  return sign | mag;
}

static float clamp448(float q) { return fminf(fmaxf(q, -448.0f), 448.0f); }
/* e4m3_code() of magnitudes in (448, 464] gives 0x7E, as the conversion
   instruction does (ties at 464 go to the even code, 448). */

int main(int argc, char** argv) {
  if (argc > 1 && strcmp(argv[1], "encode") == 0) {
    char line[128];
    while (fgets(line, sizeof line, stdin)) {
      float v;
      if (sscanf(line, "%a", &v) == 1) printf("%u\n", e4m3_code(clamp448(v)));
    }
    return 0;
  }
  const uint32_t first_amax = 31u << 7; /* bf16 exponent field 31: 2^-96 */
  const uint32_t last_amax = 0x7F7Fu;   /* largest finite bf16 */
  unsigned long long pairs = 0, quot_diff = 0, code_diff = 0;
  unsigned long long g_code_diff = 0, g_zero_sign = 0, g_over = 0;
  const float qbound = 448.0f * (1.0f + 0x1p-23f);
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, quot_diff, code_diff, g_code_diff, g_zero_sign, g_over)
  for (uint32_t pa = first_amax; pa <= last_amax; ++pa) {
    const float amax = bf16_value(pa);
    const float s = amax / 448.0f;
    const float y = 1.0f / s;
    const float y_lo = fmaf(-s, y, 1.0f) * y;
    const int with_negative = (pa % 17u) == 0;
    for (uint32_t px = 0; px <= pa; ++px) {
      for (int neg = 0; neg <= with_negative; ++neg) {
        const float x = neg ? -bf16_value(px) : bf16_value(px);
        const float q_div = x / s;
        const float q0 = x * y;
        const float r = fmaf(-q0, s, x);
#ifdef UNCORRECTED
        const float q_fma = q0 + 0.0f * r;
#else
        const float q_fma = copysignf(fmaf(r, y, q0), x);
#endif
        ++pairs;
        if (memcmp(&q_div, &q_fma, sizeof q_div) != 0) ++quot_diff;
        const float q_gemm = fmaf(x, y, x * y_lo);
        if (fabsf(q_gemm) > qbound) ++g_over;
        if (e4m3_code(clamp448(q_div)) != e4m3_code(q_gemm)) {
          if (x == 0.0f) ++g_zero_sign;
          else ++g_code_diff;
        }
        if (e4m3_code(clamp448(q_div)) != e4m3_code(clamp448(q_fma))) {
          ++code_diff;
#ifndef UNCORRECTED
#pragma omp critical
          fprintf(stderr, "code mismatch: amax %a x %a: div %a fma %a\n", amax, x, q_div, q_fma);
#endif
        }
      }
    }
  }
  printf("pairs %llu quotient_differs %llu code_differs %llu gemm_code_differs %llu gemm_zero_sign_differs %llu "
         "gemm_qmax_over %llu\n",
         pairs, quot_diff, code_diff, g_code_diff, g_zero_sign, g_over);
  return code_diff == 0 && g_code_diff == 0 && g_over == 0 ? 0 : 1;
}
