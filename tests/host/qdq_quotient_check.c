/* Host check of the FP8 QDQ quotient used by the GPU kernels: for a scale s in
 * [2^-90, 2^90] with y = RN(1/s), and every finite bfloat16 x,
 *   q  = clamp(RN(x * y), +-512)
 *   r  = RN(q * s - x)            (one fused multiply-add: exact)
 *   q1 = RN(q - r * y)            (one fused multiply-add)
 *   v  = copysign(clamp(q1, +-448), x)
 * must round to the same E4M3 value (sign of zero included) as the IEEE
 * quotient RN(x / s) clamped to +-448, and q1 must equal RN(x / s) wherever
 * 2^-12 <= |x / s| <= 512.  (A correction step of Markstein's: the residual
 * of a quotient within an ulp is exact, and one more step rounds correctly.)
 * Usage: qdq_quotient_check <stride over bf16 amax values> <random scales>
 * Prints the number of cases checked and of mismatches; exit status 1 on any. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
/* the GPU's v_med3 against +-c: ordered compares, a zero keeps its sign */
static float med3c(float v, float c) { return v < -c ? -c : (v > c ? c : v); }
/* E4M3 (OCP, bias 7, 3 mantissa bits, subnormal step 2^-9) round to nearest
 * even of |v| <= 448, by exact scaling and nearbyintf (ties to even) */
static float e4m3(float v) {
  float a = fabsf(v), r;
  if (a < 0x1p-6f) {
    r = nearbyintf(a * 512.0f) / 512.0f;
  } else {
    int e;
    frexpf(a, &e);
    const float quantum = ldexpf(1.0f, e - 4);
    r = nearbyintf(a / quantum) * quantum;
  }
  return copysignf(r, v);
}

static long long checked = 0, bad = 0;

static void check_scale(float s) {
  if (!(s >= 0x1p-90f && s <= 0x1p90f)) return;
  volatile float one = 1.0f;
  const float y = one / s;
  for (uint32_t b = 0; b < 65536; ++b) {
    const float x = f_of(b << 16);
    if (isnan(x)) continue;
    const float t = x / s;
    const float q = med3c(x * y, 512.0f);
    const float r = fmaf(q, s, -x);
    const float q1 = fmaf(-r, y, q);
    const float v = copysignf(med3c(q1, 448.0f), x);
    ++checked;
    int ok = u_of(e4m3(v)) == u_of(e4m3(med3c(t, 448.0f)));
    const float at = fabsf(t);
    if (at >= 0x1p-12f && at <= 512.0f) ok = ok && u_of(q1) == u_of(t);
    if (!ok) {
      if (bad < 5) printf("mismatch: s=%a x=%a x/s=%a corrected=%a\n", s, x, t, q1);
      ++bad;
    }
  }
}

int main(int argc, char** argv) {
  const int stride = argc > 1 ? atoi(argv[1]) : 1;
  const int nrand = argc > 2 ? atoi(argv[2]) : 1000;
  /* the scales the method produces: RN(amax / 448) for bf16 amax */
  for (uint32_t b = 1; b < 0x7f80; b += (uint32_t)stride) check_scale(f_of(b << 16) / 448.0f);
  /* random scales over the range, and mantissa edge patterns */
  srand(12345);
  for (int i = 0; i < nrand; ++i) {
    const uint32_t m = (((uint32_t)rand() << 8) ^ (uint32_t)rand()) & 0x7fffffu;
    check_scale(f_of((uint32_t)(37 + rand() % 181) << 23 | m));
  }
  const uint32_t edges[] = {0, 1, 2, 0x7fffff, 0x7ffffe, 0x400000, 0x3fffff, 0x400001, 0x555555};
  for (int e = 37; e <= 217; e += 9)
    for (unsigned k = 0; k < sizeof edges / sizeof edges[0]; ++k)
      check_scale(f_of((uint32_t)e << 23 | edges[k]));
  printf("checked %lld mismatches %lld\n", checked, bad);
  return bad != 0;
}
