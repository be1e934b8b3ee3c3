/* Host check of the short form of the row quantization used by the library's
 * kernels (the same float operations, written again here in C):
 *   scale448(a)       = q0 + (a - q0 * 448) * r448 (fused), q0 = a * r448,
 *                       r448 = RN(1/448)
 *   div_signed(x,s,r) = q0 - (q0 * s - x) * r (fused),  q0 = x * r, r = RN(1/s)
 * Claims checked:
 *   1. scale448(a) == RN(a / 448) for EVERY float a in [448 * 2^-100, FLT_MAX];
 *   2. div_signed(x, s, r) == RN(x / s), sign of zero included, for sampled x
 *      and s >= 2^-100 (normal), including x = +-0 and |x| = amax.
 * Prints "scale448 mismatches N" and "div_signed mismatches M" (both 0 when
 * the claims hold). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float fbits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bitsf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float scale448(float a) {
  const float r = 1.0f / 448.0f;
  const float q0 = a * r;
  return fmaf(fmaf(-q0, 448.0f, a), r, q0);
}
/* (compiled without optimization: GCC rewrites -(a b + c) as (-a) b - c, which
 * gives the opposite sign when the result is an exact zero) */
__attribute__((noinline, optimize("O0"))) static float div_signed(float x, float s, float r) {
  const float q0 = x * r;
  const float e = fmaf(q0, s, -x);
  return fmaf(-e, r, q0);
}
/* splitmix64: a counter-based generator for the sampled part */
static uint64_t mix(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int main(void) {
  const uint32_t lo = bitsf(0x1.cp-92f), hi = 0x7F7FFFFFu;
  unsigned long bad1 = 0;
#pragma omp parallel for reduction(+ : bad1) schedule(static)
  for (int64_t u = lo; u <= (int64_t)hi; ++u) {
    const float a = fbits((uint32_t)u);
    if (bitsf(scale448(a)) != bitsf(a / 448.0f)) ++bad1;
  }
  printf("scale448 mismatches %lu\n", bad1);

  unsigned long bad2 = 0;
  const long n = 1L << 26;
#pragma omp parallel for reduction(+ : bad2) schedule(static)
  for (long i = 0; i < n; ++i) {
    const uint64_t z = mix((uint64_t)i);
    /* amax over the fast range's exponents, a scale from it, x a fraction of amax */
    const uint32_t ea = 35 + (uint32_t)(z % 219);               /* amax exponent field 35..253 */
    const float amax = fbits((ea << 23) | (uint32_t)((z >> 8) & 0x7FFFFF));
    const float s = amax / 448.0f;
    const float r = 1.0f / s;
    float x;
    switch ((z >> 40) & 7) {
      case 0: x = amax; break;
      case 1: x = -amax; break;
      case 2: x = 0.0f; break;
      case 3: x = -0.0f; break;
      default: {
        const float f = (float)((z >> 44) & 0xFFFFF) / 1048576.0f;  /* [0, 1) */
        x = ((z >> 43) & 1) ? -amax * f : amax * f;
      }
    }
    const float got = div_signed(x, s, r), want = x / s;
    if (bitsf(got) != bitsf(want)) ++bad2;
  }
  printf("div_signed mismatches %lu\n", bad2);
  return 0;
}
