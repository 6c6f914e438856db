// Exhaustive host check of the FP8 quantizers' quotient (div_by_scale in the
// library): for every block scale s = max(amax, 1e-4f) / 448 (amax any finite
// bf16 magnitude) and every finite bf16 value |a| <= max(amax, 1e-4), the
// quotient from y = 1/s (correctly rounded), q = a*y, r = fma(-q, s, a) and
// q + r*y (fma; q itself when r == 0) gives the e4m3 code the correctly
// rounded a / s gives: equal bits where |a/s| > 2^-11, otherwise the same sign
// and a magnitude <= 2^-10 (both round to the code +-0).  The arithmetic is
// written out here from that description, independently of the library.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float bf16_to_f(uint16_t h) { uint32_t u = (uint32_t)h << 16; float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
int main(void) {
  long n = 0, bad = 0;
  for (uint32_t hb = 0; hb < 0x7f80; ++hb) {           // amax: every finite non-negative bf16
    const float amax = bf16_to_f((uint16_t)hb);
    const float s = fmaxf(amax, 1e-4f) / 448.0f;
    if (hb > 0 && fmaxf(bf16_to_f((uint16_t)(hb - 1)), 1e-4f) == fmaxf(amax, 1e-4f)) continue;  // same scale
    const float y = 1.0f / s;
    for (uint32_t ha = 0; ha < 0x10000; ++ha) {
      if ((ha & 0x7f80) == 0x7f80) continue;            // inf / nan
      const float a = bf16_to_f((uint16_t)ha);
      if (fabsf(a) > fmaxf(amax, 1e-4f)) continue;       // a block's values never exceed its amax
      const float want = a / s;
      const float q = a * y;
      const float r = fmaf(-q, s, a);
      const float got = r == 0.0f ? q : fmaf(r, y, q);
      ++n;
      // quotients of magnitude <= 2^-10 all take the e4m3 code +-0: there only
      // the sign has to agree
      const int tiny = fabsf(want) <= 0x1p-11f;
      const int same = tiny ? (fabsf(got) <= 0x1p-10f && signbit(got) == signbit(want))
                            : (bits(got) == bits(want));
      if (!same) {
        if (bad < 10) printf("mismatch amax %g a %g: want %.9g got %.9g\n", amax, a, want, got);
        ++bad;
      }
    }
  }
  printf("checked %ld, mismatches %ld\n", n, bad);
  return bad != 0;
}
