/* Exhaustive CPU check of the blockwise INT8 quantiser's arithmetic as the
 * gfx950 kernels perform it (block_scale and quant8 in the library's device
 * helpers), against the definition of the quantiser (paperlayer.ai summary of
 * arXiv 2608.17336, "TileMix", §3 Preliminaries and App. C: blockwise
 * symmetric INT8, one scale per block):
 *
 *   scale = fl32(a / 127) for a block maximum a > 0,
 *   q     = clamp(rint_half_even(fl32(x / scale)), -127, 127).
 *
 * The kernels avoid a division per element.  Once per block they form
 * rs = fl32(1 / scale); per element they compute q0 = fl32(x rs),
 * e = fma(-q0, scale, x), q1 = fma(e, rs, q0) (the correction step of
 * Markstein's division), then add 1.5 * 2^23 and keep the low byte of the
 * sum's bit pattern.  This program replays those IEEE single-precision steps
 * (C float arithmetic and fmaf are correctly rounded, ties to even) for every
 * finite fp16 block maximum a and every fp16 x with |x| <= a, both signs, and
 * counts:
 *   - int8 results that differ from the definition;
 *   - quotients q1 that differ from fl32(x / scale) other than in the sign of a zero;
 *   - |q1| above 127 (1 + 2^-23), where a clamp would be needed.
 * It prints "pairs=<n> byte_mismatch=<n> quotient_mismatch=<n> over_range=<n>".
 * Every finite value involved is a normal float32, so the result does not
 * depend on how subnormal float32 values are handled. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float fp16_to_f32(uint16_t h) { /* exact */
  const int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  float v = (e == 0) ? ldexpf((float)m, -24) : ldexpf((float)(m | 0x400), e - 25);
  return s ? -v : v;
}

static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

int main(void) {
  long long pairs = 0, byte_bad = 0, quot_bad = 0, over = 0;
  const float bound = 127.0f * (1.0f + ldexpf(1.0f, -23));
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, byte_bad, quot_bad, over)
  for (int abits = 1; abits <= 0x7BFF; ++abits) {
    const float a = fp16_to_f32((uint16_t)abits);
    const float scale = a / 127.0f;     /* correctly rounded fp32 division */
    const float rs = 1.0f / scale;
    for (int xb = 0; xb <= abits; ++xb) {
      for (int sign = 0; sign < 2; ++sign) {
        const float x = fp16_to_f32((uint16_t)(xb | (sign << 15)));
        /* the kernel's steps */
        const float q0 = x * rs;
        const float er = fmaf(-q0, scale, x);
        const float q1 = fmaf(er, rs, q0);
        const int8_t got = (int8_t)(f32_bits(q1 + 12582912.0f) & 0xFFu);
        /* the definition */
        const float quo = x / scale;
        float r = nearbyintf(quo);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        const int8_t want = (int8_t)r;
        ++pairs;
        if (got != want) ++byte_bad;
        if (!(q1 == quo)) ++quot_bad;   /* +0 == -0: only the sign of a zero may differ */
        if (fabsf(q1) > bound) ++over;
      }
    }
  }
  printf("pairs=%lld byte_mismatch=%lld quotient_mismatch=%lld over_range=%lld\n", pairs, byte_bad, quot_bad, over);
  return (byte_bad || quot_bad || over) ? 1 : 0;
}
