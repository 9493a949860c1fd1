/* The quotient identity the coding kernels rely on, checked exhaustively on the host.
 *
 * For a block maximum m (every positive finite fp16 value), the scale is s = fl32(m / L) and its
 * reciprocal r = fl32(1 / s), both IEEE fp32 divisions.  For every fp16 value x with |x| <= m the
 * kernels form y = fl32(x * r), e = fma(-y, s, x), q = fma(e, r, y) and use q in place of the
 * division fl32(x / s).  This program checks q == fl32(x / s) for every such (m, x) pair and that
 * |rint(x / s)| <= L.  Usage: quotient_identity L  (prints one line; exit status 0 when it holds).
 * Build without contraction (-ffp-contract=off) so that every product is rounded as written. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

static float half_value(uint16_t h) {
  const uint32_t e = (h >> 10) & 31, m = h & 1023;
  return e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), (int)e - 25);
}

int main(int argc, char** argv) {
  const float L = argc > 1 ? (float)atof(argv[1]) : 127.f;
  static float mag[0x7C00];
  int n = 0;
  for (uint32_t h = 0; h < 0x7C00; ++h) mag[n++] = half_value((uint16_t)h);  /* ascending */
  long long checked = 0, wrong = 0, out_of_range = 0;
  for (int im = 1; im < n; ++im) {
    volatile float lv = L, one = 1.f;
    const float s = mag[im] / lv;
    const float r = one / s;
    for (int ix = 0; ix <= im; ++ix) {
      for (int neg = 0; neg < 2; ++neg) {
        const float x = neg ? -mag[ix] : mag[ix];
        volatile float yv = x * r;
        const float y = yv;
        const float q = fmaf(fmaf(-y, s, x), r, y);
        volatile float dv = x / s;
        const float d = dv;
        ++checked;
        if (q != d) {
          if (wrong < 5) printf("differs: m=%a s=%a x=%a q=%a x/s=%a\n", mag[im], s, x, q, d);
          ++wrong;
        }
        if (fabsf(rintf(d)) > L) ++out_of_range;
      }
    }
  }
  printf("L=%g pairs=%lld differ=%lld codes_out_of_range=%lld\n", L, checked, wrong, out_of_range);
  return (wrong || out_of_range) ? 1 : 0;
}
