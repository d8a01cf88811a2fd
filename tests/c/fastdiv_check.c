/* Exhaustive check, over every float32 numerator n, that the three-operation
 * division used by the four-over-six kernel,
 *     r = fl(1/D); q0 = n*r; rem = fma(-q0, D, n); q = fma(rem, r, q0),
 * equals the correctly rounded n / D whenever |n| >= 2^-117 and n is finite
 * (exponent field 10..254).  Also checks the block-scale division a / 6 for
 * every bf16 value a >= 0 with exponent field >= 10.  Prints the number of
 * mismatches inside the claimed range (must be 0) and outside it (a count
 * only: the kernel takes the true division there).  Usage: fastdiv_check D. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t fb(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static int in_range(uint32_t u) { uint32_t e = (u >> 23) & 0xFF; return e >= 10 && e <= 254; }

int main(int argc, char** argv) {
  const float D = (float)atof(argv[1]);
  const float r = 1.0f / D;
  unsigned long long bad_in = 0, bad_out = 0;
  const int full = argc < 3 || strcmp(argv[2], "bf16") != 0;
#pragma omp parallel for reduction(+ : bad_in, bad_out) schedule(static)
  for (long long hi = 0; hi < (full ? 65536 : 1); ++hi) {
    for (uint32_t lo = 0; lo < 65536; ++lo) {
      uint32_t u = full ? ((uint32_t)hi << 16) | lo : (lo << 16);
      float n = bf(u);
      if (isnan(n)) continue;
      float q = n / D;
      float q0 = n * r;
      float rem = fmaf(-q0, D, n);
      float q1 = fmaf(rem, r, q0);
      if (fb(q1) != fb(q)) {
        if (in_range(u)) bad_in++; else bad_out++;
      }
    }
  }
  printf("D=%g mode=%s bad_in_range=%llu bad_out_of_range=%llu\n", D, full ? "f32" : "bf16", bad_in, bad_out);
  return bad_in != 0;
}
