/* CPU replica of the four-over-six candidate choice made by the HIP kernels,
 * checked against the exact rule on adversarial near-tie blocks and tiles.
 *
 * Exact rule (four-over-six pull request, CuTe DSL kernel Design; the
 * oracle's algorithm): for candidate c in {6, 4} with scale byte
 * e4m3(min(sigma_c, 448)), s_c its value, rho_c = min(1 / (s_c S_dec), FLT_MAX),
 * codes q_i = RTN(|x_i| rho_c), d_i = ((q_i s_c) A) / D (true division),
 * e_i = |x_i - d_i| (MAE) or (x_i - d_i)^2 (MSE), E_c = the element-order sum
 * over a 1x16 block, or for a 16x16 tile the 16 row sums combined by the
 * width-16 tree.  Map-to-4 iff E_4 < E_6.
 *
 * Replica of the kernels' shortcut (every operation one fp32 rounding, fma
 * where the kernel writes one; compiled with -ffp-contract=off):
 *   v_i = |x_i| rho_c, q_i = RTN(v_i), E'_c = sum |v_i - q_i| in element
 *   order (MSE: E' = fma(t, t, E')), W_c = s_c S_dec, Z_c = W_c E'_c
 *   (MSE: (W_c W_c) E'_c; tiles tree-sum E' first).
 *   - the lean test of plain 1x16 blocks: B = fma(a + (Z4 + Z6), 2^-15,
 *     2^-90) for MAE, the 1x16 MSE margin below for MSE, dZ = Z6 - Z4:
 *     map-to-4 iff dZ > B, map-to-6 iff dZ <= -B, else undecided;
 *   - the guarded test (blocks outside the plain class, and 16x16 tiles):
 *     B = k a + 2^-15 (Z4 + Z6) + 2^-90 (k = 2^-15 for 1x16, 2^-11 for
 *     tiles; for MSE tiles k a^2, for MSE 1x16 blocks the 1x16 MSE margin):
 *     map-to-4 iff Z4 + B < Z6, map-to-6 iff Z4 - B >= Z6, else undecided;
 *     range guards as in the kernel.
 *   - the 1x16 MSE margin: fma(a, fma(sqrt(Zs), 2^-16, a 2^-30),
 *     fma(Zs, 2^-15, 2^-90)) with Zs = Z4 + Z6 (correctly rounded sqrtf
 *     here; the kernels' hardware square root is within an ulp of it).
 *   - undecided blocks: the kernel's exact sums, d_i = 2^k fl(fl(mu s A) / D)
 *     for q_i = mu 2^k (mu in {1, 1.5}), and the identical-dequant test.
 *
 * Blocks are driven to the decision boundary: one element (not the block
 * maximum) is moved by bisection over its float32 (or bf16) bit pattern
 * between two values whose exact choices differ, down to adjacent values.
 * Every evaluated block asserts that (a) a decided shortcut agrees with the
 * exact rule, (b) the kernel's exact sums equal the exact rule's sums bit for
 * bit, (c) the identical-dequant test only fires on exact ties.  It also
 * reports the largest (|Z4 - E4| + |Z6 - E6|) / B, the fraction of the margin
 * the rounding actually used.
 *
 * Usage: fos_check <mode> <n_blocks> <seed> [out.bin [A]]
 *   mode: 1x16 | tile; cycles through MAE and MSE, bounds 256 and 448, fp32
 *   and bf16 values.  The amax A is the block's own (a row amax computed in
 *   the pass), a larger row or tensor amax, or a smaller one (outside the
 *   plain class); with the optional A every block uses that one value.
 *   out.bin (optional): the two bracketing blocks of every bisection, each a
 *   record of n fp32 values (16 or 256, row-major), then A, bound, err (1 =
 *   MSE) and bf16 flag as fp32, then the exact pick as int32 (1 = map-to-4),
 *   for the parity tests against the oracle and the GPU.
 * Exit status 0 iff no check failed.  The last line is a summary. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t fb(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static const float kGrid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
static const float kFltMax = 3.40282346638528859812e+38f;
static float E4[127];

static void init_tables(void) {
  for (int c = 0; c < 127; ++c) {
    int e = c >> 3, m = c & 7;
    E4[c] = e ? ldexpf(1.0f + m / 8.0f, e - 7) : (float)m * 0x1p-9f;
  }
}

/* nearest table value, ties to the even index, saturating; v >= 0, not NaN */
static int nearest_even(double v, const float* t, int n) {
  if (v >= t[n - 1]) return n - 1;
  int hi = 0;
  while (hi < n && (double)t[hi] < v) ++hi;
  if (hi == 0) return 0;
  double dl = v - t[hi - 1], dh = (double)t[hi] - v;
  if (dh < dl) return hi;
  if (dl < dh) return hi - 1;
  return (hi % 2 == 0) ? hi : hi - 1;
}
static int e4m3_enc(float s) { return nearest_even((double)s, E4, 127); }
static int e2m1_rtn(float v) { return nearest_even((double)v, kGrid, 8); }

typedef struct {
  int k6, k4;
  float s6, s4, rho6, rho4, W6, W4;
  float S_enc, S_dec, A, D;
} Scales;

static void scales_of(float a, float A, float D, Scales* sc) {
  sc->A = A;
  sc->D = D;
  sc->S_enc = fminf(D / A, kFltMax);
  sc->S_dec = A / D;
  const float sig6 = (a / 6.0f) * sc->S_enc;
  const float sig4 = sig6 * 1.5f;
  sc->k6 = e4m3_enc(fminf(sig6, 448.0f));
  sc->k4 = e4m3_enc(fminf(sig4, 448.0f));
  sc->s6 = E4[sc->k6];
  sc->s4 = E4[sc->k4];
  sc->rho6 = fminf(1.0f / (sc->s6 * sc->S_dec), kFltMax);
  sc->rho4 = fminf(1.0f / (sc->s4 * sc->S_dec), kFltMax);
  sc->W6 = sc->s6 * sc->S_dec;
  sc->W4 = sc->s4 * sc->S_dec;
}

/* one candidate over n elements: exact element-order error (oracle rule),
 * approximate scaled-domain error (kernel), the kernel's exact sums, codes */
typedef struct { float E, Ea, Ek; int code[16]; } Cand;

static void candidate(const float* x, int n, float s, float rho, float A, float D, int mse, Cand* c) {
  const float Q1 = (s * A) / D, Q15 = ((1.5f * s) * A) / D;
  float E = 0.0f, Ea = 0.0f, Ek = 0.0f;
  for (int i = 0; i < n; ++i) {
    const float ax = fabsf(x[i]);
    const float v = ax * rho;
    const int idx = e2m1_rtn(v);
    const float q = kGrid[idx];
    c->code[i] = idx | (signbit(x[i]) ? 8 : 0);
    /* exact rule */
    const float d = ((q * s) * A) / D;
    const float t = ax - d;
    const float e = mse ? t * t : fabsf(t);
    E = (i == 0) ? e : E + e;
    /* kernel shortcut */
    const float ta = v - q;
    Ea = mse ? fmaf(ta, ta, Ea) : Ea + fabsf(ta);
    /* kernel exact sums: d = 2^k fl(fl(mu s A) / D) */
    const uint32_t qb = fb(q);
    const float dk = bf(qb & 0x7F800000u) * ((qb & 0x400000u) ? Q15 : Q1);
    const float tk = ax - dk;
    const float ek = mse ? tk * tk : fabsf(tk);
    Ek = (i == 0) ? ek : Ek + ek;
  }
  c->E = E;
  c->Ea = Ea;
  c->Ek = Ek;
}

static float tree16(const float* g) {
  const float left = ((g[0] + g[8]) + (g[4] + g[12])) + ((g[2] + g[10]) + (g[6] + g[14]));
  const float right = ((g[1] + g[9]) + (g[5] + g[13])) + ((g[3] + g[11]) + (g[7] + g[15]));
  return left + right;
}

/* kernel decisions: 1 map-to-4, 0 map-to-6, -1 undecided, -2 outside guards */
static float mse_margin16(float a, float Zs) {
  return fmaf(a, fmaf(sqrtf(Zs), 0x1p-16f, a * 0x1p-30f), fmaf(Zs, 0x1p-15f, 0x1p-90f));
}

static int lean_pick(int mse, float E6a, float E4a, float W6, float W4, float a, double* ratio_den) {
  const float Z6 = (mse ? W6 * W6 : W6) * E6a;
  const float Z4 = (mse ? W4 * W4 : W4) * E4a;
  const float B = mse ? mse_margin16(a, Z4 + Z6) : fmaf(a + (Z4 + Z6), 0x1p-15f, 0x1p-90f);
  const float dZ = Z6 - Z4;
  *ratio_den = B;
  if (dZ > B) return 1;
  if (dZ <= -B) return 0;
  return -1;
}

static int guarded_pick(int mse, int log2n, float E6a, float E4a, float W6, float W4, float a,
                        double* ratio_den) {
  *ratio_den = 0;
  if (!(W6 >= 0x1p-50f && W4 <= 0x1p50f && a <= 0x1p50f)) return -2;
  if (E6a != E6a || E4a != E4a) return -2;
  const float Z6 = mse ? (W6 * W6) * E6a : W6 * E6a;
  const float Z4 = mse ? (W4 * W4) * E4a : W4 * E4a;
  if (!(Z6 <= kFltMax && Z4 <= kFltMax)) return -2;
  const float kA = log2n == 4 ? 0x1p-15f : 0x1p-11f;
  const float B = (mse && log2n == 4) ? mse_margin16(a, Z4 + Z6)
                                      : kA * (mse ? a * a : a) + 0x1p-15f * (Z4 + Z6) + 0x1p-90f;
  *ratio_den = B;
  if (Z4 + B < Z6) return 1;
  if (Z4 - B >= Z6) return 0;
  return -1;
}

static int same_dequant(const int* c6, const int* c4, int n, float s6, float s4) {
  if (s4 != 1.5f * s6) return 0;
  for (int i = 0; i < n; ++i) {
    const float q6 = kGrid[c6[i] & 7] * ((c6[i] & 8) ? -1.0f : 1.0f);
    const float q4 = kGrid[c4[i] & 7] * ((c4[i] & 8) ? -1.0f : 1.0f);
    if (!(q6 == 1.5f * q4)) return 0;
  }
  return 1;
}

/* ------------------------------------------------------------ statistics */
static long long n_eval, n_fail, n_undec, n_dec, n_same, n_guard_out;
static double worst_ratio;

static void fail(const char* what, const float* x, int n, float A) {
  if (n_fail < 20) {
    fprintf(stderr, "FAIL %s A=%a x=", what, A);
    for (int i = 0; i < n; ++i) fprintf(stderr, " %a", x[i]);
    fprintf(stderr, "\n");
  }
  n_fail++;
}

/* Evaluate one 1x16 block (plain = the kernel's lean class); returns the
 * exact pick (1 = map-to-4). */
static int eval_block(const float* x, float A, float D, int mse, int plain) {
  float a = 0.0f;
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(x[i]));
  Scales sc;
  scales_of(a, A, D, &sc);
  Cand c6, c4;
  candidate(x, 16, sc.s6, sc.rho6, A, D, mse, &c6);
  candidate(x, 16, sc.s4, sc.rho4, A, D, mse, &c4);
  const int exact = c4.E < c6.E;
  n_eval++;
  double B;
  int pick;
  /* the kernels' plain class: row/tensor in range, finite a >= 2^-117, a <= A
   * (the caller's flag), map-to-6 scale not zero */
  const int row_in_range = A <= 0x1p50f && sc.S_dec >= 0x1p-41f && sc.S_dec <= 0x1p41f;
  const int use_lean = plain && row_in_range && a >= 0x1p-117f && sc.k6 != 0;
  if (use_lean) pick = lean_pick(mse, c6.Ea, c4.Ea, sc.W6, sc.W4, a, &B);
  else pick = guarded_pick(mse, 4, c6.Ea, c4.Ea, sc.W6, sc.W4, a, &B);
  if (pick >= 0) {
    n_dec++;
    if (pick != exact) fail("decided pick differs from the exact rule", x, 16, A);
    const double Z6 = (double)((mse ? sc.W6 * sc.W6 : sc.W6) * c6.Ea);
    const double Z4 = (double)((mse ? sc.W4 * sc.W4 : sc.W4) * c4.Ea);
    const double r = (fabs(Z6 - (double)c6.E) + fabs(Z4 - (double)c4.E)) / B;
    if (r > worst_ratio) worst_ratio = r;
  } else if (pick == -1) {
    n_undec++;
    if (fb(c6.Ek) != fb(c6.E) || fb(c4.Ek) != fb(c4.E)) fail("kernel exact sums differ", x, 16, A);
    if (same_dequant(c6.code, c4.code, 16, sc.s6, sc.s4)) {
      n_same++;
      if (fb(c6.E) != fb(c4.E)) fail("identical-dequant test on a non-tie", x, 16, A);
    }
  } else {
    n_guard_out++;
  }
  return exact;
}

static int eval_tile(const float* x, float A, float D, int mse) {
  float a = 0.0f;
  for (int i = 0; i < 256; ++i) a = fmaxf(a, fabsf(x[i]));
  Scales sc;
  scales_of(a, A, D, &sc);
  float e6[16], e4[16], e6a[16], e4a[16], e6k[16], e4k[16];
  int same = sc.s4 == 1.5f * sc.s6;
  for (int r = 0; r < 16; ++r) {
    Cand c6, c4;
    candidate(x + 16 * r, 16, sc.s6, sc.rho6, A, D, mse, &c6);
    candidate(x + 16 * r, 16, sc.s4, sc.rho4, A, D, mse, &c4);
    e6[r] = c6.E; e4[r] = c4.E; e6a[r] = c6.Ea; e4a[r] = c4.Ea; e6k[r] = c6.Ek; e4k[r] = c4.Ek;
    same = same && same_dequant(c6.code, c4.code, 16, sc.s6, sc.s4);
  }
  const float E6 = tree16(e6), E4 = tree16(e4);
  const int exact = E4 < E6;
  n_eval++;
  double B;
  const int pick = guarded_pick(mse, 8, tree16(e6a), tree16(e4a), sc.W6, sc.W4, a, &B);
  if (pick >= 0) {
    n_dec++;
    if (pick != exact) fail("decided tile pick differs from the exact rule", x, 256, A);
    const double Z6 = (double)((mse ? sc.W6 * sc.W6 : sc.W6) * tree16(e6a));
    const double Z4 = (double)((mse ? sc.W4 * sc.W4 : sc.W4) * tree16(e4a));
    const double r = (fabs(Z6 - (double)E6) + fabs(Z4 - (double)E4)) / B;
    if (r > worst_ratio) worst_ratio = r;
  } else if (pick == -1) {
    n_undec++;
    if (fb(tree16(e6k)) != fb(E6) || fb(tree16(e4k)) != fb(E4)) fail("kernel exact tile sums differ", x, 256, A);
    if (same) {
      n_same++;
      if (fb(E6) != fb(E4)) fail("identical-dequant tile test on a non-tie", x, 256, A);
    }
  } else {
    n_guard_out++;
  }
  return exact;
}

/* ------------------------------------------------------------ generation */
static uint64_t rs;
static uint64_t nxt(void) {
  rs += 0x9E3779B97F4A7C15ull;
  uint64_t z = rs;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static double unif(void) { return (nxt() >> 11) * 0x1p-53; }
static double gauss(void) {
  double u = unif(), v = unif();
  if (u < 1e-300) u = 1e-300;
  return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}
static float to_bf16(float f) { /* RNE to bf16, finite inputs */
  uint32_t u = fb(f);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
  return bf(u);
}

/* fill n values of one of several kinds around a random block scale */
static void fill(float* x, int n, int kind, int bf16) {
  const double c = exp(-8.0 + 16.0 * unif());
  for (int i = 0; i < n; ++i) {
    double v;
    switch (kind) {
      case 0: v = gauss() * c; break;                                   /* Gaussian */
      case 1: v = (double)((int)(nxt() % 97) - 48) / 16.0 * c; break;  /* lattice: ties */
      case 2: v = c * kGrid[nxt() % 8] * (nxt() & 1 ? -1 : 1); break;   /* on one grid */
      case 3: v = c * (0.66 + 0.02 * unif()) * (nxt() & 1 ? -1 : 1); break; /* near 4/6 of the max */
      default: {  /* on both candidates' grids: identical dequant values */
        static const float common[4] = {0.0f, 1.5f, 3.0f, 6.0f};
        v = ldexp(1.0, (int)(nxt() % 40) - 20) * common[nxt() % 4] * (nxt() & 1 ? -1 : 1);
      }
    }
    x[i] = (float)v;
    if (bf16) x[i] = to_bf16(x[i]);
  }
  if (kind == 3) x[nxt() % n] = (float)c * 1.0f;
  if (kind == 4) {  /* one power-of-two scale for the block, amax 6 * 2^k */
    const double p2 = ldexp(1.0, (int)(nxt() % 40) - 20);
    for (int i = 0; i < n; ++i) x[i] = (float)(p2 * (double)kGrid[(nxt() % 2) ? 0 : (nxt() % 2 ? 3 : 5)] * (nxt() & 1 ? -1 : 1));
    x[nxt() % n] = (float)(6.0 * p2);
  }
}

static int argmax_abs(const float* x, int n) {
  int j = 0;
  for (int i = 1; i < n; ++i)
    if (fabsf(x[i]) > fabsf(x[j])) j = i;
  return j;
}

/* bisection over the bit pattern of |x[j]| between lo and hi (patterns of
 * non-negative floats, or bf16 patterns << 16) whose exact picks differ */
typedef int (*EvalFn)(const float* x, float A, float D, int mse, int plain);
static int eval_tile_fn(const float* x, float A, float D, int mse, int plain) {
  (void)plain;
  return eval_tile(x, A, D, mse);
}

static FILE* out;

static void record(const float* x, int n, float A, float bound, int mse, int bf16, int exact_pick) {
  if (!out) return;
  float hdr[4] = {A, bound, (float)mse, (float)bf16};
  int32_t p = exact_pick;
  fwrite(x, sizeof(float), n, out);
  fwrite(hdr, sizeof(float), 4, out);
  fwrite(&p, sizeof(p), 1, out);
}

static void bisect(float* x, int n, int j, float A, float D, float bound, int mse, int bf16, int plain,
                   EvalFn ev) {
  const float neg = signbit(x[j]) ? -1.0f : 1.0f;
  const int mx = argmax_abs(x, n);
  const float a = fabsf(x[mx]);
  /* coarse scan of |x_j| over [0, a) for a change of the exact pick */
  int prev = -1;
  float tprev = 0.0f;
  for (int k = 0; k <= 96; ++k) {
    float t = a * (float)k / 97.0f;
    if (bf16) t = to_bf16(t);
    if (t >= a) break;
    x[j] = neg * t;
    const int p = ev(x, A, D, mse, plain);
    if (prev >= 0 && p != prev) {
      uint32_t lo = fb(tprev), hi = fb(t);
      if (bf16) { lo >>= 16; hi >>= 16; }
      int plo = prev;
      while (hi - lo > 1) {
        const uint32_t mid = lo + (hi - lo) / 2;
        x[j] = neg * bf(bf16 ? mid << 16 : mid);
        const int pm = ev(x, A, D, mse, plain);
        if (pm == plo) lo = mid;
        else hi = mid;
      }
      x[j] = neg * bf(bf16 ? lo << 16 : lo);
      record(x, n, A, bound, mse, bf16, ev(x, A, D, mse, plain));
      x[j] = neg * bf(bf16 ? hi << 16 : hi);
      record(x, n, A, bound, mse, bf16, ev(x, A, D, mse, plain));
      return;
    }
    prev = p;
    tprev = t;
  }
}

int main(int argc, char** argv) {
  if (argc < 4) {
    fprintf(stderr, "usage: fos_check 1x16|tile n_blocks seed [out.bin]\n");
    return 2;
  }
  const int tile = strcmp(argv[1], "tile") == 0;
  const long n_blocks = atol(argv[2]);
  rs = strtoull(argv[3], 0, 0);
  if (argc > 4) out = fopen(argv[4], "wb");
  const float fixedA = argc > 5 ? (float)atof(argv[5]) : 0.0f;
  init_tables();
  const int n = tile ? 256 : 16;
  float* x = malloc(sizeof(float) * n);
  for (long b = 0; b < n_blocks; ++b) {
    const int mse = (int)(b & 1);
    const float bound = (b & 2) ? 448.0f : 256.0f;
    const float D = 6.0f * bound;
    const int bf16 = (int)((b >> 2) & 1);
    const int kind = (int)(nxt() % 5);
    fill(x, n, kind, bf16);
    const float a = fabsf(x[argmax_abs(x, n)]);
    if (a == 0.0f) continue;
    /* A: the block's own amax (a row amax computed in the pass), a larger
     * row or tensor amax, or (1x16, outside the plain class) a smaller one */
    float A;
    int plain = 1;
    const int amode = (int)(nxt() % 8);
    if (amode < 3) A = a;
    else if (amode < 7) A = a * (float)exp2(18.0 * unif());
    else { A = a * (float)exp2(-12.0 * unif()); plain = 0; }
    if (fixedA > 0.0f) {
      A = fixedA;
      plain = a <= A;
    }
    if (!(A > 0.0f) || A > 0x1p100f) continue;
    int j = (int)(nxt() % n);
    if (j == argmax_abs(x, n)) j = (j + 1) % n;
    bisect(x, n, j, A, D, bound, mse, bf16, plain, tile ? eval_tile_fn : eval_block);
  }
  if (out) fclose(out);
  printf("%s evals=%lld decided=%lld undecided=%lld same_dequant=%lld outside_guards=%lld "
         "failures=%lld worst_margin_use=%.6f\n",
         tile ? "tile" : "1x16", n_eval, n_dec, n_undec, n_same, n_guard_out, n_fail, worst_ratio);
  free(x);
  return n_fail != 0;
}
