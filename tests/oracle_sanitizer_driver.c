/* oracle_sanitizer_driver.c -- runs the C oracle (oracle/ssm_oracle.c, compiled into this
 * program) on small random problems with every buffer allocated at its exact size, so that a
 * sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer, or ThreadSanitizer) reports
 * any out-of-bounds access, undefined operation or data race of the oracle's threaded loops.
 * Also checks that the threaded forward equals the one-thread forward bit for bit.
 * Test infrastructure: built and run by tests/test_oracle_sanitizers.py.  Prints "ok" and
 * exits 0 on success. */
#include "../oracle/ssm_oracle.c"

#include <stdio.h>

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static double uniform(void) {               /* xorshift64*, in [0, 1) */
  g_rng ^= g_rng >> 12; g_rng ^= g_rng << 25; g_rng ^= g_rng >> 27;
  return (double)((g_rng * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}
static float* rnd(int64_t n, double lo, double hi) {
  float* p = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) p[i] = (float)(lo + (hi - lo) * uniform());
  return p;
}
static double* dbuf(int64_t n) { return (double*)calloc((size_t)(n > 0 ? n : 1), sizeof(double)); }

static int finite_all(const double* p, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

/* One forward (threaded and single-threaded) and one backward on a random problem. */
static int run_case(int64_t batch, int64_t L, int64_t D, int64_t N, int ti, int euler, int softplus,
                    int gate, int with_h0) {
  const int64_t tok = batch * L * D, bc = ti ? D * N : batch * L * N, st = batch * D * N;
  float* u = rnd(tok, -1.0, 1.0);
  float* delta = rnd(ti ? D : tok, softplus ? -2.0 : 1e-3, softplus ? 1.0 : 0.1);
  float* A = rnd(D * N, -2.0, -0.1);
  float* B = rnd(bc, -1.0, 1.0);
  float* C = rnd(bc, -1.0, 1.0);
  float* Dskip = rnd(D, 0.5, 1.5);
  float* z = gate ? rnd(tok, -2.0, 2.0) : NULL;
  float* h0 = with_h0 ? rnd(st, -0.5, 0.5) : NULL;
  float* bias = softplus ? rnd(D, -1.0, 0.0) : NULL;
  double* y1 = dbuf(tok);
  double* y3 = dbuf(tok);
  double* last1 = dbuf(st);
  double* last3 = dbuf(st);
  int rc = ssm_oracle_fwd(u, delta, A, B, C, Dskip, z, h0, bias, y1, last1, batch, L, D, N, ti, euler,
                          softplus, 1);
  rc |= ssm_oracle_fwd(u, delta, A, B, C, Dskip, z, h0, bias, y3, last3, batch, L, D, N, ti, euler,
                       softplus, 3);
  if (rc != 0) return 1;
  if (memcmp(y1, y3, sizeof(double) * (size_t)tok) != 0) return 2;
  if (memcmp(last1, last3, sizeof(double) * (size_t)st) != 0) return 3;
  if (!finite_all(y1, tok) || !finite_all(last1, st)) return 4;
  int ret = 0;
  if (!ti) {                                 /* the backward takes selective coefficients here */
    float* dy = rnd(tok, -1.0, 1.0);
    float* dlast = rnd(st, -1.0, 1.0);
    double *du = dbuf(tok), *dd = dbuf(tok), *dA = dbuf(D * N), *dB = dbuf(bc), *dC = dbuf(bc);
    double *dD = dbuf(D), *dz = dbuf(tok), *dbias = dbuf(D), *dh0 = dbuf(st);
    rc = ssm_oracle_bwd(u, delta, A, B, C, Dskip, z, h0, bias, dy, dlast, du, dd, dA, dB, dC, dD, dz,
                        softplus ? dbias : NULL, with_h0 ? dh0 : NULL, batch, L, D, N, 0, euler, softplus);
    if (rc != 0) ret = 5;
    else if (!finite_all(du, tok) || !finite_all(dd, tok) || !finite_all(dA, D * N) || !finite_all(dB, bc) ||
             !finite_all(dC, bc) || !finite_all(dD, D))
      ret = 6;
    free(dy); free(dlast); free(du); free(dd); free(dA); free(dB); free(dC); free(dD); free(dz);
    free(dbias); free(dh0);
  }
  free(u); free(delta); free(A); free(B); free(C); free(Dskip); free(z); free(h0); free(bias);
  free(y1); free(y3); free(last1); free(last3);
  return ret;
}

int main(void) {
  /* shapes: ragged sizes, one state, one channel, several batch rows and threads */
  const int64_t shapes[][4] = {{2, 37, 5, 3}, {1, 64, 4, 4}, {3, 17, 1, 1}, {2, 9, 6, 16}, {1, 1, 3, 2}};
  for (int s = 0; s < (int)(sizeof(shapes) / sizeof(shapes[0])); ++s) {
    for (int variant = 0; variant < 6; ++variant) {
      const int ti = variant == 5, euler = variant == 1, softplus = variant == 2 || variant == 4;
      const int gate = variant != 3, h0 = variant >= 3 && !ti;
      const int r = run_case(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], ti, euler, softplus,
                             gate, h0);
      if (r != 0) {
        printf("case %d variant %d failed: %d\n", s, variant, r);
        return 1;
      }
    }
  }
  /* empty sequence: the state handed back */
  double last[6];
  float h0[6] = {1, 2, 3, 4, 5, 6}, A[6] = {-1, -1, -1, -1, -1, -1};
  if (ssm_oracle_fwd(NULL, NULL, A, NULL, NULL, NULL, NULL, h0, NULL, NULL, last, 1, 0, 2, 3, 0, 0, 0, 2) != 0)
    return 1;
  for (int i = 0; i < 6; ++i)
    if (last[i] != h0[i]) return 1;
  printf("ok\n");
  return 0;
}
