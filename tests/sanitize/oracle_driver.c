/* Drives the C oracle (oracle/gdn_oracle.c, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer): forward and backward on dense and packed inputs
 * (an empty sequence and one-token chunks included) with 1 and 3 threads, which
 * must agree bit for bit, and argument errors.  Writes the inputs and the forward
 * outputs of the last case to argv[1] (raw float64) for comparison with the
 * regular build. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_fwd(int N, const int64_t* cu, int H, int Dk, int Dv, const double* q, const double* k,
               const double* v, const double* g, const double* beta, const double* S0, double scale,
               double* o, double* S_final, int nthreads);
int oracle_bwd(int N, const int64_t* cu, int H, int Dk, int Dv, const double* q, const double* k,
               const double* v, const double* g, const double* beta, const double* S0, double scale,
               const double* dO, const double* dS_final, double* dq, double* dk, double* dv, double* dg,
               double* dbeta, double* dS0, int nthreads);

static uint64_t rng = 88172645463325252ull;
static double uni(void) { /* xorshift64, uniform in [0, 1) */
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (double)(rng >> 11) / 9007199254740992.0;
}
static double* fill(size_t n, double lo, double hi) {
  double* p = malloc(n * sizeof *p);
  for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * uni();
  return p;
}
static double* zeros(size_t n) { return calloc(n ? n : 1, sizeof(double)); }
static int failures = 0;
#define EXPECT(c) do { if (!(c)) { printf("FAILED line %d: %s\n", __LINE__, #c); ++failures; } } while (0)

static void run_case(int N, const int64_t* cu, int H, int Dk, int Dv, const char* dump) {
  const size_t T = (size_t)cu[N];
  double *q = fill(T * H * Dk, -1, 1), *k = fill(T * H * Dk, -0.3, 0.3), *v = fill(T * H * Dv, -1, 1);
  double *g = fill(T * H, -0.5, 0), *beta = fill(T * H, 0, 1), *S0 = fill((size_t)N * H * Dk * Dv, -0.1, 0.1);
  double *dO = fill(T * H * Dv, -1, 1), *dSf = fill((size_t)N * H * Dk * Dv, -1, 1);
  double* o[2]; double* Sf[2]; double* gr[2][6];
  const size_t gsz[6] = {T * H * Dk, T * H * Dk, T * H * Dv, T * H, T * H, (size_t)N * H * Dk * Dv};
  for (int r = 0; r < 2; ++r) {
    const int nt = r == 0 ? 1 : 3;
    o[r] = zeros(T * H * Dv); Sf[r] = zeros((size_t)N * H * Dk * Dv);
    for (int i = 0; i < 6; ++i) gr[r][i] = zeros(gsz[i]);
    EXPECT(oracle_fwd(N, cu, H, Dk, Dv, q, k, v, g, beta, S0, 0.5, o[r], Sf[r], nt) == 0);
    EXPECT(oracle_bwd(N, cu, H, Dk, Dv, q, k, v, g, beta, S0, 0.5, dO, dSf, gr[r][0], gr[r][1], gr[r][2],
                      gr[r][3], gr[r][4], gr[r][5], nt) == 0);
  }
  EXPECT(memcmp(o[0], o[1], T * H * Dv * sizeof(double)) == 0);
  EXPECT(memcmp(Sf[0], Sf[1], (size_t)N * H * Dk * Dv * sizeof(double)) == 0);
  for (int i = 0; i < 6; ++i) EXPECT(memcmp(gr[0][i], gr[1][i], gsz[i] * sizeof(double)) == 0);
  for (size_t i = 0; i < T * H * Dv; ++i) EXPECT(isfinite(o[0][i]));
  if (dump) {
    FILE* f = fopen(dump, "wb");
    EXPECT(f != NULL);
    if (f) {
      fwrite(q, sizeof(double), T * H * Dk, f);
      fwrite(k, sizeof(double), T * H * Dk, f);
      fwrite(v, sizeof(double), T * H * Dv, f);
      fwrite(g, sizeof(double), T * H, f);
      fwrite(beta, sizeof(double), T * H, f);
      fwrite(S0, sizeof(double), (size_t)N * H * Dk * Dv, f);
      fwrite(o[0], sizeof(double), T * H * Dv, f);
      fwrite(Sf[0], sizeof(double), (size_t)N * H * Dk * Dv, f);
      fclose(f);
    }
  }
  free(q); free(k); free(v); free(g); free(beta); free(S0); free(dO); free(dSf);
  for (int r = 0; r < 2; ++r) {
    free(o[r]); free(Sf[r]);
    for (int i = 0; i < 6; ++i) free(gr[r][i]);
  }
}

int main(int argc, char** argv) {
  const int64_t dense[] = {0, 70, 140};
  const int64_t packed[] = {0, 0, 1, 65, 200};
  run_case(2, dense, 2, 16, 8, NULL);
  run_case(4, packed, 3, 8, 24, NULL);
  const int64_t last[] = {0, 33, 100};
  run_case(2, last, 2, 12, 10, argc > 1 ? argv[1] : NULL);
  /* argument errors */
  const int64_t bad[] = {0, 10, 5};
  double x[64] = {0};
  EXPECT(oracle_fwd(2, bad, 1, 2, 2, x, x, x, x, x, NULL, 1.0, x, NULL, 1) == 2);
  EXPECT(oracle_fwd(1, dense, 0, 2, 2, x, x, x, x, x, NULL, 1.0, x, NULL, 1) == 2);
  EXPECT(oracle_fwd(0, NULL, 1, 2, 2, NULL, NULL, NULL, NULL, NULL, NULL, 1.0, NULL, NULL, 1) == 0);
  printf("%s: %d failures\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
