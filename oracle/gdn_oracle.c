/*
 * CPU fp64 oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the package smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The GPU library never links, loads or calls it, and
 * this file shares no code, header, table or helper with the GPU path.
 *
 * What it computes is the plain token-by-token recurrence stated on the page
 * "Research Sprint Day 1 - Verifying the flash-linear-attention Gated DeltaNet
 * kernel on GB10", section "The GDN update" (four steps: forget, read the value
 * currently stored under the key, write the beta-scaled error, read with the
 * query), in double precision, one (sequence, head) at a time:
 *
 *     alpha_t = exp(g_t)                       (log-space decay, page "Research
 *                                               Sprint Day 2 - Rooflines",
 *                                               section "Building some
 *                                               intuition", gates step 5)
 *     S      <- alpha_t * S                    forget
 *     r      =  S^T k_t                        read (v_old)
 *     e      =  beta_t * (v_t - r)             error
 *     S      <- S + k_t e^T                    write
 *     o_t    =  scale * S^T q_t                read after the write
 *
 * S is d_k x d_v (the Day-1 orientation; the closed form on the Day-2 page is
 * its transpose).  `scale` multiplies the output only: the Day-1 update has no
 * query scale, and the cuLA issue page passes D^-0.5 to its kernels as a
 * separate argument.
 *
 * The backward pass is the reverse mode of exactly these steps, taken token by
 * token from the last token to the first (the six gradients dq, dk, dv, dg,
 * dbeta and the initial-state gradient dS0; the Day-1 page measures the first
 * five, "Results" tables).
 *
 * Layout (all row-major, doubles):
 *   q, k : [Ttot, H, Dk]   v, o, dO, dv : [Ttot, H, Dv]   g, beta, dg, dbeta : [Ttot, H]
 *   S0, S_final, dS_final, dS0 : [N, H, Dk, Dv]
 * Sequences are token ranges [cu[n], cu[n+1]) of the packed token axis; a dense
 * batch of B rows of T tokens is the packed case cu = {0, T, 2T, ..., B*T}.
 *
 * Work is spread over POSIX threads by (sequence, head) and, in the forward
 * pass, also by blocks of d_v columns: column j of S only ever mixes with
 * column j of v (k, alpha and beta are shared by all columns), so column blocks
 * are independent.  Threading changes no arithmetic order inside a unit.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int N, H, Dk, Dv, nblk;
  const int64_t* cu;
  const double *q, *k, *v, *g, *beta, *S0, *dO, *dSf;
  double scale;
  double *o, *Sf;
  double *dq, *dk, *dv, *dg, *dbeta, *dS0;
  int64_t units;
  int64_t next; /* shared work counter */
  int status;
} job_t;

static int64_t grab(job_t* J) { return __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED); }

/* ---- forward: one (sequence, head, column block) ---------------------------------- */
static void fwd_unit(job_t* J, int64_t u) {
  const int H = J->H, Dk = J->Dk, Dv = J->Dv;
  const int blk = (int)(u % J->nblk);
  const int h = (int)((u / J->nblk) % H);
  const int n = (int)(u / ((int64_t)J->nblk * H));
  const int cols = (Dv + J->nblk - 1) / J->nblk;
  const int j0 = blk * cols;
  const int j1 = (j0 + cols < Dv) ? j0 + cols : Dv;
  if (j0 >= j1) return;
  const int w = j1 - j0;

  double* S = (double*)malloc(sizeof(double) * (size_t)Dk * w);
  double* r = (double*)malloc(sizeof(double) * (size_t)w);
  if (!S || !r) { J->status = 1; free(S); free(r); return; }

  for (int i = 0; i < Dk; ++i)
    for (int j = 0; j < w; ++j)
      S[(size_t)i * w + j] =
          J->S0 ? J->S0[(((size_t)n * H + h) * Dk + i) * Dv + j0 + j] : 0.0;

  for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t) {
    const double* kt = J->k + ((size_t)t * H + h) * Dk;
    const double* qt = J->q + ((size_t)t * H + h) * Dk;
    const double* vt = J->v + ((size_t)t * H + h) * Dv + j0;
    const double a = exp(J->g[(size_t)t * H + h]);
    const double b = J->beta[(size_t)t * H + h];
    /* forget */
    for (size_t x = 0; x < (size_t)Dk * w; ++x) S[x] *= a;
    /* read what is stored under k_t */
    for (int j = 0; j < w; ++j) r[j] = 0.0;
    for (int i = 0; i < Dk; ++i)
      for (int j = 0; j < w; ++j) r[j] += S[(size_t)i * w + j] * kt[i];
    /* write the beta-scaled error (r becomes e) */
    for (int j = 0; j < w; ++j) r[j] = b * (vt[j] - r[j]);
    for (int i = 0; i < Dk; ++i)
      for (int j = 0; j < w; ++j) S[(size_t)i * w + j] += kt[i] * r[j];
    /* read with the query, after the write */
    double* ot = J->o + ((size_t)t * H + h) * Dv + j0;
    for (int j = 0; j < w; ++j) ot[j] = 0.0;
    for (int i = 0; i < Dk; ++i)
      for (int j = 0; j < w; ++j) ot[j] += S[(size_t)i * w + j] * qt[i];
    for (int j = 0; j < w; ++j) ot[j] *= J->scale;
  }
  if (J->Sf)
    for (int i = 0; i < Dk; ++i)
      for (int j = 0; j < w; ++j)
        J->Sf[(((size_t)n * H + h) * Dk + i) * Dv + j0 + j] = S[(size_t)i * w + j];
  free(S);
  free(r);
}

/* ---- backward: one (sequence, head), reverse mode of the steps above --------------- */
static void bwd_unit(job_t* J, int64_t u) {
  const int H = J->H, Dk = J->Dk, Dv = J->Dv;
  const int h = (int)(u % H);
  const int n = (int)(u / H);
  const int64_t t0 = J->cu[n], L = J->cu[n + 1] - J->cu[n];
  const size_t SZ = (size_t)Dk * Dv;

  /* states S_0 .. S_L of this sequence (S_0 = initial state) */
  double* St = (double*)malloc(sizeof(double) * SZ * (size_t)(L + 1));
  double* dS = (double*)malloc(sizeof(double) * SZ);
  double* Sp = (double*)malloc(sizeof(double) * SZ);
  double* r = (double*)malloc(sizeof(double) * Dv);
  double* e = (double*)malloc(sizeof(double) * Dv);
  double* de = (double*)malloc(sizeof(double) * Dv);
  if (!St || !dS || !Sp || !r || !e || !de) {
    J->status = 1;
    goto out;
  }

  for (size_t x = 0; x < SZ; ++x) St[x] = J->S0 ? J->S0[((size_t)n * H + h) * SZ + x] : 0.0;
  for (int64_t s = 0; s < L; ++s) {
    const int64_t t = t0 + s;
    const double* kt = J->k + ((size_t)t * H + h) * Dk;
    const double* vt = J->v + ((size_t)t * H + h) * Dv;
    const double a = exp(J->g[(size_t)t * H + h]);
    const double b = J->beta[(size_t)t * H + h];
    const double* Sprev = St + (size_t)s * SZ;
    double* Snew = St + (size_t)(s + 1) * SZ;
    for (size_t x = 0; x < SZ; ++x) Snew[x] = a * Sprev[x];
    for (int j = 0; j < Dv; ++j) r[j] = 0.0;
    for (int i = 0; i < Dk; ++i)
      for (int j = 0; j < Dv; ++j) r[j] += Snew[(size_t)i * Dv + j] * kt[i];
    for (int j = 0; j < Dv; ++j) e[j] = b * (vt[j] - r[j]);
    for (int i = 0; i < Dk; ++i)
      for (int j = 0; j < Dv; ++j) Snew[(size_t)i * Dv + j] += kt[i] * e[j];
  }

  for (size_t x = 0; x < SZ; ++x) dS[x] = J->dSf ? J->dSf[((size_t)n * H + h) * SZ + x] : 0.0;

  for (int64_t s = L - 1; s >= 0; --s) {
    const int64_t t = t0 + s;
    const double* kt = J->k + ((size_t)t * H + h) * Dk;
    const double* qt = J->q + ((size_t)t * H + h) * Dk;
    const double* vt = J->v + ((size_t)t * H + h) * Dv;
    const double* dot = J->dO + ((size_t)t * H + h) * Dv;
    const double a = exp(J->g[(size_t)t * H + h]);
    const double b = J->beta[(size_t)t * H + h];
    const double* Sprev = St + (size_t)s * SZ;
    const double* Scur = St + (size_t)(s + 1) * SZ;
    double* dqt = J->dq + ((size_t)t * H + h) * Dk;
    double* dkt = J->dk + ((size_t)t * H + h) * Dk;
    double* dvt = J->dv + ((size_t)t * H + h) * Dv;

    /* recompute the forward quantities of this token */
    for (size_t x = 0; x < SZ; ++x) Sp[x] = a * Sprev[x];
    for (int j = 0; j < Dv; ++j) r[j] = 0.0;
    for (int i = 0; i < Dk; ++i)
      for (int j = 0; j < Dv; ++j) r[j] += Sp[(size_t)i * Dv + j] * kt[i];
    for (int j = 0; j < Dv; ++j) e[j] = b * (vt[j] - r[j]);

    /* o_t = scale * S_t^T q_t */
    for (int i = 0; i < Dk; ++i) {
      double acc = 0.0;
      for (int j = 0; j < Dv; ++j) {
        dS[(size_t)i * Dv + j] += J->scale * qt[i] * dot[j];
        acc += Scur[(size_t)i * Dv + j] * dot[j];
      }
      dqt[i] = J->scale * acc;
    }
    /* S_t = S' + k_t e^T */
    for (int j = 0; j < Dv; ++j) de[j] = 0.0;
    for (int i = 0; i < Dk; ++i) {
      double acc = 0.0;
      for (int j = 0; j < Dv; ++j) {
        acc += dS[(size_t)i * Dv + j] * e[j];
        de[j] += dS[(size_t)i * Dv + j] * kt[i];
      }
      dkt[i] = acc;
    }
    /* e = beta (v - r) */
    double db = 0.0;
    for (int j = 0; j < Dv; ++j) {
      db += de[j] * (vt[j] - r[j]);
      dvt[j] = b * de[j];
      de[j] = -b * de[j]; /* de now holds dr */
    }
    J->dbeta[(size_t)t * H + h] = db;
    /* r = S'^T k_t : dS' = dS + k_t dr^T ; dk_t += S' dr */
    for (int i = 0; i < Dk; ++i) {
      double acc = 0.0;
      for (int j = 0; j < Dv; ++j) {
        dS[(size_t)i * Dv + j] += kt[i] * de[j];
        acc += Sp[(size_t)i * Dv + j] * de[j];
      }
      dkt[i] += acc;
    }
    /* S' = a S_{t-1}, a = exp(g_t) : dg = a <dS', S_{t-1}> ; dS_{t-1} = a dS' */
    double dga = 0.0;
    for (size_t x = 0; x < SZ; ++x) dga += dS[x] * Sprev[x];
    J->dg[(size_t)t * H + h] = a * dga;
    for (size_t x = 0; x < SZ; ++x) dS[x] *= a;
  }
  if (J->dS0)
    for (size_t x = 0; x < SZ; ++x) J->dS0[((size_t)n * H + h) * SZ + x] = dS[x];
out:
  free(St);
  free(dS);
  free(Sp);
  free(r);
  free(e);
  free(de);
}

static void* fwd_worker(void* p) {
  job_t* J = (job_t*)p;
  for (int64_t u; (u = grab(J)) < J->units;) fwd_unit(J, u);
  return NULL;
}
static void* bwd_worker(void* p) {
  job_t* J = (job_t*)p;
  for (int64_t u; (u = grab(J)) < J->units;) bwd_unit(J, u);
  return NULL;
}

static int run(job_t* J, void* (*fn)(void*), int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > J->units) nthreads = (int)(J->units > 0 ? J->units : 1);
  pthread_t th[256];
  int started = 0;
  for (int i = 1; i < nthreads; ++i)
    if (pthread_create(&th[started], NULL, fn, J) == 0) ++started;
  fn(J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  return J->status;
}

static int check_cu(int N, const int64_t* cu) {
  if (N < 0 || (N > 0 && !cu)) return 2;
  if (N > 0 && cu[0] != 0) return 2;
  for (int n = 0; n < N; ++n)
    if (cu[n + 1] < cu[n]) return 2;
  return 0;
}

/* Forward.  Returns 0 on success, 1 on allocation failure, 2 on bad arguments.
 * S0 and S_final may be NULL (zero initial state / final state not wanted). */
int oracle_fwd(int N, const int64_t* cu, int H, int Dk, int Dv, const double* q,
               const double* k, const double* v, const double* g, const double* beta,
               const double* S0, double scale, double* o, double* S_final, int nthreads) {
  if (check_cu(N, cu) || H <= 0 || Dk <= 0 || Dv <= 0) return 2;
  if (N == 0) return 0;
  if (!q || !k || !v || !g || !beta || !o) return 2;
  job_t J;
  memset(&J, 0, sizeof J);
  J.N = N; J.H = H; J.Dk = Dk; J.Dv = Dv; J.cu = cu;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.S0 = S0;
  J.scale = scale; J.o = o; J.Sf = S_final;
  /* split columns only when (sequence, head) units are too few to keep threads busy */
  int64_t nh = (int64_t)N * H;
  int nblk = 1;
  if (nh < 2 * (int64_t)nthreads) {
    nblk = (int)((2 * (int64_t)nthreads + nh - 1) / nh);
    if (nblk > Dv) nblk = Dv;
  }
  J.nblk = nblk;
  J.units = nh * nblk;
  return run(&J, fwd_worker, nthreads);
}

/* Backward.  dS_final may be NULL (zero); dS0 may be NULL (not wanted).
 * All of dq, dk, dv, dg, dbeta are fully overwritten. */
int oracle_bwd(int N, const int64_t* cu, int H, int Dk, int Dv, const double* q,
               const double* k, const double* v, const double* g, const double* beta,
               const double* S0, double scale, const double* dO, const double* dS_final,
               double* dq, double* dk, double* dv, double* dg, double* dbeta, double* dS0,
               int nthreads) {
  if (check_cu(N, cu) || H <= 0 || Dk <= 0 || Dv <= 0) return 2;
  if (N == 0) return 0;
  if (!q || !k || !v || !g || !beta || !dO || !dq || !dk || !dv || !dg || !dbeta) return 2;
  job_t J;
  memset(&J, 0, sizeof J);
  J.N = N; J.H = H; J.Dk = Dk; J.Dv = Dv; J.cu = cu;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.S0 = S0; J.dO = dO; J.dSf = dS_final;
  J.scale = scale;
  J.dq = dq; J.dk = dk; J.dv = dv; J.dg = dg; J.dbeta = dbeta; J.dS0 = dS0;
  J.nblk = 1;
  J.units = (int64_t)N * H;
  return run(&J, bwd_worker, nthreads);
}
