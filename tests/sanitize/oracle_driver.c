/* Exercises every entry point of the CPU oracle (oracle/mala_oracle.c) on
 * small seeded problems, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer: ragged and rectangular shapes, causal and not,
 * GQA, decision tiles of 1 .. 128, every rounding / magnitude flag, forced
 * decisions, selected blocks and split counts. The sanitizers do the
 * checking; the driver only asserts that the outputs it asked for are
 * finite. Test infrastructure: it links the oracle alone. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim;
  int32_t causal;
  int32_t block_q, block_k;
  double tau;
  double scale;
  int32_t round_flags;
} orc_problem;

int orc_dense_fwd(const orc_problem*, const double*, const double*, const double*, double*,
                  double*);
int orc_dense_bwd(const orc_problem*, const double*, const double*, const double*, const double*,
                  double*, double*, double*);
int orc_mala_fwd(const orc_problem*, const double*, const double*, const double*, const int8_t*,
                 double*, double*, int8_t*, double*, const int32_t*, int64_t);
int orc_mala_bwd(const orc_problem*, const double*, const double*, const double*, const double*,
                 const double*, const double*, const int8_t*, double*, double*, double*, int8_t*,
                 double*, const int32_t*, int64_t, const int32_t*, int64_t);
int orc_mala_decode(const orc_problem*, const double*, const double*, const double*, int32_t,
                    const int8_t*, double*, double*, int8_t*, double*);
int orc_merge(int32_t, int32_t, const double*, const double*, const double*, double*, double*);
void orc_round_bf16_array(const double*, double*, int64_t);

static uint64_t rng = 88172645463325252ull;
static double gauss(void) { /* xorshift64 + Box-Muller */
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  const double u1 = ((rng >> 11) + 1.0) / 9007199254740993.0;
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  const double u2 = (rng >> 11) / 9007199254740992.0;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}
static double* randn(int64_t n, double s) {
  double* x = malloc(sizeof(double) * (n ? n : 1));
  for (int64_t i = 0; i < n; ++i) x[i] = s * gauss();
  return x;
}
static void finite(const double* x, int64_t n, const char* what) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) {
      fprintf(stderr, "%s[%lld] = %g\n", what, (long long)i, x[i]);
      exit(2);
    }
}

static void one(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, int bq, int bk,
                double tau, int flags) {
  orc_problem p = {B, Hq, Hkv, Nq, Nk, d, causal, bq, bk, tau, 1.0 / sqrt(d), flags};
  const int64_t nq = (int64_t)B * Hq * Nq * d, nk = (int64_t)B * Hkv * Nk * d;
  const int64_t Tr = (Nq + bq - 1) / bq, Tc = (Nk + bk - 1) / bk;
  const int64_t nt = (int64_t)B * Hq * Tr * Tc;
  double *q = randn(nq, 1.5), *k = randn(nk, 1.5), *v = randn(nk, 1.0), *dout = randn(nq, 1.0);
  double *o = malloc(sizeof(double) * nq), *lse = malloc(sizeof(double) * B * Hq * Nq);
  double *dq = malloc(sizeof(double) * nq), *dk = malloc(sizeof(double) * nk),
         *dv = malloc(sizeof(double) * nk);
  int8_t *dec = malloc(nt), *force = malloc(nt);
  double* mrg = malloc(sizeof(double) * nt);
  /* dense reference */
  orc_dense_fwd(&p, q, k, v, o, lse);
  finite(o, nq, "dense o");
  orc_dense_bwd(&p, q, k, v, dout, dq, dk, dv);
  finite(dq, nq, "dense dq");
  /* MALA forward, free and forced (every other legal tile flipped) */
  orc_mala_fwd(&p, q, k, v, NULL, o, lse, dec, mrg, NULL, 0);
  finite(o, nq, "mala o");
  for (int64_t t = 0; t < nt; ++t) force[t] = dec[t] < 0 ? -1 : (int8_t)((t & 1) ? dec[t] : 1);
  orc_mala_fwd(&p, q, k, v, force, o, lse, dec, mrg, NULL, 0);
  /* selected query blocks only */
  int32_t sel[6] = {0, 0, 0, B - 1, Hq - 1, (int32_t)(Tr - 1)};
  orc_mala_fwd(&p, q, k, v, NULL, o, lse, NULL, NULL, sel, 2);
  /* MALA backward on the forward's outputs: everything, then selections */
  orc_mala_fwd(&p, q, k, v, NULL, o, lse, dec, mrg, NULL, 0);
  orc_mala_bwd(&p, q, k, v, o, lse, dout, NULL, dq, dk, dv, dec, mrg, NULL, 0, NULL, 0);
  finite(dq, nq, "mala dq");
  finite(dk, nk, "mala dk");
  int32_t selk[3] = {B - 1, Hkv - 1, (int32_t)(Tc - 1)};
  orc_mala_bwd(&p, q, k, v, o, lse, dout, force, dq, dk, dv, NULL, NULL, sel, 2, selk, 1);
  free(q); free(k); free(v); free(dout); free(o); free(lse); free(dq); free(dk); free(dv);
  free(dec); free(force); free(mrg);
}

static void decode(int B, int Hq, int Hkv, int Nk, int d, int bk, int S, double tau, int flags) {
  orc_problem p = {B, Hq, Hkv, 1, Nk, d, 0, 1, bk, tau, 1.0 / sqrt(d), flags};
  const int64_t Tc = (Nk + bk - 1) / bk;
  double *q = randn((int64_t)B * Hq * d, 1.5), *k = randn((int64_t)B * Hkv * Nk * d, 1.5),
         *v = randn((int64_t)B * Hkv * Nk * d, 1.0);
  double *o = malloc(sizeof(double) * B * Hq * d), *lse = malloc(sizeof(double) * B * Hq);
  int8_t* dec = malloc((size_t)B * Hq * Tc);
  double* mrg = malloc(sizeof(double) * B * Hq * Tc);
  orc_mala_decode(&p, q, k, v, S, NULL, o, lse, dec, mrg);
  finite(o, (int64_t)B * Hq * d, "decode o");
  free(q); free(k); free(v); free(o); free(lse); free(dec); free(mrg);
}

int main(void) {
  const int flags[] = {0, 1 | 8, 2 | 4 | 8, 2 | 4 | 8 | 16, 32, 8};
  const double taus[] = {0.0, 0.25, 1.0, 4.0, INFINITY};
  int n = 0;
  for (int f = 0; f < 6; ++f)
    for (int t = 0; t < 5; ++t) {
      one(1, 2, 1, 37, 37, 8, 1, 4, 4, taus[t], flags[f]);
      one(2, 3, 3, 20, 20, 4, 1, 1, 2, taus[t], flags[f]);
      one(1, 4, 2, 9, 45, 8, 1, 2, 4, taus[t], flags[f]);   /* chunk against a cache */
      one(1, 2, 2, 30, 70, 8, 0, 8, 16, taus[t], flags[f]);  /* not causal */
      n += 4;
    }
  one(1, 2, 1, 200, 200, 16, 1, 64, 64, 1.0, 0);
  one(1, 2, 1, 130, 300, 16, 1, 128, 128, 1.0, 2 | 4 | 8);
  one(1, 1, 1, 1, 1, 4, 1, 64, 64, 1.0, 0);
  for (int S = 1; S <= 5; ++S) decode(2, 4, 2, 333, 8, 64, S, 1.0, S & 1 ? 0 : 8);
  decode(1, 8, 1, 1000, 16, 128, 3, 0.25, 1);
  /* merge: empty summaries are left out */
  double m[3] = {0.0, -INFINITY, log(2.0)}, l[3] = {2.0, 0.0, 1.0}, u[6] = {2, 2, 0, 0, 4, 4};
  double o2[2], z;
  orc_merge(3, 2, m, l, u, o2, &z);
  if (fabs(o2[0] - 2.5) > 1e-12) return 3;
  double x[5] = {1.0, -3.25, 1e-40, 65504.0, 3.0e38}, y[5];
  orc_round_bf16_array(x, y, 5);
  printf("oracle driver ok: %d problems\n", n + 3);
  return 0;
}
