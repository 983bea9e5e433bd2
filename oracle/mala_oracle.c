/*
 * CPU oracle for MassAlloc Attention (MALA) and dense softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing here is part of the operator library:
 * only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * load it. It shares no code, header, table or helper with the HIP path.
 *
 * Plain, slow, obviously correct: fp64 arithmetic with libm exp/log, loops in
 * the order the paper states them, OpenMP only across independent blocks.
 *
 * Sources (the paper "MassAlloc Attention: Let Attention Allocate Its Own
 * Compute" and the review "Why exact attention does not need a quadratic
 * matrix"):
 *   - tolerance tau/L_q and L_q = the keys query q sees (causal) / N_k
 *     (decode): Sec. 2.1
 *   - online forward test, Eqs. (1)-(3), descending traversal: Sec. 2.2
 *   - forward procedure: Appendix A, Algorithm 1
 *   - offline backward test, Eq. (4): Sec. 2.2
 *   - backward procedure: Appendix A, Algorithm 2
 *   - split-KV decode: Sec. 2.4 and the decoding part of Appendix A.1
 *   - (m, l, u) merge: the review's "Method/Mechanism" section
 *   - dense attention: Sec. 2.1 (FullAttn), the review's first paragraph of
 *     "Method/Mechanism"
 *
 * Readings where the pages leave a step open:
 *   - the softmax scale is applied to Q.K inside (scores s = scale * <q,k>);
 *   - causal traversal starts at the last key block holding a legal key of the
 *     query block; non-causal starts at the last key block;
 *   - causal with fewer queries than keys (prefill against a cache) aligns the
 *     queries with the last keys: query q sits at position q + N_k - N_q, sees
 *     keys k <= q + N_k - N_q, and L_q = q + N_k - N_q + 1 (the pages define
 *     only N_q = N_k and single-token decode, which both cases reduce to);
 *   - a row constrains a forward tile only if it has a legal key in the tile;
 *   - skip is strict ("<"): a margin of exactly zero retains;
 *   - tau = 0 means log(tau/L) = -inf (never skip); tau = +inf means +inf;
 *   - every valid row of a retained tile is updated (tile-level decision);
 *   - query head h reads KV head h / (Hq/Hkv);
 *   - D = rowsum(O o dO) uses the O handed in (the stored forward output);
 *   - decode splits are ceil(ceil(Nk/Bk)/S) tiles long, each split starts with
 *     fresh (m, l) and keeps L = Nk; empty splits are skipped by the merge.
 *
 * Rounding model (flags): the GPU path feeds bf16 operands to its matrix
 * units. With the corresponding flag set the oracle rounds the same
 * intermediate to bf16 (value -> fp32 RNE -> bf16 RNE) before it is used as a
 * product operand, and rounds outputs to bf16. Everything else stays fp64.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_ROUND_P_FWD 1  /* P~ before the PV product (forward and decode) */
#define ORC_ROUND_P_BWD 2  /* P before the dV product */
#define ORC_ROUND_DS 4     /* dS before the dK and dQ products */
#define ORC_ROUND_OUT 8    /* O, dQ, dK, dV stored as bf16; LSE as fp32 */
#define ORC_ABS 16         /* magnitude mode: every product term a*b is replaced
                              by |a|*|b| (P >= 0 stays P), giving per output
                              element the sum of absolute terms that rounding
                              error bounds scale with */
#define ORC_ABS_D 32       /* backward sensitivity to D: dS replaced by
                              P * sum_d |O||dO| in the dQ / dK sums (|K|, |Q|
                              operands), dV gets no term (it has no D) */
#define ORC_LAZY_REF 64    /* forward model only: the exponentials of a retained
                              tile are taken against a reference maximum that
                              moves only when a tile's row maximum exceeds it by
                              more than 8 log2 units (P <= 2^8), as the kernel
                              forms them; a 128-key tile whose upper 64 keys
                              pass the test alone updates as those 64 keys and
                              then the lower 64, each moving the reference. In
                              exact arithmetic m + log l, and so the test and
                              the result, are the same for either reference;
                              what changes is where P~ is rounded */

typedef struct {
  int32_t batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim;
  int32_t causal;
  int32_t block_q, block_k;
  double tau;
  double scale;
  int32_t round_flags;
} orc_problem;

/* Decision codes written to the per-tile decision arrays. */
#define ORC_ILLEGAL (-1)
#define ORC_SKIP 0
#define ORC_RETAIN 1

/* ------------------------------------------------------------------------ */
/* small helpers                                                             */

static double round_bf16(double x) {
  float f = (float)x; /* RNE to fp32 */
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return (double)f; /* inf / nan */
  u += 0x7fffu + ((u >> 16) & 1u);                        /* RNE to bf16 */
  u &= 0xffff0000u;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double round_f32(double x) { return (double)(float)x; }

/* Position offset of the queries in causal problems: query q sits at key
 * position q + N_k - N_q (0 when N_q = N_k). */
static int64_t causal_offset(const orc_problem* p) {
  return (int64_t)p->seqlen_k - (int64_t)p->seqlen_q;
}

static int legal(const orc_problem* p, int64_t q, int64_t k) {
  if (k < 0 || k >= p->seqlen_k) return 0;
  if (p->causal && k > q + causal_offset(p)) return 0;
  return 1;
}

/* L_q: number of causally visible keys (Sec. 2.1). */
static double visible(const orc_problem* p, int64_t q) {
  return p->causal ? (double)(q + causal_offset(p) + 1) : (double)p->seqlen_k;
}

/* log(tau / L_q), with log 0 = -inf and tau = inf giving +inf. */
static double log_threshold(const orc_problem* p, int64_t q) {
  if (p->tau == 0.0) return -INFINITY;
  if (isinf(p->tau)) return INFINITY;
  return log(p->tau / visible(p, q));
}

/* Inner product in fp64. Four partial sums (lanes i mod 4) only shorten the
 * dependency chain; the order of an fp64 sum of this length is immaterial. */
static double dot(const double* a, const double* b, int n) {
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int i = 0;
  for (; i + 4 <= n; i += 4) {
    s0 += a[i] * b[i];
    s1 += a[i + 1] * b[i + 1];
    s2 += a[i + 2] * b[i + 2];
    s3 += a[i + 3] * b[i + 3];
  }
  for (; i < n; ++i) s0 += a[i] * b[i];
  return (s0 + s1) + (s2 + s3);
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Index of the last key block that holds a legal key for some row of the
 * query block [q0, q1). */
static int64_t last_key_block(const orc_problem* p, int64_t q1) {
  int64_t tc = ceil_div(p->seqlen_k, p->block_k);
  if (!p->causal) return tc - 1;
  int64_t last_key = q1 - 1 + causal_offset(p);
  if (last_key > p->seqlen_k - 1) last_key = p->seqlen_k - 1;
  return last_key / p->block_k;
}

/* ------------------------------------------------------------------------ */
/* Dense attention (the textbook definition; no tiling)                      */

/* O_q = sum_k softmax_k(s_qk) v_k over the visible keys; lse_q = log sum_k
 * exp(s_qk), evaluated with the maximum subtracted. */
int orc_dense_fwd(const orc_problem* p, const double* q, const double* k,
                  const double* v, double* o, double* lse) {
  const int d = p->head_dim, G = p->heads_q / p->heads_kv;
  const int64_t Nq = p->seqlen_q, Nk = p->seqlen_k;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < p->batch; ++b)
    for (int h = 0; h < p->heads_q; ++h) {
      const int g = h / G;
      double* s = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
      for (int64_t qi = 0; qi < Nq; ++qi) {
        const double* qv = q + (((int64_t)b * p->heads_q + h) * Nq + qi) * d;
        double mx = -INFINITY;
        for (int64_t kj = 0; kj < Nk; ++kj) {
          if (!legal(p, qi, kj)) { s[kj] = -INFINITY; continue; }
          s[kj] = p->scale * dot(qv, k + (((int64_t)b * p->heads_kv + g) * Nk + kj) * d, d);
          if (s[kj] > mx) mx = s[kj];
        }
        double z = 0.0;
        for (int64_t kj = 0; kj < Nk; ++kj)
          if (s[kj] > -INFINITY) z += exp(s[kj] - mx);
        const double logz = mx + log(z);
        double* ov = o + (((int64_t)b * p->heads_q + h) * Nq + qi) * d;
        for (int c = 0; c < d; ++c) ov[c] = 0.0;
        for (int64_t kj = 0; kj < Nk; ++kj) {
          if (s[kj] == -INFINITY) continue;
          const double pr = exp(s[kj] - logz);
          const double* vv = v + (((int64_t)b * p->heads_kv + g) * Nk + kj) * d;
          for (int c = 0; c < d; ++c) ov[c] += pr * vv[c];
        }
        if (lse) lse[((int64_t)b * p->heads_q + h) * Nq + qi] = logz;
      }
      free(s);
    }
  return 0;
}

/* Gradients of dense attention. P = softmax(s); dP = dO V^T;
 * dS = P o (dP - rowsum(P o dP)); dQ = scale dS K; dK = scale dS^T Q;
 * dV = P^T dO. dK, dV sum over the query heads sharing a KV head. */
int orc_dense_bwd(const orc_problem* p, const double* q, const double* k,
                  const double* v, const double* dout, double* dq, double* dk,
                  double* dv) {
  const int d = p->head_dim, G = p->heads_q / p->heads_kv;
  const int64_t Nq = p->seqlen_q, Nk = p->seqlen_k;
  memset(dk, 0, sizeof(double) * (size_t)p->batch * p->heads_kv * Nk * d);
  memset(dv, 0, sizeof(double) * (size_t)p->batch * p->heads_kv * Nk * d);
  /* one KV group per task so dK/dV accumulate without races */
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < p->batch; ++b)
    for (int g = 0; g < p->heads_kv; ++g) {
      double* s = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
      double* dp = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
      for (int h = g * G; h < (g + 1) * G; ++h)
        for (int64_t qi = 0; qi < Nq; ++qi) {
          const int64_t row = ((int64_t)b * p->heads_q + h) * Nq + qi;
          const double* qv = q + row * d;
          const double* dov = dout + row * d;
          double mx = -INFINITY;
          for (int64_t kj = 0; kj < Nk; ++kj) {
            if (!legal(p, qi, kj)) { s[kj] = -INFINITY; continue; }
            s[kj] = p->scale * dot(qv, k + (((int64_t)b * p->heads_kv + g) * Nk + kj) * d, d);
            if (s[kj] > mx) mx = s[kj];
          }
          double z = 0.0;
          for (int64_t kj = 0; kj < Nk; ++kj)
            if (s[kj] > -INFINITY) z += exp(s[kj] - mx);
          const double logz = mx + log(z);
          double rs = 0.0; /* rowsum(P o dP) */
          for (int64_t kj = 0; kj < Nk; ++kj) {
            if (s[kj] == -INFINITY) { dp[kj] = 0.0; continue; }
            const double* vv = v + (((int64_t)b * p->heads_kv + g) * Nk + kj) * d;
            dp[kj] = dot(dov, vv, d);
            rs += exp(s[kj] - logz) * dp[kj];
          }
          double* dqv = dq + row * d;
          for (int c = 0; c < d; ++c) dqv[c] = 0.0;
          for (int64_t kj = 0; kj < Nk; ++kj) {
            if (s[kj] == -INFINITY) continue;
            const double pr = exp(s[kj] - logz);
            const double ds = pr * (dp[kj] - rs);
            const int64_t krow = ((int64_t)b * p->heads_kv + g) * Nk + kj;
            const double* kv = k + krow * d;
            for (int c = 0; c < d; ++c) {
              dqv[c] += p->scale * ds * kv[c];
              dk[krow * d + c] += p->scale * ds * qv[c];
              dv[krow * d + c] += pr * dov[c];
            }
          }
        }
      free(s);
      free(dp);
    }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* MALA forward (Algorithm 1; Eqs. 1-3)                                       */

/* Online-softmax update (Sec. 2.2; Algorithm 1) of every valid row by the
 * columns [c0, c1) of a retained tile whose scores are s (bk per row, -inf
 * where not legal): m_new from the row maximum over those columns, the
 * rescale of l and acc, and the exponentials added to l and, times V, to acc. */
static void online_update(const orc_problem* p, const double* s, int bk, const double* vbase,
                          int64_t k0, int64_t nrows, int c0, int c1, double* m, double* l,
                          double* acc) {
  const int d = p->head_dim;
  for (int64_t r = 0; r < nrows; ++r) {
    double mx = -INFINITY;
    for (int c = c0; c < c1; ++c)
      if (s[r * bk + c] > mx) mx = s[r * bk + c];
    double m_new = mx > m[r] ? mx : m[r];
    if (p->round_flags & ORC_LAZY_REF) /* 8 log2 units = 8 ln 2 nats */
      m_new = mx > m[r] + 8.0 * 0.69314718055994530942 ? mx : m[r];
    if (m_new == -INFINITY) continue;
    const double alpha = (m[r] == -INFINITY) ? 0.0 : exp(m[r] - m_new);
    double rowsum = 0.0;
    for (int c = 0; c < d; ++c) acc[r * d + c] *= alpha;
    for (int c = c0; c < c1; ++c) {
      const double sv = s[r * bk + c];
      if (sv == -INFINITY) continue;
      const double pt = exp(sv - m_new);
      rowsum += pt;
      const double pu = (p->round_flags & ORC_ROUND_P_FWD) ? round_bf16(pt) : pt;
      const double* vv = vbase + (k0 + c) * d;
      if (p->round_flags & ORC_ABS)
        for (int e = 0; e < d; ++e) acc[r * d + e] += pu * fabs(vv[e]);
      else
        for (int e = 0; e < d; ++e) acc[r * d + e] += pu * vv[e];
    }
    l[r] = alpha * l[r] + rowsum;
    m[r] = m_new;
  }
}

/* Runs the online rule for one query-row block over key blocks
 * [j_lo, j_hi] visited in descending order and returns the unnormalised
 * running state (m, l, acc) per row, which the forward finalises and the
 * decode merges. Rows are [q0, q1); `nrows` = q1 - q0.
 * dec / mrg (nullable) receive one entry per key block j at index j.
 * force (nullable) overrides the decision of block j when force[j] >= 0. */
static void online_block(const orc_problem* p, const double* q, int64_t q_stride_row,
                         const double* kbase, const double* vbase, int64_t q0, int64_t nrows,
                         int64_t j_lo, int64_t j_hi, const int8_t* force, int8_t* dec,
                         double* mrg, double* m, double* l, double* acc) {
  const int d = p->head_dim, bk = p->block_k;
  const int64_t Nk = p->seqlen_k;
  double* s = (double*)malloc(sizeof(double) * (size_t)nrows * bk);
  double* mt = (double*)malloc(sizeof(double) * (size_t)nrows);
  for (int64_t r = 0; r < nrows; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.0;
    for (int c = 0; c < d; ++c) acc[r * d + c] = 0.0;
  }
  for (int64_t j = j_hi; j >= j_lo; --j) {
    const int64_t k0 = j * bk;
    /* score discovery with the causal mask, then the tile row maxima */
    for (int64_t r = 0; r < nrows; ++r) {
      mt[r] = -INFINITY;
      for (int c = 0; c < bk; ++c) {
        const int64_t kj = k0 + c;
        double sv = -INFINITY;
        if (kj < Nk && legal(p, q0 + r, kj))
          sv = p->scale * dot(q + r * q_stride_row, kbase + kj * d, d);
        s[r * bk + c] = sv;
        if (sv > mt[r]) mt[r] = sv;
      }
    }
    /* the blockwise test of Eq. (3): the tile margin is the largest row
     * margin over rows that have a legal key in the tile */
    int any = 0;
    double tile_margin = -INFINITY;
    for (int64_t r = 0; r < nrows; ++r) {
      if (mt[r] == -INFINITY) continue;
      any = 1;
      double mg;
      if (l[r] == 0.0)
        mg = INFINITY; /* Z = 0: ratio defined as +inf (Sec. 2.2) */
      else
        mg = mt[r] - (m[r] + log(l[r])) - log_threshold(p, q0 + r);
      if (mg > tile_margin) tile_margin = mg;
    }
    if (!any) {
      if (dec) dec[j] = ORC_ILLEGAL;
      if (mrg) mrg[j] = NAN;
      continue;
    }
    int retain = !(tile_margin < 0.0);
    if (force && force[j] >= 0) retain = force[j] == ORC_RETAIN;
    if (dec) dec[j] = retain ? ORC_RETAIN : ORC_SKIP;
    if (mrg) mrg[j] = tile_margin;
    if (!retain) continue; /* m, l, O unchanged */
    /* retained tile: online-softmax update of every valid row. In the
     * lazy-reference model a 128-key tile is formed as the kernel forms it,
     * as two 64-key halves: when the upper half passes the test on its own
     * (against the state before the tile), the halves update in turn, upper
     * first, each moving the reference by its own row maxima; otherwise both
     * are exponentiated against one reference. In exact arithmetic the two
     * orders give the same result (Sec. 2.2); they differ only in where P~
     * is rounded. */
    if ((p->round_flags & ORC_LAZY_REF) && bk == 128) {
      double hi_margin = -INFINITY;
      for (int64_t r = 0; r < nrows; ++r) {
        double mh = -INFINITY;
        for (int c = 64; c < 128; ++c)
          if (s[r * bk + c] > mh) mh = s[r * bk + c];
        if (mh == -INFINITY) continue;
        const double mg = (l[r] == 0.0)
                              ? INFINITY
                              : mh - (m[r] + log(l[r])) - log_threshold(p, q0 + r);
        if (mg > hi_margin) hi_margin = mg;
      }
      if (!(hi_margin < 0.0)) {
        online_update(p, s, bk, vbase, k0, nrows, 64, 128, m, l, acc);
        online_update(p, s, bk, vbase, k0, nrows, 0, 64, m, l, acc);
        continue;
      }
    }
    online_update(p, s, bk, vbase, k0, nrows, 0, bk, m, l, acc);
  }
  free(s);
  free(mt);
}

/* MALA forward. sel (nullable): list of nsel (b, h, i) triples; only those
 * query blocks are computed. dec / mrg (nullable): [B][Hq][Tr][Tc] per-tile
 * decision and tile margin; force (nullable): same shape, entries >= 0 force
 * the decision. Returns 0 on success. */
int orc_mala_fwd(const orc_problem* p, const double* q, const double* k, const double* v,
                 const int8_t* force, double* o, double* lse, int8_t* dec, double* mrg,
                 const int32_t* sel, int64_t nsel) {
  const int d = p->head_dim, G = p->heads_q / p->heads_kv;
  const int64_t Nq = p->seqlen_q, Nk = p->seqlen_k;
  const int64_t Tr = ceil_div(Nq, p->block_q), Tc = ceil_div(Nk, p->block_k);
  const int64_t nblocks = sel ? nsel : (int64_t)p->batch * p->heads_q * Tr;
  if (dec && !sel) memset(dec, ORC_ILLEGAL, (size_t)p->batch * p->heads_q * Tr * Tc);
#pragma omp parallel for schedule(dynamic)
  for (int64_t t = 0; t < nblocks; ++t) {
    int64_t b, h, i;
    if (sel) {
      b = sel[3 * t];
      h = sel[3 * t + 1];
      i = sel[3 * t + 2];
    } else {
      b = t / (p->heads_q * Tr);
      h = (t / Tr) % p->heads_q;
      i = t % Tr;
    }
    const int64_t g = h / G;
    const int64_t q0 = i * p->block_q;
    const int64_t q1 = (q0 + p->block_q < Nq) ? q0 + p->block_q : Nq;
    const int64_t nrows = q1 - q0;
    const int64_t tile_base = ((b * p->heads_q + h) * Tr + i) * Tc;
    double* m = (double*)malloc(sizeof(double) * nrows);
    double* l = (double*)malloc(sizeof(double) * nrows);
    double* acc = (double*)malloc(sizeof(double) * nrows * d);
    if (dec)
      for (int64_t j = 0; j < Tc; ++j) dec[tile_base + j] = ORC_ILLEGAL;
    online_block(p, q + ((b * p->heads_q + h) * Nq + q0) * d, d,
                 k + (b * p->heads_kv + g) * Nk * d, v + (b * p->heads_kv + g) * Nk * d, q0,
                 nrows, 0, last_key_block(p, q1), force ? force + tile_base : NULL,
                 dec ? dec + tile_base : NULL, mrg ? mrg + tile_base : NULL, m, l, acc);
    /* finalisation: O = u / l and LSE = m + log l */
    for (int64_t r = 0; r < nrows; ++r) {
      const int64_t row = (b * p->heads_q + h) * Nq + q0 + r;
      for (int c = 0; c < d; ++c) {
        double x = acc[r * d + c] / l[r];
        if (p->round_flags & ORC_ROUND_OUT) x = round_bf16(x);
        o[row * d + c] = x;
      }
      double z = m[r] + log(l[r]);
      if (p->round_flags & ORC_ROUND_OUT) z = round_f32(z);
      lse[row] = z;
    }
    free(m);
    free(l);
    free(acc);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* MALA backward (Algorithm 2; Eq. 4)                                        */

/* Offline test of Eq. (4) for tile (b, h, i, j): returns the tile margin,
 * the largest s_qk - z_q - log(tau/L_q) over legal entries, or NaN if the
 * tile has no legal entry. */
static double bwd_tile_margin(const orc_problem* p, const double* q, const double* k,
                              const double* lse, int64_t b, int64_t h, int64_t i, int64_t j) {
  const int d = p->head_dim, G = p->heads_q / p->heads_kv;
  const int64_t Nq = p->seqlen_q, Nk = p->seqlen_k, g = h / G;
  double best = NAN;
  for (int64_t qi = i * p->block_q; qi < (i + 1) * p->block_q && qi < Nq; ++qi) {
    const int64_t row = (b * p->heads_q + h) * Nq + qi;
    for (int64_t kj = j * p->block_k; kj < (j + 1) * p->block_k && kj < Nk; ++kj) {
      if (!legal(p, qi, kj)) continue;
      const double sv = p->scale * dot(q + row * d, k + ((b * p->heads_kv + g) * Nk + kj) * d, d);
      const double mg = sv - lse[row] - log_threshold(p, qi);
      if (isnan(best) || mg > best) best = mg;
    }
  }
  return best;
}

/* Contribution of one retained tile (retained per Eq. 4) to dQ rows, or to
 * dK/dV rows. Exactly one of (dq_rows) or (dk_rows, dv_rows) is non-NULL;
 * the pointers address the first row of the tile's query / key block. */
static void bwd_tile_apply(const orc_problem* p, const double* q, const double* k,
                           const double* v, const double* lse, const double* dout,
                           const double* D, const double* Dabs, int64_t b, int64_t h, int64_t i,
                           int64_t j, double* dq_rows, double* dk_rows, double* dv_rows) {
  const int d = p->head_dim, G = p->heads_q / p->heads_kv;
  const int64_t Nq = p->seqlen_q, Nk = p->seqlen_k, g = h / G;
  for (int64_t qi = i * p->block_q; qi < (i + 1) * p->block_q && qi < Nq; ++qi) {
    const int64_t row = (b * p->heads_q + h) * Nq + qi;
    for (int64_t kj = j * p->block_k; kj < (j + 1) * p->block_k && kj < Nk; ++kj) {
      if (!legal(p, qi, kj)) continue;
      const int64_t krow = (b * p->heads_kv + g) * Nk + kj;
      const double sv = p->scale * dot(q + row * d, k + krow * d, d);
      const double pr = exp(sv - lse[row]);                    /* P from the saved LSE */
      const double dp = dot(dout + row * d, v + krow * d, d);  /* dP = dO . v */
      const double ds = pr * (dp - D[row]);                    /* dS = P (dP - D) */
      const double pu = (p->round_flags & ORC_ROUND_P_BWD) ? round_bf16(pr) : pr;
      double du = (p->round_flags & ORC_ROUND_DS) ? round_bf16(ds) : ds;
      const int dsens = (p->round_flags & ORC_ABS_D) != 0;
      const int mag = (p->round_flags & ORC_ABS) != 0 || dsens;
      if (mag) du = dsens ? pr * Dabs[row] : fabs(du);
      if (dq_rows) {
        double* dqr = dq_rows + (qi - i * p->block_q) * d;
        for (int c = 0; c < d; ++c) dqr[c] += du * (mag ? fabs(k[krow * d + c]) : k[krow * d + c]);
      } else {
        double* dkr = dk_rows + (kj - j * p->block_k) * d;
        double* dvr = dv_rows + (kj - j * p->block_k) * d;
        for (int c = 0; c < d; ++c) {
          dkr[c] += du * (mag ? fabs(q[row * d + c]) : q[row * d + c]);
          if (!dsens) dvr[c] += pu * (mag ? fabs(dout[row * d + c]) : dout[row * d + c]);
        }
      }
    }
  }
}

/* MALA backward. o, lse: the forward's stored output and log-normaliser.
 * sel_q (nullable): (b, h, i) triples whose dQ rows are computed;
 * sel_k (nullable): (b, g, j) triples whose dK/dV rows are computed.
 * With both NULL everything is computed. dec / mrg / force: [B][Hq][Tr][Tc]
 * as in the forward. dQ, dK and dV are overwritten on the selected rows. */
int orc_mala_bwd(const orc_problem* p, const double* q, const double* k, const double* v,
                 const double* o, const double* lse, const double* dout, const int8_t* force,
                 double* dq, double* dk, double* dv, int8_t* dec, double* mrg,
                 const int32_t* sel_q, int64_t nsel_q, const int32_t* sel_k, int64_t nsel_k) {
  const int d = p->head_dim, G = p->heads_q / p->heads_kv;
  const int64_t Nq = p->seqlen_q, Nk = p->seqlen_k;
  const int64_t Tr = ceil_div(Nq, p->block_q), Tc = ceil_div(Nk, p->block_k);
  const int all = !sel_q && !sel_k;
  const int64_t nq = sel_q ? nsel_q : (all ? (int64_t)p->batch * p->heads_q * Tr : 0);
  const int64_t nk = sel_k ? nsel_k : (all ? (int64_t)p->batch * p->heads_kv * Tc : 0);
  const int64_t ntiles = (int64_t)p->batch * p->heads_q * Tr * Tc;

  /* D_q = rowsum(O o dO) from the stored O (Algorithm 2) */
  const int64_t nrow = (int64_t)p->batch * p->heads_q * Nq;
  double* D = (double*)malloc(sizeof(double) * (size_t)(nrow > 0 ? nrow : 1));
  double* Dabs = (double*)malloc(sizeof(double) * (size_t)(nrow > 0 ? nrow : 1));
  for (int64_t r = 0; r < nrow; ++r) {
    D[r] = dot(o + r * d, dout + r * d, d);
    double a = 0.0;
    for (int c = 0; c < d; ++c) a += fabs(o[r * d + c] * dout[r * d + c]);
    Dabs[r] = a;
  }

  /* decisions for every tile the selected blocks touch */
  int8_t* dd = dec ? dec : (int8_t*)malloc((size_t)(ntiles > 0 ? ntiles : 1));
  memset(dd, ORC_ILLEGAL, (size_t)ntiles);
#pragma omp parallel for schedule(dynamic)
  for (int64_t t = 0; t < nq; ++t) {
    int64_t b, h, i;
    if (sel_q) { b = sel_q[3 * t]; h = sel_q[3 * t + 1]; i = sel_q[3 * t + 2]; }
    else { b = t / (p->heads_q * Tr); h = (t / Tr) % p->heads_q; i = t % Tr; }
    for (int64_t j = 0; j < Tc; ++j) {
      const int64_t ti = ((b * p->heads_q + h) * Tr + i) * Tc + j;
      const double mg = bwd_tile_margin(p, q, k, lse, b, h, i, j);
      if (isnan(mg)) continue;
      int retain = !(mg < 0.0);
      if (force && force[ti] >= 0) retain = force[ti] == ORC_RETAIN;
      dd[ti] = retain ? ORC_RETAIN : ORC_SKIP;
      if (mrg) mrg[ti] = mg;
    }
  }
  /* (with everything selected the first loop already covered every tile) */
#pragma omp parallel for schedule(dynamic)
  for (int64_t t = 0; t < (all ? 0 : nk); ++t) {
    int64_t b, g, j;
    if (sel_k) { b = sel_k[3 * t]; g = sel_k[3 * t + 1]; j = sel_k[3 * t + 2]; }
    else { b = t / (p->heads_kv * Tc); g = (t / Tc) % p->heads_kv; j = t % Tc; }
    for (int64_t h = g * G; h < (g + 1) * G; ++h)
      for (int64_t i = 0; i < Tr; ++i) {
        const int64_t ti = ((b * p->heads_q + h) * Tr + i) * Tc + j;
        const double mg = bwd_tile_margin(p, q, k, lse, b, h, i, j);
        if (isnan(mg)) continue;
        int retain = !(mg < 0.0);
        if (force && force[ti] >= 0) retain = force[ti] == ORC_RETAIN;
        dd[ti] = retain ? ORC_RETAIN : ORC_SKIP;
        if (mrg) mrg[ti] = mg;
      }
  }

  /* dQ rows, query-major */
#pragma omp parallel for schedule(dynamic)
  for (int64_t t = 0; t < nq; ++t) {
    int64_t b, h, i;
    if (sel_q) { b = sel_q[3 * t]; h = sel_q[3 * t + 1]; i = sel_q[3 * t + 2]; }
    else { b = t / (p->heads_q * Tr); h = (t / Tr) % p->heads_q; i = t % Tr; }
    const int64_t q0 = i * p->block_q;
    const int64_t q1 = (q0 + p->block_q < Nq) ? q0 + p->block_q : Nq;
    double* rows = dq + ((b * p->heads_q + h) * Nq + q0) * d;
    for (int64_t x = 0; x < (q1 - q0) * d; ++x) rows[x] = 0.0;
    for (int64_t j = 0; j < Tc; ++j) {
      const int64_t ti = ((b * p->heads_q + h) * Tr + i) * Tc + j;
      if (dd[ti] == ORC_RETAIN)
        bwd_tile_apply(p, q, k, v, lse, dout, D, Dabs, b, h, i, j, rows, NULL, NULL);
    }
    for (int64_t x = 0; x < (q1 - q0) * d; ++x) {
      rows[x] *= p->scale;
      if (p->round_flags & ORC_ROUND_OUT) rows[x] = round_bf16(rows[x]);
    }
  }
  /* dK / dV rows, key-major, summed over the G query heads of the group */
#pragma omp parallel for schedule(dynamic)
  for (int64_t t = 0; t < nk; ++t) {
    int64_t b, g, j;
    if (sel_k) { b = sel_k[3 * t]; g = sel_k[3 * t + 1]; j = sel_k[3 * t + 2]; }
    else { b = t / (p->heads_kv * Tc); g = (t / Tc) % p->heads_kv; j = t % Tc; }
    const int64_t k0 = j * p->block_k;
    const int64_t k1 = (k0 + p->block_k < Nk) ? k0 + p->block_k : Nk;
    double* krows = dk + ((b * p->heads_kv + g) * Nk + k0) * d;
    double* vrows = dv + ((b * p->heads_kv + g) * Nk + k0) * d;
    for (int64_t x = 0; x < (k1 - k0) * d; ++x) krows[x] = vrows[x] = 0.0;
    for (int64_t h = g * G; h < (g + 1) * G; ++h)
      for (int64_t i = 0; i < Tr; ++i) {
        const int64_t ti = ((b * p->heads_q + h) * Tr + i) * Tc + j;
        if (dd[ti] == ORC_RETAIN)
          bwd_tile_apply(p, q, k, v, lse, dout, D, Dabs, b, h, i, j, NULL, krows, vrows);
      }
    for (int64_t x = 0; x < (k1 - k0) * d; ++x) {
      krows[x] *= p->scale;
      if (p->round_flags & ORC_ROUND_OUT) {
        krows[x] = round_bf16(krows[x]);
        vrows[x] = round_bf16(vrows[x]);
      }
    }
  }
  if (!dec) free(dd);
  free(D);
  free(Dabs);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Merge of (m, l, u) summaries (the review's merge identity)                 */

/* O = u / l and lse = M + log l after bringing every nonempty summary to the
 * common scale M = max m_s. Summaries with l_s = 0 (no retained key) are
 * left out, as the review requires for fully masked blocks. */
int orc_merge(int32_t nsum, int32_t d, const double* m, const double* l, const double* u,
              double* o, double* lse) {
  double M = -INFINITY;
  for (int s = 0; s < nsum; ++s)
    if (l[s] > 0.0 && m[s] > M) M = m[s];
  double lt = 0.0;
  for (int c = 0; c < d; ++c) o[c] = 0.0;
  for (int s = 0; s < nsum; ++s) {
    if (!(l[s] > 0.0)) continue;
    const double w = exp(m[s] - M);
    lt += w * l[s];
    for (int c = 0; c < d; ++c) o[c] += w * u[(int64_t)s * d + c];
  }
  for (int c = 0; c < d; ++c) o[c] /= lt;
  *lse = M + log(lt);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Split-KV decode (Sec. 2.4, Appendix A.1)                                   */

/* One query row per (b, h); q is [B][Hq][d]; k, v are [B][Hkv][Nk][d].
 * The Nk keys are cut into num_splits ranges of ceil(ceil(Nk/Bk)/S) tiles;
 * each range runs the forward rule with fresh state and L = Nk; the partial
 * (m, l, u) are merged. dec / mrg / force: [B][Hq][Tc]. */
int orc_mala_decode(const orc_problem* p, const double* q, const double* k, const double* v,
                    int32_t num_splits, const int8_t* force, double* o, double* lse,
                    int8_t* dec, double* mrg) {
  const int d = p->head_dim, G = p->heads_q / p->heads_kv;
  const int64_t Nk = p->seqlen_k;
  const int64_t Tc = ceil_div(Nk, p->block_k);
  const int64_t per = ceil_div(Tc, num_splits);
  orc_problem pd = *p;
  pd.causal = 0; /* the single query sees all N_k keys: L = N_k */
  pd.seqlen_q = 1;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < p->batch; ++b)
    for (int h = 0; h < p->heads_q; ++h) {
      const int64_t g = h / G;
      const int64_t row = (int64_t)b * p->heads_q + h;
      double* ms = (double*)malloc(sizeof(double) * num_splits);
      double* ls = (double*)malloc(sizeof(double) * num_splits);
      double* us = (double*)malloc(sizeof(double) * (size_t)num_splits * d);
      if (dec)
        for (int64_t j = 0; j < Tc; ++j) dec[row * Tc + j] = ORC_ILLEGAL;
      for (int s = 0; s < num_splits; ++s) {
        const int64_t j_lo = s * per;
        int64_t j_hi = (s + 1) * per - 1;
        if (j_hi > Tc - 1) j_hi = Tc - 1;
        if (j_lo > j_hi) { /* empty split */
          ms[s] = -INFINITY;
          ls[s] = 0.0;
          for (int c = 0; c < d; ++c) us[(int64_t)s * d + c] = 0.0;
          continue;
        }
        online_block(&pd, q + row * d, d, k + ((int64_t)b * p->heads_kv + g) * Nk * d,
                     v + ((int64_t)b * p->heads_kv + g) * Nk * d, 0, 1, j_lo, j_hi,
                     force ? force + row * Tc : NULL, dec ? dec + row * Tc : NULL,
                     mrg ? mrg + row * Tc : NULL, ms + s, ls + s, us + (int64_t)s * d);
      }
      double z;
      orc_merge(num_splits, d, ms, ls, us, o + row * d, &z);
      if (p->round_flags & ORC_ROUND_OUT) {
        for (int c = 0; c < d; ++c) o[row * d + c] = round_bf16(o[row * d + c]);
        z = round_f32(z);
      }
      lse[row] = z;
      free(ms);
      free(ls);
      free(us);
    }
  return 0;
}

/* bf16 rounding exposed for the tests' own rounding of inputs/expectations */
/* Number of OpenMP threads the parallel loops above use (reported with the
 * oracle's timings). */
int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_round_bf16_array(const double* x, double* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = round_bf16(x[i]);
}
