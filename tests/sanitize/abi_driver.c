/* Drives the host-side argument validation of the C ABI (include/mala.h),
 * for a build of the API source with AddressSanitizer and
 * UndefinedBehaviorSanitizer against stub kernel launches and no GPU: every
 * entry point with null, misaligned, out-of-range and extreme arguments,
 * and a seeded sweep of random shapes and configs. Expected status codes
 * are checked where the header fixes them; valid calls end in
 * MALA_ERR_DEVICE (no device). The sanitizers check the rest. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "mala.h"

static int fails = 0;
#define EXPECT(call, want)                                                        \
  do {                                                                            \
    const int got_ = (call);                                                      \
    if (got_ != (want)) {                                                         \
      fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #call, got_, \
              (int)(want));                                                       \
      ++fails;                                                                    \
    }                                                                             \
  } while (0)

static char* const A = (char*)(uintptr_t)0x100000; /* aligned fake device pointers */
static char* const M = (char*)(uintptr_t)0x100001; /* misaligned */

static int fwd(const mala_shape* s, const mala_config* c, void* q) {
  return mala_fwd(s, c, q, A, A, A, (float*)A, NULL, NULL);
}
static int bwd(const mala_shape* s, const mala_config* c, void* ws, size_t wsb) {
  return mala_bwd(s, c, A, A, A, A, (const float*)A, A, A, A, A, ws, wsb, NULL, NULL);
}
static int dec(const mala_shape* s, const mala_config* c, int S, void* ws, size_t wsb) {
  return mala_decode(s, c, A, A, A, A, (float*)A, S, ws, wsb, NULL, NULL);
}

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static int64_t pick(const int64_t* v, int n) {
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return v[rng % (uint64_t)n];
}

int main(void) {
  mala_shape s = {1, 4, 2, 300, 300, 128};
  mala_config c = {1, 64, 64, 1.0f, 0.088f};
  mala_stats st = {(unsigned long long*)A, (uint8_t*)A};
  /* null structs and tensors */
  EXPECT(mala_fwd(NULL, &c, A, A, A, A, (float*)A, NULL, NULL), MALA_ERR_INVALID_ARG);
  EXPECT(mala_fwd(&s, NULL, A, A, A, A, (float*)A, NULL, NULL), MALA_ERR_INVALID_ARG);
  EXPECT(fwd(&s, &c, NULL), MALA_ERR_INVALID_ARG);
  EXPECT(fwd(&s, &c, M), MALA_ERR_INVALID_ARG);
  EXPECT(fwd(&s, &c, A), MALA_ERR_DEVICE);
  EXPECT(fullattn_fwd(&s, &c, A, A, A, A, (float*)A, &st, NULL), MALA_ERR_DEVICE);
  mala_stats bad_st = {(unsigned long long*)(A + 4), NULL};
  EXPECT(mala_fwd(&s, &c, A, A, A, A, (float*)A, &bad_st, NULL), MALA_ERR_INVALID_ARG);
  /* shapes */
  mala_shape t = s;
  t.head_dim = 96; EXPECT(fwd(&t, &c, A), MALA_ERR_UNSUPPORTED);
  t = s; t.heads_q = 3; EXPECT(fwd(&t, &c, A), MALA_ERR_INVALID_ARG);
  t = s; t.seqlen_q = 0; EXPECT(fwd(&t, &c, A), MALA_ERR_INVALID_ARG);
  t = s; t.seqlen_q = (1 << 24) + 1; EXPECT(fwd(&t, &c, A), MALA_ERR_UNSUPPORTED);
  t = s; t.seqlen_q = 400; EXPECT(fwd(&t, &c, A), MALA_ERR_UNSUPPORTED); /* causal, Nq > Nk */
  t = s; t.batch = INT32_MAX; t.heads_q = INT32_MAX; t.heads_kv = 1; t.seqlen_q = t.seqlen_k = 1 << 24;
  EXPECT(fwd(&t, &c, A), MALA_ERR_UNSUPPORTED);
  EXPECT(mala_bwd_workspace_bytes(&t, &c) == 0, 1); /* unsupported shape: no size */
  /* configs */
  mala_config e = c;
  e.causal = 2; EXPECT(fwd(&s, &e, A), MALA_ERR_INVALID_ARG);
  e = c; e.block_q = 32; EXPECT(fwd(&s, &e, A), MALA_ERR_UNSUPPORTED);
  e = c; e.block_k = 0; EXPECT(fwd(&s, &e, A), MALA_ERR_INVALID_ARG);
  e = c; e.softmax_scale = 0.f; EXPECT(fwd(&s, &e, A), MALA_ERR_INVALID_ARG);
  e = c; e.softmax_scale = INFINITY; EXPECT(fwd(&s, &e, A), MALA_ERR_INVALID_ARG);
  e = c; e.softmax_scale = NAN; EXPECT(fwd(&s, &e, A), MALA_ERR_INVALID_ARG);
  e = c; e.tau = NAN; EXPECT(fwd(&s, &e, A), MALA_ERR_INVALID_ARG);
  e = c; e.tau = -1.f; EXPECT(fwd(&s, &e, A), MALA_ERR_INVALID_ARG);
  e = c; e.tau = INFINITY; EXPECT(fwd(&s, &e, A), MALA_ERR_DEVICE);
  e = c; e.tau = NAN;
  EXPECT(fullattn_fwd(&s, &e, A, A, A, A, (float*)A, NULL, NULL), MALA_ERR_DEVICE);
  /* backward workspace */
  const size_t need = mala_bwd_workspace_bytes(&s, &c);
  EXPECT(need > 0, 1);
  EXPECT(bwd(&s, &c, NULL, need), MALA_ERR_WORKSPACE);
  EXPECT(bwd(&s, &c, A, need - 1), MALA_ERR_WORKSPACE);
  EXPECT(bwd(&s, &c, M, need), MALA_ERR_INVALID_ARG);
  EXPECT(bwd(&s, &c, A, need), MALA_ERR_DEVICE);
  EXPECT(fullattn_bwd(&s, &c, A, A, A, A, (const float*)A, A, A, A, A, A, need, NULL, NULL),
         MALA_ERR_DEVICE);
  EXPECT(mala_bwd(&s, &c, A, A, A, A, (const float*)A, A, NULL, A, A, A, need, NULL, NULL),
         MALA_ERR_INVALID_ARG);
  /* decode */
  mala_shape d = {16, 32, 8, 1, 131072, 128};
  const int S = mala_decode_default_splits(&d);
  EXPECT(S >= 1 && S <= 256, 1);
  const size_t dw = mala_decode_workspace_bytes(&d, S);
  EXPECT(dec(&d, &c, S, A, dw), MALA_ERR_DEVICE);
  EXPECT(dec(&d, &c, 0, A, dw), MALA_ERR_INVALID_ARG);
  EXPECT(dec(&d, &c, 3000, A, dw), MALA_ERR_INVALID_ARG);
  EXPECT(dec(&d, &c, S, A, dw - 1), MALA_ERR_WORKSPACE);
  mala_shape d2 = d; d2.seqlen_q = 2; EXPECT(dec(&d2, &c, S, A, dw), MALA_ERR_INVALID_ARG);
  d2 = d; d2.heads_kv = 2; EXPECT(dec(&d2, &c, S, A, mala_decode_workspace_bytes(&d2, S)),
                                  MALA_ERR_UNSUPPORTED);
  EXPECT(mala_decode_paged(&d, &c, A, A, A, NULL, (const int32_t*)A, 10, A, (float*)A, S, A, dw,
                           NULL, NULL), MALA_ERR_INVALID_ARG);
  EXPECT(mala_decode_paged(&d, &c, A, A, A, (const int32_t*)A, (const int32_t*)A, 0, A,
                           (float*)A, S, A, dw, NULL, NULL), MALA_ERR_INVALID_ARG);
  EXPECT(mala_decode_paged(&d, &c, A, A, A, (const int32_t*)(A + 2), (const int32_t*)A, 10, A,
                           (float*)A, S, A, dw, NULL, NULL), MALA_ERR_INVALID_ARG);
  EXPECT(fullattn_decode_paged(&d, &c, A, A, A, (const int32_t*)A, (const int32_t*)A, 10, A,
                               (float*)A, S, A, dw, NULL, NULL), MALA_ERR_DEVICE);
  EXPECT(mala_decode_workspace_bytes(&d, 0) == 0, 1);
  /* the allocation-free decode: its scratch holds at most 16 MiB */
  EXPECT(mala_decode_noalloc(&d, &c, A, A, A, A, (float*)A, S, NULL, NULL), MALA_ERR_DEVICE);
  mala_shape big = {64, 64, 8, 1, 131072, 128};
  EXPECT(mala_decode_noalloc(&big, &c, A, A, A, A, (float*)A, 16, NULL, NULL),
         MALA_ERR_WORKSPACE);
  EXPECT(mala_decode_noalloc(&d, &c, NULL, A, A, A, (float*)A, S, NULL, NULL),
         MALA_ERR_INVALID_ARG);
  EXPECT(mala_decode_noalloc(&d, &c, A, A, A, A, (float*)A, 0, NULL, NULL), MALA_ERR_INVALID_ARG);
  for (int x = -3; x < 12; ++x) EXPECT(mala_status_string(x) != NULL, 1);

  /* seeded sweep: random and extreme sizes; every status must be a code */
  const int64_t dims[] = {-1, 0, 1, 2, 3, 7, 63, 64, 65, 1000, 131072, 1 << 24, (1 << 24) + 1,
                          INT32_MAX, INT32_MIN};
  const int64_t hds[] = {0, 32, 64, 96, 128, -64};
  const int64_t blks[] = {0, 1, 64, 100, 128, 256, -64};
  const float fs[] = {0.f, 1.f, -1.f, 0.25f, 1e30f, INFINITY, NAN};
  int n = 0;
  for (int it = 0; it < 20000; ++it) {
    mala_shape r = {(int32_t)pick(dims, 15), (int32_t)pick(dims, 15), (int32_t)pick(dims, 15),
                    (int32_t)pick(dims, 15), (int32_t)pick(dims, 15), (int32_t)pick(hds, 6)};
    mala_config g = {(int32_t)pick(dims, 4), (int32_t)pick(blks, 7), (int32_t)pick(blks, 7),
                     fs[pick((const int64_t[]){0, 1, 2, 3, 4, 5, 6}, 7)],
                     fs[pick((const int64_t[]){0, 1, 2, 3, 4, 5, 6}, 7)]};
    const size_t wb = mala_bwd_workspace_bytes(&r, &g);
    const int32_t sp = (int32_t)pick(dims, 15);
    const size_t wd = mala_decode_workspace_bytes(&r, sp);
    (void)mala_decode_default_splits(&r);
    const int codes[] = {fwd(&r, &g, A), bwd(&r, &g, A, wb ? wb : 1),
                         dec(&r, &g, sp, A, wd ? wd : 1),
                         fullattn_bwd(&r, &g, A, A, A, A, (const float*)A, A, A, A, A, A, wb, NULL,
                                      NULL),
                         mala_decode_noalloc(&r, &g, A, A, A, A, (float*)A, sp, NULL, NULL)};
    for (int x = 0; x < 5; ++x)
      if (codes[x] < MALA_OK || codes[x] > MALA_ERR_LAUNCH) {
        fprintf(stderr, "status %d out of range\n", codes[x]);
        ++fails;
      }
    ++n;
  }
  if (fails) return 1;
  printf("abi driver ok: %d sweep calls\n", n);
  return 0;
}
