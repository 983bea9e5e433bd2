/*
 * mala.h - C ABI of the MassAlloc Attention (MALA) operator library for
 * AMD Instinct MI355X (gfx950).
 *
 * MALA ("MassAlloc Attention: Let Attention Allocate Its Own Compute") is
 * causal softmax attention that scores every legal
 * Q.K tile but runs the post-score work of a tile only when some valid query
 * row's normalised contribution reaches tau / L_q (Sec. 2.1; L_q = number of
 * keys the query sees). Forward tests against the running online-softmax
 * state (Sec. 2.2, Eqs. 1-3; Appendix A, Algorithm 1); backward tests against
 * the final log-normaliser saved by forward (Sec. 2.2, Eq. 4; Algorithm 2);
 * split-KV decode applies the forward rule per split and merges the partial
 * (m, l, u) (Sec. 2.4; Appendix A.1). A dense FullAttn path built from the
 * same kernels, with the test compiled out, serves as the comparison.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     allocates no memory, never synchronises the device, and enqueues all
 *     work on `stream` (a hipStream_t; NULL is the default stream). Between
 *     calls it keeps only a per-device record of the architecture check and,
 *     for mala_decode_noalloc, of its device array's address.
 *   - Layouts are contiguous row-major:
 *       Q, O, dO, dQ   [batch][heads_q ][seqlen_q][head_dim]  bf16
 *       K, V, dK, dV   [batch][heads_kv][seqlen_k][head_dim]  bf16
 *       LSE            [batch][heads_q ][seqlen_q]            fp32
 *     LSE holds z_q = log Z_R,q, the natural log of the retained normaliser
 *     of the scaled scores (Sec. 2.2, end of "Online Sparse Softmax").
 *   - Alignment: the bf16 tensors (Q, K, V, O, dO, dQ, dK, dV, K/V pages)
 *     and the workspace start on 16-byte boundaries; LSE, block tables and
 *     cache lengths on 4-byte boundaries; stats counters on 8-byte
 *     boundaries. hipMalloc and PyTorch allocations satisfy all of these;
 *     a misaligned pointer returns MALA_ERR_INVALID_ARG.
 *   - Query head h reads KV head h / (heads_q / heads_kv) (grouped-query
 *     attention; heads_q must be a multiple of heads_kv).
 *   - head_dim is 64 or 128. The decision tile is block_q x block_k with
 *     block_q, block_k in {64, 128} (other values: MALA_ERR_UNSUPPORTED);
 *     the kernels compute on 64 x 64 tiles and a larger decision tile
 *     decides its 64 x 64 parts together. Forward and backward must use the same tile
 *     (the nesting of Sec. 2.2 relies on one partition).
 *   - Scores are s = softmax_scale * <q, k> (the paper folds the scale into
 *     Q, Sec. 2.1); pass 1/sqrt(head_dim) for standard attention.
 *   - Every argument is validated before any device call. On an invalid
 *     argument nothing is enqueued and a mala_status code is returned;
 *     mala_status_string() gives its text. Nothing throws across the ABI.
 */
#ifndef MALA_H_
#define MALA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MALA_OK = 0,
  MALA_ERR_INVALID_ARG = 1, /* null or misaligned pointer, bad size, bad tau/scale, ... */
  MALA_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, tile size */
  MALA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  MALA_ERR_DEVICE = 4,      /* no usable HIP device / wrong architecture */
  MALA_ERR_LAUNCH = 5       /* a kernel launch failed */
} mala_status;

typedef struct {
  int32_t batch;     /* >= 1 */
  int32_t heads_q;   /* >= 1, multiple of heads_kv */
  int32_t heads_kv;  /* >= 1 */
  int32_t seqlen_q;  /* >= 1 (1 for decode) */
  int32_t seqlen_k;  /* >= 1 */
  int32_t head_dim;  /* 64 or 128 */
} mala_shape;

typedef struct {
  /* 1: causal. The queries are the last seqlen_q positions of the key
   *    sequence: query q (zero-based) sees keys k <= q + seqlen_k - seqlen_q
   *    and L_q = q + seqlen_k - seqlen_q + 1. seqlen_q == seqlen_k is
   *    equal-length causal training (Sec. 2.1, L_q = q + 1); seqlen_q <
   *    seqlen_k is prefill of a chunk against a cache (this library's reading;
   *    the pages define the equal-length and single-token cases, which it
   *    reduces to); seqlen_q > seqlen_k is rejected (MALA_ERR_UNSUPPORTED);
   * 0: every query sees all seqlen_k keys, L_q = seqlen_k. Ignored by
   *    decode, which always uses L = seqlen_k (Sec. 2.1, decoding). */
  int32_t causal;
  int32_t block_q;     /* decision tile rows: 64 or 128 (decode ignores it) */
  int32_t block_k;     /* decision tile keys: 64 or 128 */
  float tau;           /* tolerance, >= 0; 0 never skips (Sec. 2.3: tau -> 0
                          recovers FullAttn); +inf allowed; NaN / < 0
                          rejected. Ignored by the fullattn_* entry points. */
  float softmax_scale; /* > 0 and finite */
} mala_config;

/* Optional instrumentation for tests and measurement; pass NULL in timed
 * and production calls. With it NULL the operator writes only its outputs.
 *   counters  device uint64[4], accumulated (not cleared) by the call:
 *             [0] legal tiles tested, [1] retained tiles,
 *             [2] retained post-score key slots (valid rows x block_k per
 *                 retained tile: the count of Sec. 2.3 / Eq. 11),
 *             [3] 64-key V tiles loaded from HBM (forward and decode);
 *                 64-row dO tiles loaded by the dK/dV pass (backward: one
 *                 per legal 64 x 64 part of a retained tile).
 *             [0]-[2] count decision tiles (block_q x block_k).
 *   decisions device uint8, one byte per tile, written 1 (retained) or
 *             0 (skipped) for every legal tile the call tests; other bytes
 *             are left untouched. Layout [batch][heads_q][Tr][Tc] for
 *             forward and backward (Tr = ceil(seqlen_q/block_q),
 *             Tc = ceil(seqlen_k/block_k)), [batch][heads_q][Tc] for decode.
 * Either member may be NULL. */
typedef struct {
  unsigned long long* counters;
  uint8_t* decisions;
} mala_stats;

/* MALA forward (Algorithm 1; Eqs. 1-3; the forward part of Appendix A.1).
 * Per (batch, query head, query block), key blocks holding a
 * legal key are visited from the last one (the shifted diagonal when causal) down to
 * block 0. Each tile is scored; it is skipped when every valid query row with
 * a legal key in it has rowmax - m - log l < log(tau / L_q); otherwise V is
 * loaded and every valid row of the block takes the online-softmax update.
 * Writes O (bf16) and LSE (fp32) only. Works for training and prefill.
 * The waves that decide a tile together exchange their votes through LDS
 * with a bounded wait (MALA_WAIT_BOUND as for mala_bwd); if a wait reaches
 * its bound, O and LSE of that workgroup's query blocks are written as NaN
 * (never as a plausible value). */
int mala_fwd(const mala_shape* shape, const mala_config* cfg, const void* q, const void* k,
             const void* v, void* o, float* lse, const mala_stats* stats, void* stream);

/* Dense FullAttn forward from the same kernel with the test compiled out
 * (every legal tile retained). cfg->tau is ignored. */
int fullattn_fwd(const mala_shape* shape, const mala_config* cfg, const void* q, const void* k,
                 const void* v, void* o, float* lse, const mala_stats* stats, void* stream);

/* Bytes of device workspace mala_bwd / fullattn_bwd need: a 256-byte header
 * (int32 status word, see mala_bwd), fp32 row terms per 64-row query block
 * (z = LSE in log2 units, the test threshold and D = rowsum(O o dO); 1 KiB
 * per block), one decision byte per legal tile (when causal, query block i
 * reaches key blocks 0 .. i + (63 + seqlen_k - seqlen_q) / 64), fp32
 * partial dK/dV sums for 4 npair segment slots per (batch, KV head), npair
 * = ceil(seqlen_k / 64) / 2 + 1, each slot holding a pair of 64-key blocks
 * (2 x 2 x 64 x head_dim x 4 bytes: 128 KiB at head_dim 128; the dK/dV pass
 * segments long pairs so that all segments of all pairs fit, whatever the
 * decisions), and int32 tables per (batch, KV head): kept items and the
 * segment entry per key block, the npair key-block pairs of the dK/dV pass
 * with up to 8 work items each, and the work count. Returns 0 for an
 * invalid shape or config. */
size_t mala_bwd_workspace_bytes(const mala_shape* shape, const mala_config* cfg);

/* MALA backward (Algorithm 2; Eq. 4; the backward part of Appendix A.1).
 * A key-major scoring pass recomputes Q.K for every legal tile and skips a
 * tile when every legal entry has s - z_q < log(tau / L_q), with z = the
 * forward's LSE (a tile of 128 rows or keys is kept iff one of its 64 x 64
 * parts is); the decisions are stored in the workspace. A key-major
 * pass over pairs of key blocks then runs, for the kept tiles only,
 * P = exp(s - z), dP = dO V^T, dS = P o (dP - rowsum(O o dO)) and the dV and
 * dK products, and a query-major pass forms dQ over the kept tiles
 * (deterministic: no atomics). o and lse are the forward's outputs. dQ, dK, dV are
 * overwritten (rows without a kept tile get zeros). workspace must hold
 * mala_bwd_workspace_bytes(); its contents on entry are irrelevant.
 * Failure signal: the scoring pass's waves wait on one another with a
 * bound (the environment variable MALA_WAIT_BOUND, read per call, overrides
 * it for tests; 0 makes every wait give up). If a wait reaches its bound,
 * every kernel still runs to completion, dQ, dK and dV are written as NaN
 * everywhere, and the int32 at the start of the workspace reads 1 after the
 * call (0 otherwise). The status code only reports host-side errors. */
int mala_bwd(const mala_shape* shape, const mala_config* cfg, const void* q, const void* k,
             const void* v, const void* o, const float* lse, const void* dout, void* dq,
             void* dk, void* dv, void* workspace, size_t workspace_bytes,
             const mala_stats* stats, void* stream);

/* Dense FullAttn backward from the same kernel, test compiled out. */
int fullattn_bwd(const mala_shape* shape, const mala_config* cfg, const void* q, const void* k,
                 const void* v, const void* o, const float* lse, const void* dout, void* dq,
                 void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 const mala_stats* stats, void* stream);

/* Bytes of device workspace for split-KV decode with num_splits splits
 * (fp32 partial m, l and u per split and query head). 0 if invalid. */
size_t mala_decode_workspace_bytes(const mala_shape* shape, int32_t num_splits);

/* A split count that fills the GPU for this shape (advisory; decisions
 * depend on the split count, so callers comparing runs must fix it). */
int32_t mala_decode_default_splits(const mala_shape* shape);

/* Split-KV MALA decode (Sec. 2.4; the decoding part of Appendix A.1).
 * One new query per sequence: q, o are [batch][heads_q][head_dim], lse is
 * [batch][heads_q]; k_cache, v_cache are [batch][heads_kv][seqlen_k][head_dim]
 * and include the current token (L = seqlen_k, Sec. 2.1). shape->seqlen_q
 * must be 1. The Tc = ceil(seqlen_k/block_k) key tiles are cut into
 * num_splits ranges of ceil(Tc/num_splits) tiles; each range starts with
 * fresh (m, l), visits its tiles last-to-first and tests each head's row
 * against its own partial normaliser; the partial (m, l, u) are merged with
 * the normaliser-aware reduction. Every cached key is scored; a V tile is
 * read only if some query head of the KV group retains it. Decode supports
 * up to 8 query heads per KV head (else MALA_ERR_UNSUPPORTED) and requires
 * 1 <= num_splits <= Tc. */
int mala_decode(const mala_shape* shape, const mala_config* cfg, const void* q,
                const void* k_cache, const void* v_cache, void* o, float* lse,
                int32_t num_splits, void* workspace, size_t workspace_bytes,
                const mala_stats* stats, void* stream);

/* Dense split-KV decode from the same kernels, test compiled out. */
int fullattn_decode(const mala_shape* shape, const mala_config* cfg, const void* q,
                    const void* k_cache, const void* v_cache, void* o, float* lse,
                    int32_t num_splits, void* workspace, size_t workspace_bytes,
                    const mala_stats* stats, void* stream);

/* mala_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Same arguments, kernels and results as mala_decode;
 * the split partials go to a device-resident array of the library instead
 * of a caller workspace: at most 16 MiB (16 << 20 bytes) per GPU, held until
 * the process ends. A call needing more (mala_decode_workspace_bytes() >
 * 16 MiB) returns MALA_ERR_WORKSPACE before any device call. The call
 * allocates nothing (the array's device address is looked up once per
 * device, on the first call with that device current). Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (on different
 * streams, or from different host threads) race and must be serialised by
 * the caller. */
int mala_decode_noalloc(const mala_shape* shape, const mala_config* cfg, const void* q,
                        const void* k_cache, const void* v_cache, void* o, float* lse,
                        int32_t num_splits, const mala_stats* stats, void* stream);

/* Split-KV decode over a paged cache of variable-length sequences (the MALA
 * paper's Sec. 2.4 and the decoding part of its Appendix A.1; the serving
 * layout is this library's). Sequence b holds cache_lens[b] keys (1 <= cache_lens[b] <=
 * shape->seqlen_k) and its own tolerance tau / cache_lens[b] (L = its own
 * cache length, Sec. 2.1). Its keys 64 j .. 64 j + 63 sit in page
 * block_table[b * ceil(seqlen_k / 64) + j] of k_pages / v_pages, each page
 * [heads_kv][64][head_dim] bf16 (pages [num_pages][heads_kv][64][head_dim]).
 * block_table (int32 [batch][ceil(seqlen_k / 64)]) and cache_lens (int32
 * [batch]) are device arrays; only the first ceil(cache_lens[b] / 64) entries
 * of a row are read. Each sequence's ceil(cache_lens[b] / 64) tiles are cut
 * into num_splits ranges as in mala_decode (splits past a short cache are
 * empty). q, o, lse, num_splits, workspace (mala_decode_workspace_bytes) and
 * stats as for mala_decode; shape->seqlen_q must be 1. A cache length or page
 * index out of range is not read from: that sequence's o and lse become NaN,
 * the others are unaffected. Returns MALA_ERR_INVALID_ARG for null tables or
 * num_pages < 1, else as mala_decode. */
int mala_decode_paged(const mala_shape* shape, const mala_config* cfg, const void* q,
                      const void* k_pages, const void* v_pages, const int32_t* block_table,
                      const int32_t* cache_lens, int32_t num_pages, void* o, float* lse,
                      int32_t num_splits, void* workspace, size_t workspace_bytes,
                      const mala_stats* stats, void* stream);

/* Dense split-KV decode over the same paged cache (tau ignored). */
int fullattn_decode_paged(const mala_shape* shape, const mala_config* cfg, const void* q,
                          const void* k_pages, const void* v_pages, const int32_t* block_table,
                          const int32_t* cache_lens, int32_t num_pages, void* o, float* lse,
                          int32_t num_splits, void* workspace, size_t workspace_bytes,
                          const mala_stats* stats, void* stream);

/* Static text for a status code (never NULL). */
const char* mala_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MALA_H_ */
