// Definitions shared by the MALA backward passes (the dK/dV pass is
// compiled in a translation unit of its own, with its own scheduling flag):
// the passes' parameter block, the decision-map indexing and the causal tile
// predicates, and the launcher of the dK/dV pass.
#pragma once

#include "mala_common.h"
#include "mala_internal.h"

namespace mala {

// The dK/dV pass splits a pair's (query block, query head) items into at
// most kSegMax equal segments, one workgroup each, so that a key block that
// every row keeps (an attention sink) does not serialise the pass; the
// segments' fp32 partial sums are added in a fixed order by the finalize
// kernel (deterministic, no atomics). A pair keeping `kept` items gets
// min(kSegMax, ceil(kept / Lseg)) segments with Lseg = max(kSegKept,
// ceil(K / (2 npair))), K = the items all key blocks of the (batch, KV head)
// keep. A pair with more than one segment keeps more than Lseg items, so its
// segment count is below 2 kept / Lseg and all such pairs together hold
// fewer than 2 K / Lseg <= 4 npair segments: the partials need kSlotsPerPair
// = 4 slots per pair, whatever the decisions. (Measured at 128K: 2 slots per
// pair, Lseg twice as long, made the dK/dV pass 1.4 ms slower; 8 or 16 gain
// nothing over 4.)
constexpr int kSegKept = 512;

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const float* lse;
  const __bf16* dout;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  int* status;     // workspace word: 0, or 1 once a bounded wait gave up
  int spin;        // bound on every wait of the scoring pass (polls)
  float* rowinfo;  // [B*Hq*Tr][kRowInfo]
  uint8_t* dmap;   // backward decisions, see dmap_index()
  float* part;     // [B*Hkv][kSlotsPerPair npair][2 blocks][2][64][D] fp32 partial dK, dV
  int batch, heads_q, heads_kv, nq, nk, group;
  int causal;
  int off;   // causal: query q sits at key position q + off (off = nk - nq >= 0)
  int cblk;  // causal: query block i reaches key block i + cblk, cblk = (63 + off) / 64
  float scale;
  float c;         // scale * log2(e): raw score -> log2 units
  float log2_tau;  // log2(tau); -inf for tau = 0, +inf for tau = inf
  int tr, tc;
  long long dmap_per_head;   // bytes of the decision map per (batch, query head)
  int hpw, ipw, n_hg, n_ig;  // query-major grid (as the forward)
  int* kcount;  // [B*Hkv*Tc] kept items per key block (scoring pass)
  int* pairs;   // [B*Hkv][npair][2] key-block pairs of the dK/dV pass; -1 = none
  int* segtab;  // [B*Hkv*Tc] key block's pair: nseg | side << 4 | first slot << 5
  int npair;    // pair slots per (batch, KV head)
  int* work;    // [B*Hkv][wmax] dK/dV work items: pair | seg << 20 | nseg << 24
  int* wcnt;    // [B*Hkv] work items per (batch, KV head)
  int wmax;     // work item slots per (batch, KV head)
  int kq, kk;   // 64-row / 64-key sub-tiles per decision tile (block_q / 64, block_k / 64)
  unsigned long long* counters;
  uint8_t* decisions;
};

// Decision byte of tile (i, j) of (batch, query head) bh.
__device__ __forceinline__ long long dmap_index(const BwdParams& p, int bh, int i, int j) {
  const long long t = p.causal ? causal_row_start(i, p.tc, p.cblk) + j : (long long)i * p.tc + j;
  return (long long)bh * p.dmap_per_head + t;
}

// causal: first query block with a legal key in key block j (its last row
// 64 i + 63 reaches key 64 j: i >= (64 j - off - 63) / 64)
__device__ __forceinline__ int first_qblock(const BwdParams& p, int j) {
  if (!p.causal) return 0;
  const int t = 64 * j - p.off;
  return t > 0 ? min(p.tr - 1, t / 64) : 0;
}
// causal: key block j has a legal key for query block i
__device__ __forceinline__ bool reaches(const BwdParams& p, int i, int j) {
  return !p.causal || j <= i + p.cblk;
}
// causal: tile (i, j) holds a key beyond the limit of some row of block i
__device__ __forceinline__ bool diag_tile(const BwdParams& p, int i, int j) {
  return p.causal && 64 * j + 63 > 64 * i + p.off;
}

// MFMA row R of subtile x holds row 32(x/2) + 8(R/4) + 4(x%2) + R%4 of the
// 64-row tile, so output lane group g4 holds the 8 consecutive rows
// 32(x/2) + 8 g4 + 0..7 across the subtile pair (2kc, 2kc + 1): the outputs
// are then already a reduction-side MFMA operand over those rows.
__device__ __forceinline__ int qperm(int x, int R) {
  return 32 * (x >> 1) + 8 * (R >> 2) + 4 * (x & 1) + (R & 3);
}

// Launch of the dK/dV pass (bwd_kv_kernel, in mala_bwd_kv.hip) with `grid`
// workgroups on `stream`; instantiated for D in {64, 128}.
template <int D, bool kTest, bool kStats>
hipError_t launch_bwd_kv(const BwdParams& p, unsigned grid, hipStream_t stream);

}  // namespace mala
