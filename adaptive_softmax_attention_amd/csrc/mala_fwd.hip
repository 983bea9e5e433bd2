// MALA fused forward ("MassAlloc Attention: Let Attention Allocate Its Own Compute":
// Sec. 2.2 Eqs. 1-3, Appendix A Algorithm 1, and the forward part of
// Appendix A.1) and the dense FullAttn forward
// from the same template with the test compiled out.
//
// Work decomposition (gfx950):
//   * a pair of wave64s owns one 64-row decision block (query block i of
//     head h), 32 rows each, two waves per SIMD; a workgroup of 8 waves holds
//     4 blocks that share K/V tiles: 4 query heads of one KV head (GQA), or
//     2 heads x 2 blocks, or 4 consecutive query blocks of one head;
//   * scores are formed transposed, S^T = K Q^T, on 32x32x16 bf16 MFMA with
//     fp32 accumulation: each lane holds 32 keys of one query column, so
//     the row max and sum need one lane-pair exchange, and P^T is already
//     in the B-operand layout of O^T = V^T P^T;
//   * the two halves of a block agree on the test of Eq. 3 through tagged
//     words in LDS (each publishes its ballot and waits for the other's on
//     the same tile), so the softmax of a tile runs in the iteration that
//     scored it;
//   * K and V tiles are copied asynchronously from global memory straight
//     into LDS rings (global_load_lds, row-major, XOR-swizzled per row);
//     V^T operands are read with the transposing LDS read;
//   * software pipeline over the key blocks, visited from the diagonal down
//     (Sec. 2.2), one barrier per tile: K runs two tiles ahead; a tile's V is
//     requested at the barrier after every block's decision on it is known,
//     and O <- alpha O + P V of that tile runs one iteration later, inside
//     the same basic block as the next tile's softmax so that the products
//     and the exponentials overlap;
//   * exponentials use a reference maximum that moves only on jumps of more
//     than 8 (log2 units), which makes the O rescale rare;
//   * workgroups are issued longest-first (largest query block first);
//   * every wait for a partner's vote is bounded (FwdParams::spin polls): a
//     wave that reaches the bound raises a workgroup flag that ends every
//     other wait, and the workgroup then writes NaN for O and LSE, so a
//     give-up can never pass for a result.
#include "mala_common.h"
#include "mala_internal.h"

namespace mala {
namespace {

struct FwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  int batch, heads_q, heads_kv, nq, nk;
  int causal;
  int off;   // causal: query q sits at key position q + off (off = nk - nq >= 0)
  int cblk;  // causal: query block i reaches key block i + cblk, cblk = (63 + off) / 64
  float c;         // softmax_scale * log2(e): raw score -> log2 units
  float log2_tau;  // log2(tau); -inf for tau = 0, +inf for tau = inf
  int spin;        // bound on each wait for a partner wave's vote (polls)
  int group;       // heads_q / heads_kv
  int hpw, ipw;    // heads x query blocks per workgroup, hpw * ipw = 4
  int n_hg, n_ig;  // head groups per KV head, query-block groups
  int tr, tc;      // query / key tile counts
  int trd, tcd;    // decision tiles (block_q x block_k) along queries / keys
  unsigned long long* counters;
  uint8_t* decisions;
};

// kBQ2 / kBK2: decision tiles of 128 rows / 128 keys (pairs of the 64 x 64
// compute tiles); both false is the 64 x 64 tile.
template <int D, bool kTest, bool kStats, bool kBQ2, bool kBK2>
__global__ __launch_bounds__(512, 1) void fwd_kernel(FwdParams p) {
  constexpr int NDC = D / 16;         // 16-wide reduction chunks over d
  constexpr int NDT = D / 32;         // 32-row subtiles of O^T over d
  constexpr int KCH = D / 8;          // 16-byte chunks per K / V row
  constexpr int NT = 512;             // threads per workgroup (8 waves)
  constexpr int CPT = 64 * KCH / NT;  // async 16-byte copies per thread per tile
  // K ring: current tile + 2 ahead (+ the previous one, whose scores a late
  // 128-key decision forms again)
  constexpr int RK = kBK2 ? 4 : 3;
  constexpr int RV = 2;               // V ring
  constexpr uint32_t kTileBytes = 64 * D * 2;
  // The exponentials are taken against a reference maximum that moves only
  // when a tile's row maximum exceeds it by more than this (log2 units), so
  // P <= 2^8 and the O rescale is rare; m + log2(l) is the same either way.
  constexpr float kLazy = 8.f;

  __shared__ __attribute__((aligned(16))) __bf16 k_ring[RK][64 * D];
  __shared__ __attribute__((aligned(16))) __bf16 v_ring[RV][64 * D];
  // block decisions, a byte per wave, read as one word after the next barrier
  __shared__ __attribute__((aligned(8))) uint8_t vflags[2][8];
  __shared__ int pflags[8];     // row-half ballots, tagged with the tile
  __shared__ int lflags[8];     // 128-key tiles: V of the upper tile requested late
  __shared__ int fstop;         // a wait for a vote reached its bound
  __shared__ int spin_lds;      // the bound (p.spin)

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;

  // ---- work item (longest query-block group first) ----
  const int per_ig = p.batch * p.heads_kv * p.n_hg;
  const int ig = p.n_ig - 1 - (int)(blockIdx.x / per_ig);
  int rem = (int)(blockIdx.x % per_ig);
  const int hg = rem % p.n_hg;
  rem /= p.n_hg;
  const int kvh = rem % p.heads_kv;
  const int b = rem / p.heads_kv;

  const int blk = w >> 1, half = w & 1;  // decision block of the group, row half
  const int h = kvh * p.group + hg * p.hpw + (blk % p.hpw);
  const int i = ig * p.ipw + (blk / p.hpw);
  const bool valid = i < p.tr;
  const int qq = i * 64 + 32 * half + l32;  // the query column this lane holds
  // last key block with a legal key for the block (causal: the block's last
  // row sees up to key 64 i + 63 + off)
  const int jmax = valid ? (p.causal ? min(p.tc - 1, i + p.cblk) : p.tc - 1) : -1;
  const int i_top = min(ig * p.ipw + p.ipw - 1, p.tr - 1);
  const int jtop = p.causal ? min(p.tc - 1, i_top + p.cblk) : p.tc - 1;
  const int vrows = valid ? min(64, p.nq - i * 64) : 0;
  // 128-row decision tiles: the block is paired with query block i ^ 1 of
  // the same head (block pblk of the group, hpw in {1, 2}); the four waves
  // of the pair decide together, over the key tiles either block reaches
  const int pblk = blk ^ p.hpw;
  const int pi = i ^ 1;
  const bool pvalid = kBQ2 && pi < p.tr;
  const int pjmax = pvalid ? (p.causal ? min(p.tc - 1, pi + p.cblk) : p.tc - 1) : -1;
  const int jmax_x = kBQ2 ? max(jmax, pjmax) : jmax;
  const int prows = pvalid ? min(64, p.nq - pi * 64) : 0;
  // the wave that records a decision tile's outcome: the upper block of a
  // 128-row pair (or the lower one when the upper lies past the end)
  const bool recorder = kBQ2 ? ((i & 1) ? valid : (valid && !pvalid)) : valid;

  const size_t qrow0 = (size_t)(b * p.heads_q + h) * p.nq;
  const __bf16* kbase = p.k + (size_t)(b * p.heads_kv + kvh) * p.nk * D;
  const __bf16* vbase = p.v + (size_t)(b * p.heads_kv + kvh) * p.nk * D;

  const bool row_ok = valid && qq < p.nq;
  const float L = p.causal ? (float)(qq + p.off + 1) : (float)p.nk;  // visible keys
  const float thr = p.log2_tau - log2f(L);                    // log2(tau / L_q)
  float mref = -INFINITY, lsum = 0.f;

  // ---- Q^T in registers: B operand of S^T = K Q^T ----
  bf16x8 qr[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) {
    bf16x8 t = bf16x8{};
    if (row_ok) t = *(const bf16x8*)(p.q + (qrow0 + qq) * D + 16 * dc + 8 * hh);
    qr[dc] = t;
  }
  // the Q loads are the only loads the compiler tracks; retire them here so
  // that no wait for them lands inside the pipelined loop
  vmcnt_wait<0>();
  if (tid < 8) pflags[tid] = 0;
  if (tid == 0) {
    fstop = 0;
    spin_lds = p.spin;
  }

  floatx16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;

  // ---- async tile copies (rows past the end re-read the last row; those
  //      keys are masked, so only finite values reach the products) ----
  const uint32_t k_lds = lds_addr(&k_ring[0][0]), v_lds = lds_addr(&v_ring[0][0]);
  auto issue_tile = [&](const __bf16* base, int j, uint32_t slot_lds, bool vtype) {
    const __bf16* tb = base + (size_t)j * 64 * D;  // wave-uniform tile base
    const int last = p.nk - 1 - j * 64;              // last row inside the keys
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      const int s0 = x * NT + w * 64;  // first 16-byte slot of this wave
      const int s = s0 + lane;
      const int row = s / KCH, pc = s % KCH;
      const int sw = vtype ? vswz32<D>(row) : kswz32<D>(row);
      const uint32_t voff = (uint32_t)((min(row, last) * D + ((pc ^ sw) & (KCH - 1)) * 8) * 2);
      async_copy16_sa(tb, voff, slot_lds + (uint32_t)s0 * 16u);
    }
  };

  // ---- the pieces of one pipeline step ----
  // S^T of tile j: subtile kt holds keys 32kt + 8e' + 4hh + r (register
  // 4e' + r) of this lane's query column
  auto score = [&](const __bf16* kt_lds, floatx16 (&s)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
      const int row = 32 * kt + l32;
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        const int ch = ((2 * dc + hh) ^ kswz32<D>(row)) & (KCH - 1);
        const bf16x8 a = *(const bf16x8*)(kt_lds + row * D + ch * 8);
        s[kt] = mfma32x32x16(a, qr[dc], s[kt]);
      }
    }
  };
  // causal / ragged-tail mask of tile j: key offset o = 32kt + 8(e/4) + e%4
  // past 4hh is legal iff o <= lim
  auto mask = [&](floatx16 (&s)[2], int j) {
    int lim = p.nk - 1 - j * 64 - 4 * hh;
    if (p.causal) lim = min(lim, qq + p.off - j * 64 - 4 * hh);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (32 * kt + 8 * (e >> 2) + (e & 3) > lim) s[kt][e] = -INFINITY;
  };
  // tile row maximum (raw units) and this row half's vote under Eq. 3 in
  // log2 units: a row wants the tile unless rowmax*c - m - log2(l) <
  // log2(tau/L); l = 0 counts as +inf
  auto vote = [&](const floatx16 (&s)[2], float& mt) {
    float x = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) x = fmaxf(x, s[kt][e]);
    mt = pair32_max(x);
    if constexpr (kTest) {
      const float mg = mt * p.c - mref - fast_log2(lsum) - thr;
      return wave_any(row_ok && mt != -INFINITY && (lsum == 0.f || !(mg < 0.f)));
    } else {
      return true;
    }
  };
  // online-softmax update of a retained tile for every valid row: the
  // exponentials against the reference maximum, the O rescale factor, the
  // running sum and the bf16 P operand. For key chunk kc = 2kt + c the B
  // operand of O^T = V^T P^T holds keys 16kc + 8(e/4) + 4hh + e%4, i.e.
  // registers 8c .. 8c+7 of subtile kt.
  auto softmax = [&](floatx16 (&s)[2], float mt, float& alpha, bf16x8 (&pb)[4]) {
    const float mtc = mt * p.c;
    const bool mv = mtc > mref + kLazy;
    const float mnew = mv ? mtc : mref;
    const float mu = (mnew == -INFINITY) ? 0.f : mnew;
    alpha = mv ? fast_exp2(mref - mu) : 1.f;
    mref = mnew;
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = fast_exp2(s[kt][e] * p.c - mu);
        s[kt][e] = pv;
        rs += pv;
      }
    lsum = alpha * lsum + pair32_sum(rs);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      bf16x8 t;
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = to_bf16(s[kc >> 1][8 * (kc & 1) + e]);
      pb[kc] = t;
    }
  };
  // the exponentials of a tile against a given reference and its bf16 P
  // operand (as above); returns this lane's part of the row sum
  auto exp_pack = [&](floatx16 (&s)[2], float mu, bf16x8 (&pb)[4]) {
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = fast_exp2(s[kt][e] * p.c - mu);
        s[kt][e] = pv;
        rs += pv;
      }
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      bf16x8 t;
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = to_bf16(s[kc >> 1][8 * (kc & 1) + e]);
      pb[kc] = t;
    }
    return rs;
  };
  // O^T += V^T P^T over one tile; the V^T operand of key chunk kc holds keys
  // 16kc + 4hh + 0..3 and 16kc + 8 + 4hh + 0..3 of column 32dt + l32
  const int g16 = lane >> 4, j16 = lane & 15;
  const int tr_row = 4 * (g16 >> 1) + (j16 >> 2);
  const int tr_col = 16 * (g16 & 1) + 4 * (j16 & 3);
  auto pv = [&](const __bf16* vt, const bf16x8 (&pb)[4]) {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        short4v t[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int row = 16 * kc + 8 * u + tr_row;
          const int col = 32 * dt + tr_col;
          const int ch = ((col >> 3) ^ vswz32<D>(row)) & (KCH - 1);
          t[u] = lds_read_tr4(vt + row * D + ch * 8 + (col & 7));
        }
        oacc[dt] = mfma32x32x16(join_tr(t[0], t[1]), pb[kc], oacc[dt]);
      }
  };

  // ---- software pipeline, one barrier per key tile ----
  // Iteration j scores and tests tile j (the two row halves of a block agree
  // through tagged LDS words, without a barrier), then applies P V of tile
  // j+2 (its V was requested one iteration earlier, once every block's
  // decision on it was published at the barrier) while forming the softmax
  // of tile j. P of tiles j and j+2 share a register set (the products read
  // it before the softmax overwrites it); the sets alternate by tile
  // parity, so the loop body runs twice per trip.
  floatx16 sc[2];
  bf16x8 pA[4], pB[4];
  float mt = -INFINITY, alA = 1.f, alB = 1.f;
  bool pendA = false, pendB = false;  // P V outstanding for the tile in that set
  bool d_last = false;                // this block's decision on tile j+1
  // 128-key decision tiles are the pairs (2 J + 1, 2 J) of key tiles, upper
  // first: the upper tile's group decision, this block's row maximum on it
  // and whether this block has legal keys in it
  bool early = false, s_hi = false;
  float mt_hi = -INFINITY;
  unsigned long long st_legal = 0, st_kept = 0, st_slots = 0, st_vtiles = 0;  // instrumentation

  issue_tile(kbase, jtop, k_lds + (jtop % RK) * kTileBytes, false);
  if (jtop >= 1) issue_tile(kbase, jtop - 1, k_lds + ((jtop - 1) % RK) * kTileBytes, false);

  // publish this wave's vote on tile j tagged with the tile, then OR in the
  // votes of the waves that decide the tile with it: the other row half of
  // the block and, with 128-row tiles, both halves of the paired block. All
  // of them take this path for the same tiles and nothing between the
  // barrier and here waits on another wave, so the waits end. Each wait is
  // also bounded: after p.spin unsuccessful polls (at once when p.spin is 0)
  // the wave gives up and raises fstop, which makes the workgroup write NaN
  // outputs.
  auto exchange = [&](int j, bool mine) {
    const int tag = 2 * (j + 1);
    __hip_atomic_store(&pflags[w], tag | (mine ? 1 : 0), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_WORKGROUP);
    bool any = mine;
    auto take = [&](int x) {
      // poll up to the bound (kept in LDS, so that no register holds it
      // through the kernel)
      int o = 0, left = spin_lds;
      for (; left > 0; --left) {
        o = __hip_atomic_load(&pflags[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if ((o & ~1) == tag) break;
      }
      if (left == 0) {
        __hip_atomic_store(&fstop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        o = 0;
      }
      any = any || (o & 1);
    };
    take(w ^ 1);
    if constexpr (kBQ2) {
      take(2 * pblk);
      take(2 * pblk + 1);
    }
    return any;
  };
  const auto needs_mask = [&](int t) {
    return (p.causal && t * 64 + 63 > i * 64 + p.off) || (t * 64 + 63 >= p.nk);
  };

  // pset / al / pend: the register set of tiles j, j + 2; poth / aloth /
  // pendoth: the other set (tiles j + 1, j - 1)
  auto step = [&](int j, bf16x8 (&pset)[4], float& al, bool& pend, bf16x8 (&poth)[4],
                  float& aloth, bool& pendoth) {
    // K_j and V_{j+2} complete (K_{j-1} may stay in flight); decisions on
    // tile j+1 published
    vmcnt_wait_le(j >= 1 ? CPT : 0);
    lds_barrier();
    const int jn = j + 1;
    int any1 = 0;
    if (jn >= 0 && jn <= jtop) {
      any1 = *(const uint64_t*)vflags[jn & 1] != 0;
      if constexpr (!(kBQ2 || kBK2)) {
        if (kStats && valid && jn <= jmax && half == 0 && lane == 0) {
          ++st_legal;
          if (d_last) {
            ++st_kept;
            st_slots += (unsigned long long)vrows * 64ull;
          }
          if (p.decisions)
            p.decisions[((size_t)(b * p.heads_q + h) * p.tr + i) * p.tc + jn] = d_last ? 1 : 0;
        }
      }
    }
    // V of tile j+1 only if some block retains it; then K two tiles ahead
    if (any1) {
      issue_tile(vbase, jn, v_lds + (jn % RV) * kTileBytes, true);
      if (kStats) ++st_vtiles;
    }
    int anyl = 0;
    if constexpr (kBK2) {
      // an upper tile j+2 kept late (decided at iteration j+1, a lower
      // tile): its V now, and it must land before its P V below
      if (jn >= 0 && jn <= jtop && !(jn & 1)) {
#pragma unroll
        for (int x = 0; x < 8; ++x) anyl |= lflags[x];
      }
      if (anyl) {
        issue_tile(vbase, j + 2, v_lds + ((j + 2) % RV) * kTileBytes, true);
        if (kStats) ++st_vtiles;
      }
    }
    if (j >= 2) issue_tile(kbase, j - 2, k_lds + ((j - 2) % RK) * kTileBytes, false);
    if constexpr (kBK2) {
      if (anyl) {  // the same for every wave: anyl is read after the barrier
        vmcnt_wait_le(j >= 2 ? CPT : 0);
        lds_barrier();
      }
    }

    // scores and decision of tile j
    const bool do_s = j >= 0 && valid && j <= jmax;
    const bool do_x = kBQ2 ? (j >= 0 && j <= jmax_x) : do_s;  // this wave's group decides tile j
    bool dj = false;    // the group keeps tile j
    bool late = false;  // 128 keys, lower tile: the group keeps the pair only now
    if (do_s) {
      score(&k_ring[0][0] + (j % RK) * 64 * D, sc);
      if (needs_mask(j)) mask(sc, j);
    }
    if (do_x) {
      bool mine = false;
      if (do_s) {
        mine = vote(sc, mt);
      } else {
        mt = -INFINITY;
      }
      bool v = true;
      if constexpr (kTest) v = exchange(j, mine);
      if constexpr (kBK2) {
        if (j & 1) {  // upper tile: the pair is kept now iff it passes here
          early = v;
          dj = v;
          mt_hi = mt;
          s_hi = do_s;
        } else {  // lower tile, tested against the same state unless kept early
          dj = early || v;
          late = !early && v && s_hi;
        }
      } else {
        dj = v;
      }
    }
    const bool own = dj && do_s;  // this block's rows take tile j's update
    // every lane stores the same word: no divergent branch needed
    if (j >= 0) vflags[j & 1][w] = own ? 1 : 0;
    d_last = own;
    if constexpr (kBK2) {
      if (j >= 0 && !(j & 1)) {
        lflags[w] = late ? 1 : 0;
        early = false;
        s_hi = false;
      }
    }
    if constexpr (kStats && (kBQ2 || kBK2)) {
      // one wave records each decision tile (of a pair, on its lower tile)
      if (do_x && recorder && half == 0 && lane == 0 && (!kBK2 || !(j & 1))) {
        ++st_legal;
        if (dj) {
          ++st_kept;
          st_slots += (unsigned long long)(vrows + prows) * (kBK2 ? 128ull : 64ull);
        }
        if (p.decisions)
          p.decisions[((size_t)(b * p.heads_q + h) * p.trd + (kBQ2 ? i / 2 : i)) * p.tcd +
                      (kBK2 ? j / 2 : j)] = dj ? 1 : 0;
      }
    }

    // P V of tile j+2 with the softmax of tile j
    const bool pv_old = pend;
    if (pv_old && wave_any(al != 1.f)) {
      // O must be relative to the reference maximum P of tile j+2 was formed with
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] *= al;
    }
    const __bf16* vt = &v_ring[0][0] + ((j + 2) % RV) * 64 * D;
    if constexpr (kBK2) {
      if (late && do_s) {
        // the pair is kept late: one reference maximum for both tiles, the
        // lower tile's P from its scores, the upper tile's scores formed
        // again from its K (still in the ring); the upper tile's P V comes
        // first and carries the rescale
        if (pv_old) pv(vt, pset);
        const float mtc = fmaxf(mt, mt_hi) * p.c;
        const bool mv = mtc > mref + kLazy;
        const float mnew = mv ? mtc : mref;
        const float mu = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = mv ? fast_exp2(mref - mu) : 1.f;
        mref = mnew;
        float rs = exp_pack(sc, mu, pset);
        score(&k_ring[0][0] + ((j + 1) % RK) * 64 * D, sc);
        if (needs_mask(j + 1)) mask(sc, j + 1);
        rs += exp_pack(sc, mu, poth);
        lsum = alpha * lsum + pair32_sum(rs);
        aloth = alpha;
        al = 1.f;
        pendoth = true;
        pend = true;
        return;
      }
    }
    if (pv_old && own) {
      pv(vt, pset);
      softmax(sc, mt, al, pset);
    } else if (pv_old) {
      pv(vt, pset);
    } else if (own) {
      softmax(sc, mt, al, pset);
    }
    pend = own;
  };

  // j runs down to -2 to drain the pipeline
  for (int j = jtop; j >= -2; j -= 2) {
    step(j, pA, alA, pendA, pB, alB, pendB);
    if (j - 1 >= -2) step(j - 1, pB, alB, pendB, pA, alA, pendA);
  }

  if (kStats && p.counters && lane == 0) {
    if (half == 0 && valid) {
      atomicAdd(&p.counters[0], st_legal);
      atomicAdd(&p.counters[1], st_kept);
      atomicAdd(&p.counters[2], st_slots);
    }
    if (w == 0) atomicAdd(&p.counters[3], st_vtiles);
  }
  // ---- finalisation: O = O / l, LSE = m + log l (NaN if a wait gave up;
  //      every wave has passed its last exchange at this barrier) ----
  lds_barrier();
  if (fstop) lsum = NAN;
  if (row_ok) {
    const float inv = 1.f / lsum;
    __bf16* orow = p.o + (qrow0 + qq) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        bf16x4 t;
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = to_bf16(oacc[dt][4 * e4 + r] * inv);
        *(bf16x4*)(orow + 32 * dt + 8 * e4 + 4 * hh) = t;
      }
    if (hh == 0) p.lse[qrow0 + qq] = (mref + log2f(lsum)) * kLn2;
  }
}

}  // namespace

template <int D, bool kTest, bool kStats>
hipError_t launch_ft(const FwdParams& p, int mode, dim3 grid, dim3 block, hipStream_t stream) {
  switch (mode) {
    case 0: hipLaunchKernelGGL((fwd_kernel<D, kTest, kStats, false, false>), grid, block, 0, stream, p); break;
    case 1: hipLaunchKernelGGL((fwd_kernel<D, kTest, kStats, false, true>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((fwd_kernel<D, kTest, kStats, true, false>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((fwd_kernel<D, kTest, kStats, true, true>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_fm(const FwdParams& p, bool test, bool st, int mode, dim3 grid, dim3 block,
                     hipStream_t stream) {
  if (test && st) return launch_ft<D, true, true>(p, mode, grid, block, stream);
  if (test) return launch_ft<D, true, false>(p, mode, grid, block, stream);
  if (st) return launch_ft<D, false, true>(p, mode, grid, block, stream);
  // dense and not instrumented: the decision tile changes nothing
  hipLaunchKernelGGL((fwd_kernel<D, false, false, false, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, bool test, hipStream_t stream) {
  FwdParams p;
  p.q = (const __bf16*)a.q;
  p.k = (const __bf16*)a.k;
  p.v = (const __bf16*)a.v;
  p.o = (__bf16*)a.o;
  p.lse = a.lse;
  p.batch = a.batch;
  p.heads_q = a.heads_q;
  p.heads_kv = a.heads_kv;
  p.nq = a.nq;
  p.nk = a.nk;
  p.causal = a.causal;
  p.off = a.causal ? a.nk - a.nq : 0;
  p.cblk = (63 + p.off) / 64;
  p.c = a.scale * kLog2e;
  p.log2_tau = a.tau == 0.f ? -INFINITY : log2f(a.tau);
  p.spin = a.spin;
  p.group = a.heads_q / a.heads_kv;
  const bool bq2 = a.block_q == 128, bk2 = a.block_k == 128;
  if (p.group % 4 == 0 && !bq2) {
    p.hpw = 4;
    p.ipw = 1;
  } else if (p.group % 2 == 0) {
    p.hpw = 2;
    p.ipw = 2;
  } else {
    p.hpw = 1;
    p.ipw = 4;
  }
  p.tr = (a.nq + 63) / 64;
  p.tc = (a.nk + 63) / 64;
  p.trd = (a.nq + a.block_q - 1) / a.block_q;
  p.tcd = (a.nk + a.block_k - 1) / a.block_k;
  p.n_hg = p.group / p.hpw;
  p.n_ig = (p.tr + p.ipw - 1) / p.ipw;
  p.counters = a.counters;
  p.decisions = a.decisions;
  const long long nblocks = (long long)p.n_ig * p.batch * p.heads_kv * p.n_hg;
  dim3 grid((unsigned)nblocks), block(512);
  // the instrumented variant is a separate instantiation, so the timed
  // kernel carries no counter code; the decision tile matters to the test
  // and to what the instrumentation records
  const bool st = p.counters != nullptr || p.decisions != nullptr;
  const int mode = (test || st) ? (bq2 ? 2 : 0) + (bk2 ? 1 : 0) : 0;
  if (a.head_dim == 128) return launch_fm<128>(p, test, st, mode, grid, block, stream);
  return launch_fm<64>(p, test, st, mode, grid, block, stream);
}

}  // namespace mala
