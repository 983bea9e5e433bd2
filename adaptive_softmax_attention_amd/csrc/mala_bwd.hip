// MALA fused backward ("MassAlloc Attention: Let Attention Allocate Its Own Compute":
// Sec. 2.2 Eq. 4, Appendix A Algorithm 2, and the backward part of
// Appendix A.1) and the dense FullAttn backward from the same templates with
// the test compiled out.
//
// The offline test of Eq. 4 compares every legal score with the forward's
// final log-normaliser, so a tile's decision does not depend on the order in
// which tiles are visited and can be shared between passes. Kernels on the
// caller's stream:
//   1. bwd_pre: per query row, D = rowsum(O o dO) in fp32 from the stored
//      O, z2 = LSE * log2(e), and the test folded into one raw-score
//      threshold W = (z2 + log2(tau / L_q)) / (scale * log2(e)): a legal
//      entry keeps its tile iff s >= W. Written per 64-row block as
//      [z2 x64][W x64][D x64][unused x64] (padded rows: z2 = W = +inf, so
//      they neither pass the test nor contribute, P = 0).
//   2. bwd_score: key-major scoring of every legal tile (S^T = K Q^T on
//      32x32x16 MFMA, max-then-compare test per query column); writes the
//      decision byte map and the kept-item count of every key block. With
//      decision tiles larger than 64 x 64, bwd_coarsen then ORs each tile's
//      64 x 64 parts and recounts the kept items.
//   3. bwd_pair: pairs the key blocks for the dK/dV pass by kept-item count
//      (blocks most items keep, such as an attention sink or a retrieval
//      hub, keep nearly the same items and are paired with each other).
//   4. bwd_kv (mala_bwd_kv.hip): key-major dK/dV over the kept tiles, one
//      pair of key blocks per workgroup: each listed Q/dO tile is copied once
//      for both blocks;
//      long pairs are split into segments whose fp32 partial sums
//      5. bwd_kv_finalize adds in a fixed order (deterministic, no atomics).
//   6. bwd_dq: query-major, shaped like the forward (a wave pair per 64-row
//      block, 4 blocks per workgroup sharing K/V tiles). It reads the byte
//      map, lists the key blocks that some block of the workgroup keeps,
//      and for those recomputes S^T = K Q^T and dP^T = V dO^T, forms
//      dS^T and accumulates dQ^T += K^T dS^T in registers: dQ is written
//      once, in bf16, with no atomics and no fp32 accumulator in memory.
// The dense path fills the decision map with ones instead of scoring and
// pairs blocks 2p, 2p + 1 without segments.
//
// The scoring pass's waves wait on each other through LDS flags. Every wait
// is bounded (BwdParams::spin polls); a wait that reaches the bound ends all
// waits of its workgroup and sets the status word at the start of the
// workspace, and the passes that write dQ, dK and dV then write NaN
// everywhere instead of values, so a give-up can never pass for a result.
#include <type_traits>

#include "mala_bwd.h"

namespace mala {
namespace {

// ---------------------------------------------------------------- pre ----
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int LPR = D / 8;  // lanes per row (8 values each)
  const long long nprow = (long long)p.batch * p.heads_q * p.tr * 64;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long prow = t / LPR;  // row index padded to whole blocks
  const int part = (int)(t % LPR);
  const long long blk = prow / 64;
  const int r = (int)(prow % 64);
  const long long bh = blk / p.tr;
  const int i = (int)(blk % p.tr);
  const int qq = 64 * i + r;
  const bool valid = prow < nprow && qq < p.nq;
  const long long row = bh * p.nq + qq;
  if (t == 0) *p.status = 0;  // no wait has given up (read by the later passes)
  float acc = 0.f;
  if (valid) {
    const bf16x8 a = *(const bf16x8*)(p.o + row * D + 8 * part);
    const bf16x8 b = *(const bf16x8*)(p.dout + row * D + 8 * part);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off);
  if (prow < nprow && part == 0) {
    float* ri = p.rowinfo + blk * kRowInfo;
    if (valid) {
      const float z2 = p.lse[row] * kLog2e;
      const float L = p.causal ? (float)(qq + p.off + 1) : (float)p.nk;  // visible keys
      ri[r] = z2;
      ri[64 + r] = (z2 + p.log2_tau - log2f(L)) / p.c;
      ri[128 + r] = acc;
    } else {
      ri[r] = INFINITY;
      ri[64 + r] = INFINITY;
      ri[128 + r] = 0.f;
    }
  }
}

// -------------------------------------------------------------- score ----
// Offline test of every legal tile (Eq. 4), key-major. A workgroup owns 4 key
// blocks (256 keys) of one KV head and walks every (query block, query head)
// item from the last query block down; every workgroup walks the items in the
// same order, so concurrent workgroups find each Q tile in L2.
//   * Eight compute waves (two per SIMD): wave w holds all 64 keys of block
//     w % 4 as the A operand of S^T = K Q^T (32x32x16 bf16 MFMA, fp32
//     accumulation) and scores every other item (waves 0-3 the even items,
//     waves 4-7 the odd ones), deciding its own tiles with no exchange. A
//     lane holds one query column of 32 keys per subtile: its test is the
//     maximum of those scores against W_q, then one ballot.
//   * One copy wave moves each item's Q tile and thresholds from global
//     memory into an LDS ring with asynchronous copies and publishes the item
//     in the slot's flag once its copies have landed; the compute waves count
//     their completions per slot, and the copy wave refills a slot only after
//     all four of an item's waves are done with it. There is no workgroup
//     barrier in the loop, and the compute waves issue no copies.
//   * The copy wave publishes everything it has issued before it waits, so
//     no wait can be circular. Every wait also has a bound (p.spin polls, by
//     default far beyond any legal schedule); a wait that reaches it raises a
//     workgroup flag that ends every other wait, so that every wave exits
//     whatever happens, and sets the status word, which makes the later
//     passes write NaN gradients.
// Decisions go straight to the byte map read by the dK/dV and dQ passes; the
// kept-item count of every key block goes to the pairing pass.
template <int D, bool kTest, bool kStats>
__global__ __launch_bounds__(576, 1) void bwd_score_kernel(BwdParams p) {
  constexpr int NC = 8;                  // compute waves
  constexpr int NDC = D / 16;            // 16-wide reduction chunks over d
  constexpr int KCH = D / 8;             // 16-byte chunks per row
  constexpr int TB = 64 * D * 2;         // bytes of a 64-row tile
  constexpr int WB = 64 * 4;             // bytes of a block's thresholds
  constexpr int SQ = TB + WB;            // ring slot
  constexpr int CPI = TB / 16 / 64;      // tile copies of the copy wave per item
  constexpr int OPS = CPI + 1;           // + the thresholds
  constexpr int LAG = 3;                 // items the copy wave keeps in flight
  static_assert(OPS * LAG < 64, "vmcnt range");
  constexpr int RQ = 8;                  // ring slots (even: a slot keeps its parity)
  constexpr int NB = 4;                  // key blocks per workgroup

  __shared__ __attribute__((aligned(16))) char ring[RQ * SQ];
  __shared__ int full[RQ];  // 1 + the item whose data the slot holds
  __shared__ int done[RQ];  // compute-wave completions of the slot's items
  __shared__ int csum[NC];
  __shared__ int stop;      // set by a wait that reached its bound

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hh = lane >> 5;

  const int per = p.batch * p.heads_kv;
  const int G4 = (int)(blockIdx.x / per);  // key blocks 4 G4 .. 4 G4 + 3, longest first
  const int bk = (int)(blockIdx.x % per);
  const int b = bk / p.heads_kv, kvh = bk % p.heads_kv;
  const int jb0 = NB * G4;
  const int i_lo = first_qblock(p, jb0);
  // item it is (group head it % group, query block tr - 1 - it / group); both
  // sides walk the items in order and step these indices instead of dividing
  const int n_items = p.group * (p.tr - i_lo);

  if (tid < RQ) {
    full[tid] = 0;
    done[tid] = 0;
  }
  if (tid == 0) stop = 0;
  lds_barrier();
  // wait until ready() holds, or give up: after p.spin unsuccessful polls
  // (at once when p.spin is 0) this wave raises `stop`, and every wait of
  // the workgroup returns as soon as it sees it
  auto wait_for = [&](auto ready) {
    for (int g = 0;; ++g) {
      if (g >= p.spin) {
        __hip_atomic_store(&stop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return;
      }
      if (ready()) return;
      if (__hip_atomic_load(&stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return;
      __builtin_amdgcn_s_sleep(1);
    }
  };

  if (w == NC) {
    // ======== copy wave ========
    // copies of the next item: row-major tile, chunks XOR-swizzled per row as
    // the 32-row operand reads expect (rows past the end re-read the last
    // row), then the 64 thresholds
    int fi = p.tr - 1, fh = 0;  // query block and group head of the next item fetched
    auto fetch = [&](uint32_t slot) {
      const int h = kvh * p.group + fh, i = fi;
      const __bf16* rows0 = p.q + ((size_t)(b * p.heads_q + h) * p.nq + (size_t)64 * i) * D;
      const int last = p.nq - 1 - 64 * i;  // last row inside the queries
#pragma unroll
      for (int x = 0; x < CPI; ++x) {
        const int s = x * 64 + lane;
        const int row = s / KCH, pc = s % KCH;
        const uint32_t voff =
            (uint32_t)((min(row, last) * D + ((pc ^ kswz32<D>(row)) & (KCH - 1)) * 8) * 2);
        async_copy16_sa(rows0, voff, slot + x * 1024);
      }
      const float* ri = p.rowinfo + ((size_t)(b * p.heads_q + h) * p.tr + i) * kRowInfo + 64;
      if (lane < 16) async_copy16_sa(ri, (uint32_t)(16 * lane), slot + TB);
    };
    auto publish = [&](int it) {
      if (lane == 0)
        __hip_atomic_store(&full[it % RQ], it + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    int marked = 0;  // items published so far
    for (int nf = 0; nf < n_items; ++nf) {
      if (nf >= RQ) {
        // the slot's previous item must be released by its four compute waves
        const int need = NB * (nf / RQ);
        if (__hip_atomic_load(&done[nf % RQ], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < need) {
          vmcnt_wait<0>();  // publish everything issued before waiting
          while (marked < nf) publish(marked++);
          wait_for([&] {
            return __hip_atomic_load(&done[nf % RQ], __ATOMIC_ACQUIRE,
                                     __HIP_MEMORY_SCOPE_WORKGROUP) >= need;
          });
        }
      }
      fetch(lds_addr(ring) + (uint32_t)((nf % RQ) * SQ));
      if (++fh == p.group) {
        fh = 0;
        --fi;
      }
      if (nf + 1 - marked > LAG) {  // keep LAG items in flight, publish the older ones
        vmcnt_wait<OPS * LAG>();
        while (marked <= nf - LAG) publish(marked++);
      }
    }
    vmcnt_wait<0>();
    while (marked < n_items) publish(marked++);
  } else {
    // ======== compute waves ========
    const int xb = w & 3;    // key block of this wave within the group
    const int par = w >> 2;  // parity of the items this wave scores
    const int jw = jb0 + xb;
    const bool live = jw < p.tc;
    const __bf16* kbase = p.k + (size_t)bk * p.nk * D;
    // K of the 64 keys as A operands: subtile kt, lane row 32 kt + l32
    bf16x8 kreg[2][NDC];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = 64 * jw + 32 * kt + l32;
      const bool ok = live && key < p.nk;
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc)
        kreg[kt][dc] = ok ? *(const bf16x8*)(kbase + (size_t)key * D + 16 * dc + 8 * hh) : bf16x8{};
    }
    int kept = 0;
    unsigned long long st_legal = 0, st_kept = 0, st_slots = 0;  // instrumentation
    // query block and group head of item k, advanced by two items per step
    int ci = p.tr - 1 - par / p.group, ch = par % p.group;
    // the item's decision byte, stepped with (ci, ch) rather than recomputed:
    // dmap[hoff + roff] with hoff = the map of head ch plus jw and roff = the
    // tiles stored for the query blocks before ci (a causal row i holds
    // i + cblk + 1 tiles below istar, tc from there on)
    const long long ph = p.dmap_per_head;
    const int istar = max(p.tc - p.cblk - 1, 0);
    long long hoff = (long long)(b * p.heads_q + kvh * p.group + ch) * ph + jw;
    long long roff = p.causal ? causal_row_start(ci, p.tc, p.cblk) : (long long)ci * p.tc;
    for (int k = par; k < n_items; k += 2) {
      const int slot = k % RQ;
      wait_for([&] {
        return __hip_atomic_load(&full[slot], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) ==
               k + 1;
      });
      const int i = ci;
      if (live && reaches(p, i, jw)) {
        const char* qt = ring + slot * SQ;
        const float* wr = (const float*)(qt + TB);
        const bool need_mask = diag_tile(p, i, jw) || (64 * jw + 64 > p.nk);
        // Both 32-column halves are always scored, even when the first
        // already has a passing entry (stopping early measured slower: the
        // four waves that score an item then take different times, and its
        // ring slot is refilled only after the last of them). The dense
        // path keeps every legal tile and scores nothing.
        bool hit = false;
#pragma unroll
        for (int qs = 0; qs < 2 && kTest; ++qs) {
          // B operands (Q^T: column 32 qs + l32) up front, then the products
          bf16x8 bq[NDC];
#pragma unroll
          for (int dc = 0; dc < NDC; ++dc) {
            const int row = 32 * qs + l32;
            const int ch = ((2 * dc + hh) ^ kswz32<D>(row)) & (KCH - 1);
            bq[dc] = *(const bf16x8*)(qt + row * D * 2 + ch * 16);
          }
          floatx16 s[2];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
#pragma unroll
          for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) s[kt] = mfma32x32x16(kreg[kt][dc], bq[dc], s[kt]);
          // every operand read is issued before the first product, so that
          // later reads land while earlier products run (left to itself the
          // scheduler alternates one read, a full wait and two products)
          __builtin_amdgcn_sched_group_barrier(0x100, NDC, 0);    // LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * NDC, 0);  // products
          // register 4e' + r of subtile kt holds key 32 kt + 8e' + 4hh + r
          // of query column 32 qs + l32
          if (need_mask) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                const int key = 64 * jw + 32 * kt + 8 * (e >> 2) + 4 * hh + (e & 3);
                const int qq = 64 * i + 32 * qs + l32;
                const bool ill = key >= p.nk || (p.causal && key > qq + p.off);
                s[kt][e] = ill ? -INFINITY : s[kt][e];
              }
          }
          // keep iff some legal entry has s >= W_q (masked entries are -inf;
          // W_q = -inf only for tau = 0, where every legal tile is kept, and
          // +inf for rows past the end)
          float mx = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kt][e]);
          hit = hit || mx >= wr[32 * qs + l32];
        }
        const bool want = kTest ? wave_any(hit) : true;
        kept += want ? 1 : 0;
        if (lane == 0) {
          const int bh = b * p.heads_q + kvh * p.group + ch;
          p.dmap[hoff + roff] = want ? 1 : 0;
          if (kStats) {
            ++st_legal;
            if (want) {
              ++st_kept;
              st_slots += (unsigned long long)min(64, p.nq - 64 * i) * 64ull;
            }
            if (p.decisions) p.decisions[((size_t)bh * p.tr + i) * p.tc + jw] = want ? 1 : 0;
          }
        }
      }
      // release the slot (this wave's reads of it have completed: the
      // products consumed them, and LDS operations of a wave complete in order)
      if (lane == 0)
        __hip_atomic_fetch_add(&done[slot], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      ch += 2;
      hoff += 2 * ph;
      while (ch >= p.group) {
        ch -= p.group;
        hoff -= p.group * ph;
        --ci;
        roff -= (p.causal && ci < istar) ? ci + p.cblk + 1 : p.tc;
      }
    }
    if (lane == 0) csum[w] = kept;
    if (kStats && lane == 0 && p.counters) {
      atomicAdd(&p.counters[0], st_legal);
      atomicAdd(&p.counters[1], st_kept);
      atomicAdd(&p.counters[2], st_slots);
    }
  }
  lds_barrier();
  // kept items per key block (waves x and x + 4 score block x)
  if (tid < NB && jb0 + tid < p.tc)
    p.kcount[(size_t)bk * p.tc + jb0 + tid] = csum[tid] + csum[tid + 4];
  // a wait gave up: the decisions may rest on unfinished copies
  if (tid == 0 && stop) *p.status = 1;
}

// ----------------------------------------------------------- coarsen ----
// Decision tiles of block_q x block_k = (64 kq) x (64 kk) (kq, kk in {1, 2}).
// The offline test of Eq. 4 keeps a tile iff some legal entry passes, so a
// coarse tile is kept iff one of its legal 64 x 64 sub-tiles is: the scoring
// pass decides the sub-tiles, and this pass ORs them and writes the result
// back into every legal sub-tile, so the dK/dV and dQ passes read the map as
// usual. One workgroup per (batch, KV head, coarse key column) walks the
// column's (query head, coarse query block) items; it also recounts the kept
// items of each 64-key block for the pairing pass and, when instrumented,
// counts and records the decisions per coarse tile.
template <bool kStats>
__global__ __launch_bounds__(256) void bwd_coarsen_kernel(BwdParams p) {
  __shared__ int cnt[2];
  __shared__ unsigned long long st[3];
  const int per = p.batch * p.heads_kv;
  const int bk = (int)(blockIdx.x % per), jc = (int)(blockIdx.x / per);
  const int b = bk / p.heads_kv, kvh = bk % p.heads_kv;
  const int trc = (p.tr + p.kq - 1) / p.kq, tcc = (p.tc + p.kk - 1) / p.kk;
  const int j0 = p.kk * jc, j1 = min(p.tc, j0 + p.kk);
  if (threadIdx.x < 2) cnt[threadIdx.x] = 0;
  if (threadIdx.x < 3) st[threadIdx.x] = 0;
  __syncthreads();
  int mycnt[2] = {0, 0};
  unsigned long long s_legal = 0, s_kept = 0, s_slots = 0;
  const int n_items = p.group * trc;
  for (int t = threadIdx.x; t < n_items; t += 256) {
    const int h = kvh * p.group + t % p.group, ic = t / p.group;
    const int bh = b * p.heads_q + h;
    const int i0 = p.kq * ic, i1 = min(p.tr, i0 + p.kq);
    bool any_legal = false, keep = false;
    for (int i = i0; i < i1; ++i)
      for (int j = j0; j < j1; ++j)
        if (reaches(p, i, j)) {
          any_legal = true;
          keep = keep || p.dmap[dmap_index(p, bh, i, j)] != 0;
        }
    if (!any_legal) continue;
    for (int i = i0; i < i1; ++i)
      for (int j = j0; j < j1; ++j)
        if (reaches(p, i, j)) {
          p.dmap[dmap_index(p, bh, i, j)] = keep ? 1 : 0;
          if (keep) ++mycnt[j - j0];
        }
    if (kStats) {
      ++s_legal;
      if (keep) {
        ++s_kept;
        s_slots += (unsigned long long)(min(p.nq, 64 * i1) - 64 * i0) * (64ull * p.kk);
      }
      if (p.decisions) p.decisions[((size_t)bh * trc + ic) * tcc + jc] = keep ? 1 : 0;
    }
  }
  atomicAdd(&cnt[0], mycnt[0]);
  atomicAdd(&cnt[1], mycnt[1]);
  if (kStats) {
    atomicAdd(&st[0], s_legal);
    atomicAdd(&st[1], s_kept);
    atomicAdd(&st[2], s_slots);
  }
  __syncthreads();
  if ((int)threadIdx.x < j1 - j0) p.kcount[(size_t)bk * p.tc + j0 + threadIdx.x] = cnt[threadIdx.x];
  if (kStats && threadIdx.x < 3 && p.counters) atomicAdd(&p.counters[threadIdx.x], st[threadIdx.x]);
}

// Dense path without instrumentation: every legal tile is kept, so the
// decision map is filled with ones instead of scoring.
__global__ __launch_bounds__(256) void bwd_dense_map_kernel(uint8_t* dmap, long long n) {
  const long long t = ((long long)blockIdx.x * 256 + threadIdx.x) * 16;
  if (t + 16 <= n) {
    *(uint4*)(dmap + t) = make_uint4(0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u);
  } else {
    for (long long x = t; x < n; ++x) dmap[x] = 1;
  }
}

// --------------------------------------------------------------- pair ----
// Key blocks are processed in pairs that share every Q and dO tile they
// read. The pairs come from the kept-item counts of the scoring pass: blocks
// that at least a quarter of their items keep (an attention sink, a
// retrieval hub) keep nearly the same items, every query block after them,
// so they are paired with each other in index order; the rest are paired in
// index order among themselves. Heavy pairs come first in the table, so the
// longest work is issued first. Each pair is then split into segments (see
// kSegKept), the (pair, segment) work items are listed in table order for
// the dK/dV pass, and every key block's entry in the segment table records
// its pair's segment count, its side of the pair and, for a pair of several
// segments, the first of the pair's partial-sum slots. One workgroup per
// (batch, KV head).
__global__ __launch_bounds__(256) void bwd_pair_kernel(BwdParams p) {
  __shared__ int wsum[4];
  __shared__ int scan[256];
  __shared__ int sscan[256];
  __shared__ long long ksum[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bk = blockIdx.x;
  const int* cnt = p.kcount + (size_t)bk * p.tc;
  int* pairs = p.pairs + (size_t)bk * p.npair * 2;
  auto heavy = [&](int j) {
    const long long n = (long long)p.group * (p.tr - first_qblock(p, j));
    return 4ll * cnt[j] >= n;
  };
  for (int x = tid; x < 2 * p.npair; x += 256) pairs[x] = -1;
  // number of heavy blocks
  int nh = 0;
  for (int j0 = 0; j0 < p.tc; j0 += 256) {
    const int j = j0 + tid;
    const unsigned long long bal = __ballot(j < p.tc && heavy(j));
    if (lane == 0) wsum[w] = __popcll(bal);
    __syncthreads();
    nh += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  const int ph = (nh + 1) / 2;  // heavy pairs
  int hrun = 0;                 // heavy blocks before this chunk
  for (int j0 = 0; j0 < p.tc; j0 += 256) {
    const int j = j0 + tid;
    const bool hv = j < p.tc && heavy(j);
    const unsigned long long bal = __ballot(hv);
    if (lane == 0) wsum[w] = __popcll(bal);
    __syncthreads();
    int hidx = hrun + __popcll(bal & ((1ull << lane) - 1ull));
    for (int y = 0; y < w; ++y) hidx += wsum[y];
    if (j < p.tc) {
      if (hv) {
        pairs[hidx] = j;  // pair hidx / 2, slot hidx % 2
      } else {
        const int lidx = j - hidx;  // light blocks before j
        pairs[2 * ph + lidx] = j;
      }
    }
    hrun += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  // segment length from the items all key blocks keep
  long long kall = 0;
  for (int j = tid; j < p.tc; j += 256) kall += cnt[j];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) kall += __shfl_xor(kall, off);
  if (lane == 0) ksum[w] = kall;
  __syncthreads();
  kall = ksum[0] + ksum[1] + ksum[2] + ksum[3];
  const long long lseg = max((long long)kSegKept, (2 * kall + (long long)kSlotsPerPair * p.npair - 1) /
                                                        ((long long)kSlotsPerPair * p.npair));
  // work items in table order and partial-sum slots (the barrier above also
  // made the pair table visible to the whole workgroup)
  int* work = p.work + (size_t)bk * p.wmax;
  int* seg = p.segtab + (size_t)bk * p.tc;
  int base = 0, sbase = 0;
  for (int x0 = 0; x0 < p.npair; x0 += 256) {
    const int pr = x0 + tid;
    int nseg = 0, jA = -1, jB = -1;
    if (pr < p.npair) {
      jA = pairs[2 * pr];
      jB = pairs[2 * pr + 1];
      if (jA >= 0) {
        const long long kept = cnt[jA] + (jB >= 0 ? cnt[jB] : 0);
        nseg = (int)min((long long)kSegMax, max(1ll, (kept + lseg - 1) / lseg));
      }
    }
    const int nslot = nseg > 1 ? nseg : 0;
    scan[tid] = nseg;
    sscan[tid] = nslot;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {  // inclusive prefix sums
      const int v = tid >= off ? scan[tid - off] : 0;
      const int u = tid >= off ? sscan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      sscan[tid] += u;
      __syncthreads();
    }
    const int first = base + scan[tid] - nseg;
    const int slot = sbase + sscan[tid] - nslot;  // < kSlotsPerPair npair (see kSegKept)
    for (int sg = 0; sg < nseg; ++sg) work[first + sg] = pr | (sg << 20) | (nseg << 24);
    if (jA >= 0) seg[jA] = nseg | (0 << 4) | (slot << 5);
    if (jB >= 0) seg[jB] = nseg | (1 << 4) | (slot << 5);
    base += scan[255];
    sbase += sscan[255];
    __syncthreads();
  }
  if (tid == 0) p.wcnt[bk] = base;
}

// ----------------------------------------------------------- finalize ----
// dK = scale * sum of the segments' partial sums, dV = their sum (segments
// added in index order), for the key blocks whose pair was split into
// several segments (the count is recorded per block by the dK/dV pass).
template <int D>
__global__ __launch_bounds__(256) void bwd_kv_finalize_kernel(BwdParams p) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;  // 8 values each
  const long long n = (long long)p.batch * p.heads_kv * p.tc * 64 * D / 8;
  if (t >= n) return;
  const long long e = t * 8;
  const int col = (int)(e % D);
  const int row = (int)((e / D) % 64);
  const long long bj = e / D / 64;  // bk * Tc + j
  const int j = (int)(bj % p.tc);
  const long long bk = bj / p.tc;
  const int st = p.segtab[bj];
  const int nseg = st & 15, side = (st >> 4) & 1, slot = st >> 5;
  const int kk = 64 * j + row;
  if (nseg <= 1 || kk >= p.nk) return;
  const float poison = *p.status ? NAN : 1.f;
  float ak[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float av[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int sg = 0; sg < nseg; ++sg) {
    const float* pk =
        p.part + (((bk * kSlotsPerPair * p.npair + slot + sg) * 2 + side) * 2 * 64 + row) * D + col;
    const float* pv = pk + 64 * D;
    const float4 k0 = *(const float4*)pk, k1 = *(const float4*)(pk + 4);
    const float4 v0 = *(const float4*)pv, v1 = *(const float4*)(pv + 4);
    ak[0] += k0.x; ak[1] += k0.y; ak[2] += k0.z; ak[3] += k0.w;
    ak[4] += k1.x; ak[5] += k1.y; ak[6] += k1.z; ak[7] += k1.w;
    av[0] += v0.x; av[1] += v0.y; av[2] += v0.z; av[3] += v0.w;
    av[4] += v1.x; av[5] += v1.y; av[6] += v1.z; av[7] += v1.w;
  }
  bf16x8 ok, ov;
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    ok[x] = to_bf16(ak[x] * p.scale * poison);
    ov[x] = to_bf16(av[x] * poison);
  }
  *(bf16x8*)(p.dk + ((size_t)bk * p.nk + kk) * D + col) = ok;
  *(bf16x8*)(p.dv + ((size_t)bk * p.nk + kk) * D + col) = ov;
}

// ----------------------------------------------------------------- dq ----
template <int D, bool kTest>  // (kTest only names the MALA / dense instances apart)
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(BwdParams p) {
  constexpr int NDC = D / 32;
  constexpr int NDS = D / 16;
  constexpr int KCH = D / 8;
  constexpr int NT = 512;
  constexpr int NQS = 2;              // 16-query subtiles per wave (32 rows)
  constexpr int CPT = 64 * KCH / NT;  // async copies per thread per tile
  constexpr int RK = 3;               // K and V rings: current + 2 ahead
  constexpr int LMAX = 2048;          // list entries per segment of key blocks

  __shared__ __attribute__((aligned(16))) __bf16 k_ring[RK][64 * D];
  __shared__ __attribute__((aligned(16))) __bf16 v_ring[RK][64 * D];
  __shared__ int list[LMAX];
  __shared__ int wcount[8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l16 = lane & 15, g4 = lane >> 4;

  // ---- work item (longest query-block group first), as the forward ----
  const int per_ig = p.batch * p.heads_kv * p.n_hg;
  const int ig = p.n_ig - 1 - (int)(blockIdx.x / per_ig);
  int rem = (int)(blockIdx.x % per_ig);
  const int hg = rem % p.n_hg;
  rem /= p.n_hg;
  const int kvh = rem % p.heads_kv;
  const int b = rem / p.heads_kv;

  const int blk = w >> 1, half = w & 1;
  auto blk_h = [&](int x) { return kvh * p.group + hg * p.hpw + (x % p.hpw); };
  auto blk_i = [&](int x) { return ig * p.ipw + (x / p.hpw); };
  const int h = blk_h(blk), i = blk_i(blk);
  const bool valid = i < p.tr;
  const int q0 = 64 * i + 32 * half;
  const int i_top = min(ig * p.ipw + p.ipw - 1, p.tr - 1);
  const int jtop = p.causal ? min(p.tc - 1, i_top + p.cblk) : p.tc - 1;
  const size_t qrow0 = (size_t)(b * p.heads_q + h) * p.nq;
  const __bf16* kbase = p.k + (size_t)(b * p.heads_kv + kvh) * p.nk * D;
  const __bf16* vbase = p.v + (size_t)(b * p.heads_kv + kvh) * p.nk * D;

  // Q and dO rows of this wave as B operands; row terms per query column
  bf16x8 qr[NQS][NDC], dr[NQS][NDC];
  float z2[NQS], dq_d[NQS];
  floatx4 acc[NDS][NQS];
#pragma unroll
  for (int qs = 0; qs < NQS; ++qs) {
    const int qq = q0 + 16 * qs + l16;
    const bool ok = valid && qq < p.nq;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      qr[qs][dc] = ok ? *(const bf16x8*)(p.q + (qrow0 + qq) * D + 32 * dc + 8 * g4) : bf16x8{};
      dr[qs][dc] = ok ? *(const bf16x8*)(p.dout + (qrow0 + qq) * D + 32 * dc + 8 * g4) : bf16x8{};
    }
    const float* ri =
        p.rowinfo + ((size_t)(b * p.heads_q + h) * p.tr + (valid ? i : 0)) * kRowInfo;
    const int ql = 32 * half + 16 * qs + l16;
    z2[qs] = valid ? ri[ql] : INFINITY;
    dq_d[qs] = valid ? ri[128 + ql] : 0.f;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) acc[ds][qs] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  auto issue_tile = [&](const __bf16* base, int j, __bf16* slot) {
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      const int s0 = x * NT + w * 64;
      const int s = s0 + lane;
      const int row = s / KCH, pc = s % KCH;
      const int kk = min(j * 64 + row, p.nk - 1);
      async_copy16_a(base + (size_t)kk * D + ((pc ^ dqswz<D>(row)) & (KCH - 1)) * 8,
                     lds_addr(slot) + (uint32_t)s0 * 16u);
    }
  };

  // K^T operands of the dQ product: the transposing read for key subtile
  // pair kc, half hh and d chunk ds takes rows 32 kc + 4 hh + 8 g4 + l16 / 4
  // at columns 16 ds + 4 (l16 % 4) .. + 3. The row swizzle depends only on
  // 8 g4 + l16 / 4, so the lane's offset for chunk ds is fixed and (kc, hh)
  // add a constant (an immediate of the read)
  int ktr_off[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    const int row = 8 * g4 + (l16 >> 2);
    const int col = 16 * ds + 4 * (l16 & 3);
    ktr_off[ds] = row * D + (((col >> 3) ^ dqswz<D>(row)) & (KCH - 1)) * 8 + (col & 7);
  }

  // one kept tile: S^T, dP^T, dS^T, dQ^T += K^T dS^T, one half of the 64
  // keys (key subtiles 2kc, 2kc + 1) at a time
  // (mid runs once, after the first half's S^T and dP^T products)
  auto process = [&](const __bf16* kt, const __bf16* vt, int j, auto&& mid) {
    const bool need_mask = diag_tile(p, i, j) || (j * 64 + 64 > p.nk);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      floatx4 s[2][NQS], dp[2][NQS];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) {
          s[x][qs] = floatx4{0.f, 0.f, 0.f, 0.f};
          dp[x][qs] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          // MFMA row l16 of key subtile 2kc + x holds key qperm(2kc + x, l16)
          const int kr = qperm(2 * kc + x, l16);
          const int ch = 4 * dc + g4;
          const int off = kr * D + ((ch ^ dqswz<D>(kr)) & (KCH - 1)) * 8;
          const bf16x8 ak = *(const bf16x8*)(kt + off);
          const bf16x8 av = *(const bf16x8*)(vt + off);
#pragma unroll
          for (int qs = 0; qs < NQS; ++qs) {
            s[x][qs] = mfma16x16x32(ak, qr[qs][dc], s[x][qs]);
            dp[x][qs] = mfma16x16x32(av, dr[qs][dc], dp[x][qs]);
          }
        }
      if (need_mask) {
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int kk = j * 64 + qperm(2 * kc + x, 4 * g4 + r);
              const int qq = q0 + 16 * qs + l16;
              if (kk >= p.nk || (p.causal && kk > qq + p.off)) s[x][qs][r] = -INFINITY;
            }
      }
      if (kc == 0) mid();
      // dS^T = P^T (dP^T - D) as B operands [key][query]: keys 32kc + 8g4 + e
      bf16x8 db[NQS];
#pragma unroll
      for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pv = fast_exp2(s[x][qs][r] * p.c - z2[qs]);
            db[qs][4 * x + r] = to_bf16(pv * (dp[x][qs][r] - dq_d[qs]));
          }
      // dQ^T += K^T dS^T: A = K^T from transposing reads of the K tile
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        short4v t2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) t2[hh] = lds_read_tr4(kt + ktr_off[ds] + (32 * kc + 4 * hh) * D);
        const bf16x8 a = join_tr(t2[0], t2[1]);
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) acc[ds][qs] = mfma16x16x32(a, db[qs], acc[ds][qs]);
      }
    }
  };

  // ---- segments of at most LMAX candidate key blocks, from the top ----
  for (int jseg = jtop; jseg >= 0; jseg -= LMAX) {
    const int jlo = max(0, jseg - LMAX + 1);
    lds_barrier();  // the previous segment's list is no longer read
    // list (descending j) of key blocks some block of the group keeps:
    // entry = j | (block mask << 24)
    int base = 0;
    for (int c0 = 0; c0 <= jseg - jlo; c0 += NT) {
      const int j = jseg - (c0 + tid);
      int mask = 0;
      if (j >= jlo) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int ix = blk_i(x);
          if (ix >= p.tr || !reaches(p, ix, j)) continue;
          const int bh = b * p.heads_q + blk_h(x);
          if (p.dmap[dmap_index(p, bh, ix, j)] != 0) mask |= 1 << x;
        }
      }
      const unsigned long long bal = __ballot(mask != 0);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wcount[w] = __popcll(bal);
      lds_barrier();
      int off = base;
      for (int x = 0; x < w; ++x) off += wcount[x];
      if (mask != 0) list[off + before] = j | (mask << 24);
      int tot = 0;
#pragma unroll
      for (int x = 0; x < 8; ++x) tot += wcount[x];
      base += tot;
      lds_barrier();  // wcount reused; list entries visible
    }
    const int n = base;

    // pipeline: K and V of the listed tiles two ahead
    if (n > 0) {
      const int ja = list[0] & 0xFFFFFF;
      issue_tile(kbase, ja, k_ring[0]);
      issue_tile(vbase, ja, v_ring[0]);
    }
    if (n > 1) {
      const int jb = list[1] & 0xFFFFFF;
      issue_tile(kbase, jb, k_ring[1]);
      issue_tile(vbase, jb, v_ring[1]);
    }
    // ring slots of tiles t and t + 2, stepped rather than taken modulo RK
    // (the compiler turned t % RK into two running terms added at every
    // operand read)
    int cur = 0, ahead = 2 % RK;
    for (int t = 0; t < n; ++t) {
      vmcnt_wait_le(t + 1 < n ? 2 * CPT : 0);  // K, V of tile t + 1 may be in flight
      lds_barrier();
      // K and V of tile t + 2 into the slots of tile t - 1 (done by every
      // wave at the barrier). The two waves of a SIMD (w and w + 4) issue
      // these copies at different points: waves 0-3 now, waves 4-7 after
      // their first products when they process tile t, so that one wave's
      // wait for the copy path overlaps the other's products.
      auto issue_next = [&] {
        if (t + 2 < n) {
          const int jn = list[t + 2] & 0xFFFFFF;
          issue_tile(kbase, jn, k_ring[ahead]);
          issue_tile(vbase, jn, v_ring[ahead]);
        }
      };
      const int e = list[t];
      const bool mine = valid && ((e >> (24 + blk)) & 1);
      const bool late = w >= 4;
      if (!late || !mine) issue_next();
      if (mine)
        process(k_ring[cur], v_ring[cur], e & 0xFFFFFF, [&] {
          if (late) issue_next();
        });
      cur = cur + 1 == RK ? 0 : cur + 1;
      ahead = ahead + 1 == RK ? 0 : ahead + 1;
    }
  }

  // ---- dQ = scale * acc (bf16); lane holds query column l16, d rows 4g4+r
  //      (NaN when a wait of the scoring pass gave up) ----
  if (valid) {
    const float sc = *p.status ? NAN : p.scale;
#pragma unroll
    for (int qs = 0; qs < NQS; ++qs) {
      const int qq = q0 + 16 * qs + l16;
      if (qq >= p.nq) continue;
      __bf16* row = p.dq + (qrow0 + qq) * D;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        bf16x4 t;
        t[0] = to_bf16(acc[ds][qs][0] * sc);
        t[1] = to_bf16(acc[ds][qs][1] * sc);
        t[2] = to_bf16(acc[ds][qs][2] * sc);
        t[3] = to_bf16(acc[ds][qs][3] * sc);
        *(bf16x4*)(row + 16 * ds + 4 * g4) = t;
      }
    }
  }
}

template <int D, bool kTest, bool kStats>
hipError_t launch_all(const BwdParams& p, hipStream_t stream) {
  const long long prows = (long long)p.batch * p.heads_q * p.tr * 64;
  const long long pre_threads = prows * (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((pre_threads + 255) / 256)), dim3(256),
                     0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long per = (long long)p.batch * p.heads_kv;
  const bool coarse = p.kq * p.kk > 1;
  if (kTest && coarse) {
    // 64 x 64 sub-tile decisions; counting and recording happen per coarse tile
    hipLaunchKernelGGL((bwd_score_kernel<D, true, false>),
                       dim3((unsigned)(((p.tc + 3) / 4) * per)), dim3(576), 0, stream, p);
  } else if (kTest || (kStats && !coarse)) {
    hipLaunchKernelGGL((bwd_score_kernel<D, kTest, kStats>),
                       dim3((unsigned)(((p.tc + 3) / 4) * per)), dim3(576), 0, stream, p);
  } else {
    const long long n = (long long)p.batch * p.heads_q * p.dmap_per_head;
    hipLaunchKernelGGL(bwd_dense_map_kernel, dim3((unsigned)((n + 4095) / 4096)), dim3(256), 0,
                       stream, p.dmap, n);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (coarse && (kTest || kStats)) {
    const long long tcc = (p.tc + p.kk - 1) / p.kk;
    hipLaunchKernelGGL((bwd_coarsen_kernel<kStats>), dim3((unsigned)(tcc * per)), dim3(256), 0,
                       stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdParams q = p;
  if (kTest) {
    hipLaunchKernelGGL(bwd_pair_kernel, dim3((unsigned)per), dim3(256), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    q.pairs = nullptr;  // dense: blocks 2 pr and 2 pr + 1 keep the same items
    q.segtab = nullptr;
  }
  e = launch_bwd_kv<D, kTest, kStats>(q, (unsigned)((long long)(kTest ? p.wmax : p.npair) * per),
                                      stream);
  if (e != hipSuccess) return e;
  if (kTest) {
    const long long nfin = (long long)p.tc * per * 64 * D / 8;
    hipLaunchKernelGGL((bwd_kv_finalize_kernel<D>), dim3((unsigned)((nfin + 255) / 256)),
                       dim3(256), 0, stream, q);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long nblocks = (long long)p.n_ig * p.batch * p.heads_kv * p.n_hg;
  hipLaunchKernelGGL((bwd_dq_kernel<D, kTest>), dim3((unsigned)nblocks), dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdParams& p, bool test, hipStream_t stream) {
  const bool stats = p.counters != nullptr || p.decisions != nullptr;
  if (test)
    return stats ? launch_all<D, true, true>(p, stream) : launch_all<D, true, false>(p, stream);
  return stats ? launch_all<D, false, true>(p, stream) : launch_all<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, bool test, hipStream_t stream) {
  BwdParams p;
  p.q = (const __bf16*)a.q;
  p.k = (const __bf16*)a.k;
  p.v = (const __bf16*)a.v;
  p.o = (const __bf16*)a.o;
  p.lse = a.lse;
  p.dout = (const __bf16*)a.dout;
  p.dq = (__bf16*)a.dq;
  p.dk = (__bf16*)a.dk;
  p.dv = (__bf16*)a.dv;
  p.batch = a.batch;
  p.heads_q = a.heads_q;
  p.heads_kv = a.heads_kv;
  p.nq = a.nq;
  p.nk = a.nk;
  p.group = a.heads_q / a.heads_kv;
  p.causal = a.causal;
  p.off = a.causal ? a.nk - a.nq : 0;
  p.cblk = (63 + p.off) / 64;
  p.scale = a.scale;
  p.c = a.scale * kLog2e;
  p.log2_tau = a.tau == 0.f ? -INFINITY : log2f(a.tau);
  p.tr = (a.nq + 63) / 64;
  p.tc = (a.nk + 63) / 64;
  p.dmap_per_head = p.causal ? causal_row_start(p.tr, p.tc, p.cblk) : (long long)p.tr * p.tc;
  const size_t rowinfo = (size_t)a.batch * a.heads_q * (size_t)p.tr * kRowInfo * sizeof(float);
  p.status = (int*)a.workspace;
  p.spin = a.spin;
  p.rowinfo = (float*)((char*)a.workspace + kBwdHeader);
  p.dmap = (uint8_t*)p.rowinfo + ((rowinfo + 255) & ~(size_t)255);
  const size_t dmap_bytes = (size_t)a.batch * a.heads_q * (size_t)p.dmap_per_head;
  p.part = (float*)(p.dmap + ((dmap_bytes + 255) & ~(size_t)255));
  p.npair = p.tc / 2 + 1;
  const size_t nkb = (size_t)a.batch * a.heads_kv * p.tc;
  const size_t nbk = (size_t)a.batch * a.heads_kv;
  p.kcount = (int*)(p.part + nbk * kSlotsPerPair * p.npair * 2 * 2 * 64 * a.head_dim);
  p.segtab = p.kcount + nkb;
  p.pairs = p.segtab + nkb;
  p.wmax = p.npair * kSegMax;
  p.work = p.pairs + nbk * p.npair * 2;
  p.wcnt = p.work + nbk * p.wmax;
  if (p.group % 4 == 0) {
    p.hpw = 4;
    p.ipw = 1;
  } else if (p.group % 2 == 0) {
    p.hpw = 2;
    p.ipw = 2;
  } else {
    p.hpw = 1;
    p.ipw = 4;
  }
  p.n_hg = p.group / p.hpw;
  p.n_ig = (p.tr + p.ipw - 1) / p.ipw;
  p.kq = a.block_q / 64;
  p.kk = a.block_k / 64;
  p.counters = a.counters;
  p.decisions = a.decisions;
  return a.head_dim == 128 ? launch_d<128>(p, test, stream) : launch_d<64>(p, test, stream);
}

}  // namespace mala
