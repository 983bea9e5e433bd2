// MALA backward, dK/dV pass ("MassAlloc Attention: Let Attention Allocate
// Its Own Compute": Sec. 2.2 Eq. 4, Appendix A Algorithm 2 and the backward
// part of Appendix A.1), and the dense FullAttn dK/dV from the same template.
// The other backward passes and their launch sequence are in mala_bwd.hip;
// this pass is a translation unit of its own so that it can be compiled with
// its own instruction-scheduling strategy (the build passes it to this file
// only; the other passes measured slower with it).
#include "mala_bwd.h"

namespace mala {
namespace {

// ----------------------------------------------------------------- kv ----
// dK, dV over the kept tiles. A workgroup of 4 wave64s (one per SIMD) owns
// a pair of key blocks (or one): wave w holds keys 32 (w % 2) .. +31 of the
// pair's block w / 2, with K and V as the B operands of S = Q K^T and
// dP = dO V^T (32x32x16 bf16 MFMA) and dK^T, dV^T accumulated in registers.
// Per chunk of (query block, query head) items it reads both blocks'
// decisions from the decision map and lists the items either block keeps;
// Q, dO and the row terms of a listed item are copied once, asynchronously,
// into an LDS ring three entries ahead, and the waves of each block that
// keeps it run the post-score work for 32 queries at a time: S is
// recomputed, P = exp2(s c - z2), dS = P (dP - D); the S layout (a lane
// holds one key and 16 queries) is already the B operand of
// dV^T += dO^T P and dK^T += Q^T dS, whose A operands come from transposing
// reads of the same Q and dO tiles.
template <int D, bool kTest, bool kStats>
__global__ __launch_bounds__(256, 1) void bwd_kv_kernel(BwdParams p) {
  constexpr int NT = 256;                // 4 wave64s
  constexpr int NDC = D / 16;            // 16-wide reduction chunks over d
  constexpr int NDT = D / 32;            // 32-row subtiles of dK^T, dV^T over d
  constexpr int KCH = D / 8;             // 16-byte chunks per row
  constexpr int TB = 64 * D * 2;         // bytes of a 64-row tile
  constexpr int RB = 2 * 64 * 4;         // z2 and D of the 64 rows
  constexpr int CPW = TB / 16 / NT;      // 16-byte copies per lane per tile
  constexpr int OPS = 2 * CPW + 1;       // copies per wave per list entry
  static_assert(2 * OPS < 64, "vmcnt range");
  constexpr int RP = 4;                  // ring: the entry in use + 3 ahead
  constexpr int SP = 2 * TB + RB;        // ring slot: Q, dO, row terms
  constexpr int CH = 2048;               // items per chunk

  __shared__ __attribute__((aligned(16))) char ring[RP * SP];
  __shared__ int list[CH];
  __shared__ int list_i[CH];  // query block of each listed item
  __shared__ int wcount[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hh = lane >> 5;
  const int sb = w >> 1, kh = w & 1;  // block of the pair, 32-key half

  // ---- work item b of the list the pairing pass wrote (MALA), or pair b
  //      (dense), the first item of every (batch, KV head) first; the grid
  //      bounds the list, and workgroups past its end exit at once. Items
  //      are issued in list order (longest first) and consecutive items,
  //      such as the segments of one pair, go to different XCDs ----
  const int per = p.batch * p.heads_kv;
  const int bk = (int)(blockIdx.x % per), idx = (int)(blockIdx.x / per);
  int pr, seg, nseg;
  if (p.pairs) {
    if (idx >= p.wcnt[bk]) return;  // (whole workgroup, before any barrier)
    const int wi = p.work[(size_t)bk * p.wmax + idx];
    pr = wi & 0xFFFFF;
    seg = (wi >> 20) & 15;
    nseg = wi >> 24;
  } else {  // dense: blocks 2 pr and 2 pr + 1, one segment
    if (idx >= (p.tc + 1) / 2) return;
    pr = idx;
    seg = 0;
    nseg = 1;
  }
  const int b = bk / p.heads_kv, kvh = bk % p.heads_kv;
  int jA, jB;
  if (p.pairs) {
    jA = p.pairs[((size_t)bk * p.npair + pr) * 2];
    jB = p.pairs[((size_t)bk * p.npair + pr) * 2 + 1];
  } else {
    jA = 2 * pr;
    jB = 2 * pr + 1 < p.tc ? 2 * pr + 1 : -1;
  }
  const int jlo = jB >= 0 ? min(jA, jB) : jA;
  const int i_lo = first_qblock(p, jlo);
  const int n_all = p.group * (p.tr - i_lo);
  const int j = sb ? jB : jA;  // this wave's key block (-1: none)
  const __bf16* kbase = p.k + (size_t)bk * p.nk * D;
  const __bf16* vbase = p.v + (size_t)bk * p.nk * D;

  // K and V of this lane's key (column l32 of the B operands), chunk
  // 8 hh .. 8 hh + 7 of each 16-wide d chunk
  const int key = 64 * j + 32 * kh + l32;
  bf16x8 kb[NDC], vb[NDC];
  {
    const bool ok = j >= 0 && key < p.nk;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      kb[dc] = ok ? *(const bf16x8*)(kbase + (size_t)key * D + 16 * dc + 8 * hh) : bf16x8{};
      vb[dc] = ok ? *(const bf16x8*)(vbase + (size_t)key * D + 16 * dc + 8 * hh) : bf16x8{};
    }
  }
  floatx16 dkt[NDT], dvt[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dkt[dt][e] = 0.f;
      dvt[dt][e] = 0.f;
    }

  // items: query blocks from the last one down to the first with a legal
  // entry for either block, query heads of the group innermost
  const int seg_len = (n_all + nseg - 1) / nseg;
  const int it0 = seg * seg_len;                        // this segment's items:
  const int n_items = min(n_all, it0 + seg_len) - it0;  // it0 .. it0 + n_items - 1
  auto item_i = [&](int it) { return p.tr - 1 - (it0 + it) / p.group; };
  auto item_h = [&](int it) { return kvh * p.group + (it0 + it) % p.group; };
  auto legal = [&](int jx, int i) { return jx >= 0 && reaches(p, i, jx); };

  // ---- asynchronous tile copies: each wave moves a quarter of a tile and
  //      eight of the 32 row-term chunks ----
  const uint32_t ring_lds = lds_addr(ring);
  uint32_t toff[CPW];  // byte offset within a full tile, per copy
#pragma unroll
  for (int x = 0; x < CPW; ++x) {
    const int s = (4 * x + w) * 64 + lane;  // 16-byte chunk this lane fetches
    const int row = s / KCH, pc = s % KCH;
    toff[x] = (uint32_t)(row * D * 2 + ((pc ^ qswz32<D>(row)) & (KCH - 1)) * 16);
  }
  auto copy_tile = [&](const __bf16* rows0, int i, uint32_t slot) {
    // rows0: row 0 of (b, h); block i lands swizzled in the ring slot whose
    // part for this wave starts at `slot` (the slot plus w KiB)
    if (64 * i + 64 <= p.nq) {
      const char* src = (const char*)(rows0 + (size_t)64 * i * D);
#pragma unroll
      for (int x = 0; x < CPW; ++x) async_copy16_sa(src, toff[x], slot + x * 4096);
    } else {  // ragged last block: rows past the end re-read the last row
#pragma unroll
      for (int x = 0; x < CPW; ++x) {
        const int s = (4 * x + w) * 64 + lane;
        const int row = s / KCH, pc = s % KCH;
        const int qq = min(64 * i + row, p.nq - 1);
        async_copy16_a(rows0 + (size_t)qq * D + ((pc ^ qswz32<D>(row)) & (KCH - 1)) * 8,
                       slot + x * 4096);
      }
    }
  };
  // row terms: chunk c = 8w + lane (lanes 0..7) of [z2 x64][D x64]
  const uint32_t roff = (uint32_t)(16 * (8 * w + (lane & 7)) + (w >= 2 ? 256 : 0));
  auto copy_rowinfo = [&](int h, int i, uint32_t slot) {
    const float* src = p.rowinfo + ((size_t)(b * p.heads_q + h) * p.tr + i) * kRowInfo;
    if (lane < 8) async_copy16_sa(src, roff, slot + 128 * w);
  };

  // transposing-read coordinates (as the forward's V^T operand): a lane
  // receives column 32 dt + l32 of rows 16 c + 4 hh + 0..3 (u = 0) and
  // 16 c + 8 + 4 hh + 0..3 (u = 1)
  const int g16 = lane >> 4, j16 = lane & 15;
  const int tr_row = 4 * (g16 >> 1) + (j16 >> 2);
  const int tr_col = 16 * (g16 & 1) + 4 * (j16 & 3);
  auto a_tr = [&](const __bf16* t, int r0, int dt) {
    short4v h2[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = r0 + 8 * u + tr_row;
      const int col = 32 * dt + tr_col;
      const int ch = ((col >> 3) ^ qswz32<D>(row)) & (KCH - 1);
      h2[u] = lds_read_tr4(t + row * D + ch * 8 + (col & 7));
    }
    return join_tr(h2[0], h2[1]);
  };

  unsigned long long st_items = 0;  // instrumentation: kept (item, block) pairs listed
  for (int c0 = 0; c0 < n_items; c0 += CH) {
    const int nc = min(n_items - c0, CH);

    // ---- list of the chunk's items either block keeps (decision map
    //      written by the scoring pass): entry = item | keep mask << 28,
    //      and the item's query block in list_i ----
    lds_barrier();  // the previous chunk's list and ring are no longer read
    int n_list = 0;
    for (int x0 = 0; x0 < nc; x0 += NT) {
      const int x = x0 + tid;
      int mask = 0, i = 0;
      if (x < nc) {
        const int it = c0 + x;
        const int h = item_h(it);
        i = item_i(it);
        const int bh = b * p.heads_q + h;
        if (legal(jA, i) && p.dmap[dmap_index(p, bh, i, jA)] != 0) mask |= 1;
        if (legal(jB, i) && p.dmap[dmap_index(p, bh, i, jB)] != 0) mask |= 2;
        if (kStats) st_items += __popc(mask);
      }
      const unsigned long long bal = __ballot(mask != 0);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wcount[w] = __popcll(bal);
      lds_barrier();
      int off = n_list;
      for (int y = 0; y < w; ++y) off += wcount[y];
      if (mask) {
        list[off + before] = x | (mask << 28);
        list_i[off + before] = i;
      }
      n_list += wcount[0] + wcount[1] + wcount[2] + wcount[3];
      lds_barrier();  // wcount reused; list entries visible
    }
    vmcnt_wait<0>();  // the map reads are done (the post phase counts copies only)

    // ======== post-score work of the listed items, three entries ahead ========
    // (the item's query block comes from list_i, its head from
    // it0 + it = (tr - 1 - i) group + (h - kvh group), without a division)
    auto issue_post = [&](int t) {
      const int it = c0 + (list[t] & 0xFFFFFFF);
      const int i = list_i[t];
      const int h = kvh * p.group + (it0 + it) - (p.tr - 1 - i) * p.group;
      const uint32_t slot = ring_lds + (uint32_t)((t % RP) * SP);
      const size_t rows = (size_t)(b * p.heads_q + h) * p.nq * D;
      const uint32_t wslot = slot + (uint32_t)w * 1024u;
      copy_tile(p.q + rows, i, wslot);
      copy_tile(p.dout + rows, i, wslot + TB);
      copy_rowinfo(h, i, slot + 2 * TB);
    };
    int issued = 0;
    for (; issued < RP - 1 && issued < n_list; ++issued) issue_post(issued);
    for (int t = 0; t < n_list; ++t) {
      // entry t landed: at most two later entries in flight (a fixed count
      // per case, no run-time selection among all possible counts)
      if (issued - (t + 1) >= 2) vmcnt_wait<2 * OPS>();
      else if (issued - (t + 1) == 1) vmcnt_wait<OPS>();
      else vmcnt_wait<0>();
      lds_barrier();  // entry t visible; every wave is done with entry t - 1
      if (issued < n_list) {  // into the slot of entry t - 1
        issue_post(issued);
        ++issued;
      }
      const int e = list[t];
      if (!((e >> (28 + sb)) & 1)) continue;
      const int i = list_i[t];
      const __bf16* qt = (const __bf16*)(ring + (t % RP) * SP);
      const __bf16* dt_ = qt + 64 * D;
      const float* ri = (const float*)(qt + 2 * 64 * D);
      const bool need_mask = diag_tile(p, i, j) || (64 * j + 64 > p.nk);
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        // S and dP for queries 32 qs .. 32 qs + 31: A = Q / dO rows
        const int row = 32 * qs + l32;
        floatx16 s, dp;
#pragma unroll
        for (int e2 = 0; e2 < 16; ++e2) {
          s[e2] = 0.f;
          dp[e2] = 0.f;
        }
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
          const int ch = ((2 * dc + hh) ^ qswz32<D>(row)) & (KCH - 1);
          const bf16x8 aq = *(const bf16x8*)(qt + row * D + ch * 8);
          const bf16x8 ao = *(const bf16x8*)(dt_ + row * D + ch * 8);
          s = mfma32x32x16(aq, kb[dc], s);
          dp = mfma32x32x16(ao, vb[dc], dp);
        }
        // register 4e' + r holds query 32 qs + 8e' + 4hh + r of this lane's key
        if (need_mask) {
#pragma unroll
          for (int e2 = 0; e2 < 16; ++e2) {
            const int qq = 64 * i + 32 * qs + 8 * (e2 >> 2) + 4 * hh + (e2 & 3);
            const bool ill = key >= p.nk || (p.causal && key > qq + p.off);
            s[e2] = ill ? -INFINITY : s[e2];
          }
        }
        // P = exp2(s c - z2), dS = P (dP - D); chunk c2 of 16 queries is the
        // B operand over queries 32 qs + 16 c2 + {4hh + 0..3, 8 + 4hh + 0..3}
        bf16x8 pb[2], db[2];
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int ql = 32 * qs + 8 * e4 + 4 * hh;
          const float4 z4 = *(const float4*)(ri + ql);
          const float4 d4 = *(const float4*)(ri + 64 + ql);
          const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
          const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e2 = 4 * e4 + r;
            const float pv = fast_exp2(s[e2] * p.c - zz[r]);
            pb[e4 >> 1][4 * (e4 & 1) + r] = to_bf16(pv);
            db[e4 >> 1][4 * (e4 & 1) + r] = to_bf16(pv * (dp[e2] - dd[r]));
          }
        }
        // dV^T += dO^T P, dK^T += Q^T dS over these 32 queries
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int d2 = 0; d2 < NDT; ++d2) {
            dvt[d2] = mfma32x32x16(a_tr(dt_, 32 * qs + 16 * c2, d2), pb[c2], dvt[d2]);
            dkt[d2] = mfma32x32x16(a_tr(qt, 32 * qs + 16 * c2, d2), db[c2], dkt[d2]);
          }
      }
    }
  }

  if (kStats && p.counters) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) st_items += __shfl_xor(st_items, off);
    if (lane == 0 && st_items) atomicAdd(&p.counters[3], st_items);
  }
  // ---- output: lane holds key 32 kh + l32 of block j, register 4e' + r of
  //      subtile dt = column 32 dt + 8e' + 4hh + r: dK = scale * sum and dV
  //      directly when the pair has one segment, else fp32 partials in the
  //      pair's slots (NaN when a wait of the scoring pass gave up) ----
  if (j < 0) return;
  if (nseg == 1) {
    if (key >= p.nk) return;
    const float poison = *p.status ? NAN : 1.f;
    __bf16* dkr = p.dk + ((size_t)bk * p.nk + key) * D;
    __bf16* dvr = p.dv + ((size_t)bk * p.nk + key) * D;
#pragma unroll
    for (int d2 = 0; d2 < NDT; ++d2)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        bf16x4 tk, tv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          tk[r] = to_bf16(dkt[d2][4 * e4 + r] * p.scale * poison);
          tv[r] = to_bf16(dvt[d2][4 * e4 + r] * poison);
        }
        *(bf16x4*)(dkr + 32 * d2 + 8 * e4 + 4 * hh) = tk;
        *(bf16x4*)(dvr + 32 * d2 + 8 * e4 + 4 * hh) = tv;
      }
  } else {
    const int row = 32 * kh + l32;
    const int slot = p.segtab[(size_t)bk * p.tc + j] >> 5;
    float* pk = p.part + (((size_t)bk * kSlotsPerPair * p.npair + slot + seg) * 2 + sb) * 2 * 64 * D + row * D;
    float* pv = pk + 64 * D;
#pragma unroll
    for (int d2 = 0; d2 < NDT; ++d2)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int col = 32 * d2 + 8 * e4 + 4 * hh;
        *(float4*)(pk + col) = make_float4(dkt[d2][4 * e4], dkt[d2][4 * e4 + 1],
                                           dkt[d2][4 * e4 + 2], dkt[d2][4 * e4 + 3]);
        *(float4*)(pv + col) = make_float4(dvt[d2][4 * e4], dvt[d2][4 * e4 + 1],
                                           dvt[d2][4 * e4 + 2], dvt[d2][4 * e4 + 3]);
      }
  }
}

}  // namespace

template <int D, bool kTest, bool kStats>
hipError_t launch_bwd_kv(const BwdParams& p, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_kv_kernel<D, kTest, kStats>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

#define MALA_BWD_KV(D)                                                                   \
  template hipError_t launch_bwd_kv<D, true, true>(const BwdParams&, unsigned, hipStream_t);   \
  template hipError_t launch_bwd_kv<D, true, false>(const BwdParams&, unsigned, hipStream_t);  \
  template hipError_t launch_bwd_kv<D, false, true>(const BwdParams&, unsigned, hipStream_t);  \
  template hipError_t launch_bwd_kv<D, false, false>(const BwdParams&, unsigned, hipStream_t);
MALA_BWD_KV(64)
MALA_BWD_KV(128)
#undef MALA_BWD_KV

}  // namespace mala
