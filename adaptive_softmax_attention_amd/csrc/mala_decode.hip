// MALA split-KV decode ("MassAlloc Attention: Let Attention Allocate Its Own Compute":
// Sec. 2.4 and the decoding part of Appendix A.1) and the dense split-KV
// decode with the test compiled out.
//
// One new query per sequence sees all seqlen_k cached keys (L = seqlen_k,
// Sec. 2.1). The Tc key tiles are cut into S ranges of ceil(Tc/S) tiles; each
// (sequence, KV head, split) is an independent chain that starts with fresh
// (m, l), visits its tiles last-to-first and applies the forward rule to each
// query head of the group against its own partial normaliser. A second
// kernel merges the partial (m, l, u) with the identity of "Why exact
// attention does not need a quadratic matrix" (Method/Mechanism).
//
// Memory-bound design (gfx950):
//   * one wave64 per chain; the G query heads of the KV group share every K
//     and V tile read;
//   * K tiles go from HBM straight into MFMA A-operand registers (each lane
//     reads 64 contiguous bytes of 16 key rows per instruction, whole rows
//     over the tile), S^T = K q^T on 16x16x32 bf16 MFMA with the G heads in
//     the 16 columns; the next tile's K is requested as soon as the current
//     tile's MFMAs have consumed theirs;
//   * a V tile is read only if some head retains the tile; P V runs on the
//     vector ALUs in fp32 with fully coalesced 16-byte V loads (lanes own 8
//     columns of d and one phase of the keys), partial sums reduced once per
//     split.
#include "mala_common.h"
#include "mala_internal.h"

namespace mala {
namespace {

struct DecParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  float* part_m;
  float* part_l;
  float* part_u;
  int batch, heads_q, heads_kv, nk, group, splits, per, tc;
  int kk;   // 64-key tiles per decision tile (block_k / 64)
  int tcd;  // decision tiles of the longest cache (row length of the decision bitmap)
  float c;         // softmax_scale * log2(e)
  float thr;       // log2(tau / nk)
  float log2_tau;  // log2(tau); -inf for tau = 0
  // paged, variable-length cache (table == nullptr: one contiguous cache of
  // nk keys per sequence): K / V pages [num_pages][heads_kv][64][D]; the
  // keys 64 j .. 64 j + 63 of sequence b sit in page table[b * max_pages + j];
  // sequence b holds lens[b] keys (1 <= lens[b] <= nk)
  const int32_t* table;
  const int32_t* lens;
  int max_pages, num_pages;
  unsigned long long* counters;
  uint8_t* decisions;
};

template <int D, int GM, bool kTest, bool kStats, bool kBK2>
__global__ __launch_bounds__(64) void decode_split_kernel(DecParams p) {
  constexpr int NDC = D / 32;   // reduction chunks of d for the score MFMA
  constexpr int DG = D / 8;     // 8-column groups of d (P V lanes)
  constexpr int KPH = 64 / DG;  // key phases in P V
  constexpr int KT = 64 / KPH;  // keys per lane per tile in P V

  __shared__ float p_lds[64][GM];
  __shared__ float a_lds[GM];

  const int lane = threadIdx.x, l16 = lane & 15, g4 = lane >> 4;
  const int dg = lane % DG, kph = lane / DG;
  const int s = blockIdx.x % p.splits;
  const int bk = blockIdx.x / p.splits;  // b * heads_kv + kvh
  const int b = bk / p.heads_kv, kvh = bk % p.heads_kv;
  const int h0 = kvh * p.group;
  // this sequence's cache: its length, tiles, split range and tolerance
  // (L = its own length); a length or page outside the cache makes the
  // sequence's outputs NaN (no access outside the pages is made)
  int nk = p.nk, tc = p.tc, per = p.per;
  float thr = p.thr;
  bool bad = false;
  if (p.table) {
    nk = p.lens[b];
    bad = nk < 1 || nk > p.nk;
    nk = bad ? 0 : nk;
    tc = (nk + 63) / 64;
    // splits cut the sequence's own decision tiles
    per = p.kk * (((tc + p.kk - 1) / p.kk + p.splits - 1) / p.splits);
    thr = p.log2_tau - log2f((float)max(nk, 1));
  }
  const int j_lo = s * per;
  const int j_hi = min(tc, (s + 1) * per) - 1;
  const bool col_ok = l16 < p.group;  // this lane's MFMA column is a real head
  const size_t prow = (size_t)(b * p.heads_q + h0 + l16) * p.splits + s;

  float m2 = -INFINITY, lsum = 0.f;
  float acc[GM][8];
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  if (j_lo <= j_hi) {
    // row 0 of tile j of this sequence and KV head (nullptr: page out of range)
    auto tile_k = [&](const __bf16* base, int j) -> const __bf16* {
      if (!p.table) return base + ((size_t)bk * p.nk + (size_t)j * 64) * D;
      const int pg = p.table[(size_t)b * p.max_pages + j];
      if (pg < 0 || pg >= p.num_pages) return nullptr;
      return base + ((size_t)pg * p.heads_kv + kvh) * 64 * D;
    };
    // q^T as the B operand: column l16 = head h0 + l16
    bf16x8 qb[NDC];
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc)
      qb[dc] = col_ok ? *(const bf16x8*)(p.q + (size_t)(b * p.heads_q + h0 + l16) * D + 32 * dc + 8 * g4)
                      : bf16x8{};
    bf16x8 kr[4][NDC];
    auto load_k = [&](int j) {
      const __bf16* kt = tile_k(p.k, j);
      bad = bad || kt == nullptr;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int key = j * 64 + 16 * ks + l16;
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc)
          kr[ks][dc] = (kt && key < nk)
                           ? *(const bf16x8*)(kt + (size_t)(16 * ks + l16) * D + 32 * dc + 8 * g4)
                           : bf16x8{};
      }
    };
    load_k(j_hi);
    unsigned long long st_legal = 0, st_kept = 0, st_vtiles = 0;  // instrumentation
    // this head's maximum over a scored tile (raw units), keys past the end masked
    auto tile_max = [&](floatx4 (&sc)[4], int j) {
      float mt = -INFINITY;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = j * 64 + 16 * ks + 4 * g4 + r;
          if (key >= nk) sc[ks][r] = -INFINITY;
          mt = fmaxf(mt, sc[ks][r]);
        }
      return group4_max(mt);
    };
    // Eq. 3 for this head's single row, against the split's own (m, l)
    auto vote = [&](float mt) {
      if constexpr (kTest)
        return col_ok && (lsum == 0.f || !(mt * p.c - m2 - fast_log2(lsum) - thr < 0.f));
      else
        return col_ok;
    };
    // read V of tile j (some head retains it), update the retaining heads'
    // (m, l) and add P V for them
    auto apply = [&](floatx4 (&sc)[4], float mt, bool want, int j) {
      if (kStats) ++st_vtiles;
      bf16x8 vr[KT];
      const __bf16* vt = tile_k(p.v, j);
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const int key = j * 64 + kph + KPH * t;
        vr[t] = (vt && key < nk) ? *(const bf16x8*)(vt + (size_t)(kph + KPH * t) * D + 8 * dg)
                                 : bf16x8{};
      }
      // online-softmax update of the retaining heads
      float alpha = 1.f;
      if (want) {
        const float mn = fmaxf(m2, mt * p.c);
        alpha = fast_exp2(m2 - mn);
        float rs = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pv = fast_exp2(sc[ks][r] * p.c - mn);
            sc[ks][r] = pv;
            rs += pv;
          }
        rs = group4_sum(rs);
        lsum = alpha * lsum + rs;
        m2 = mn;
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) sc[ks] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      if (l16 < GM) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int r = 0; r < 4; ++r) p_lds[16 * ks + 4 * g4 + r][l16] = sc[ks][r];
        if (g4 == 0) a_lds[l16] = alpha;
      }
      lds_barrier();
      float al[GM];
#pragma unroll
      for (int h = 0; h < GM; ++h) al[h] = a_lds[h];
#pragma unroll
      for (int h = 0; h < GM; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= al[h];
      // u += P V over this lane's key phase
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const int key = kph + KPH * t;
        float pk[GM];
#pragma unroll
        for (int h = 0; h < GM; ++h) pk[h] = p_lds[key][h];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ve = (float)vr[t][e];
#pragma unroll
          for (int h = 0; h < GM; ++h) acc[h][e] += pk[h] * ve;
        }
      }
      lds_barrier();
    };
    // 128-key decision tiles are the pairs (2 jc + 1, 2 jc) of 64-key tiles,
    // visited upper first. A head that retains the upper tile under the
    // pair's state has retained the pair; a head whose vote passes only on
    // the lower tile (its state unchanged by the upper one) retains the pair
    // late: the upper tile is scored again from memory and applied after the
    // lower one (the online update is independent of the order).
    bool early = false;
    for (int j = j_hi; j >= j_lo; --j) {
      floatx4 sc[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        sc[ks] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) sc[ks] = mfma16x16x32(kr[ks][dc], qb[dc], sc[ks]);
      }
      if (j > j_lo) load_k(j - 1);  // next tile streams while this one is tested
      // lane holds keys 16ks + 4g4 + r of head column l16
      const float mt = tile_max(sc, j);
      const bool v = vote(mt);
      bool want = v, late = false, record = true;
      if constexpr (kBK2) {
        if (j & 1) {  // upper tile: decided with the lower one
          want = v;
          early = v;
          record = false;
        } else {
          want = early || v;
          late = !early && v && j + 1 <= j_hi;
          early = false;
        }
      }
      if (record && col_ok && g4 == 0) {
        if (kStats) {
          ++st_legal;
          if (want) ++st_kept;
        }
        if (kStats && p.decisions)
          p.decisions[(size_t)(b * p.heads_q + h0 + l16) * p.tcd + (kBK2 ? j / 2 : j)] = want ? 1 : 0;
      }
      if (wave_any(want)) apply(sc, mt, want, j);  // else no head retains: V never read
      if constexpr (kBK2) {
        if (wave_any(late)) {
          // score the upper tile again (its K straight from memory)
          const int jh = j + 1;
          const __bf16* kt = tile_k(p.k, jh);
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            sc[ks] = floatx4{0.f, 0.f, 0.f, 0.f};
            const int key = jh * 64 + 16 * ks + l16;
#pragma unroll
            for (int dc = 0; dc < NDC; ++dc) {
              const bf16x8 kk = (kt && key < nk)
                                    ? *(const bf16x8*)(kt + (size_t)(16 * ks + l16) * D + 32 * dc + 8 * g4)
                                    : bf16x8{};
              sc[ks] = mfma16x16x32(kk, qb[dc], sc[ks]);
            }
          }
          const float mh = tile_max(sc, jh);
          apply(sc, mh, late, jh);
        }
      }
    }
    if (kStats && p.counters) {
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        st_legal += __shfl_xor(st_legal, off);
        st_kept += __shfl_xor(st_kept, off);
      }
      if (lane == 0) {
        atomicAdd(&p.counters[0], st_legal);
        atomicAdd(&p.counters[1], st_kept);
        atomicAdd(&p.counters[2], 64ull * p.kk * st_kept);
        atomicAdd(&p.counters[3], st_vtiles);
      }
    }
  }
  // reduce the key phases, then write this split's partial (m, l, u)
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[h][e];
#pragma unroll
      for (int off = DG; off < 64; off <<= 1) x += __shfl_xor(x, off);
      acc[h][e] = x;
    }
  if (col_ok && g4 == 0) {
    p.part_m[prow] = m2;
    p.part_l[prow] = bad ? NAN : lsum;
  }
  if (kph == 0) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < p.group) {
        float* u = p.part_u + ((size_t)(b * p.heads_q + h0 + h) * p.splits + s) * D + 8 * dg;
        *(float4*)u = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        *(float4*)(u + 4) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
      }
    }
  }
}

// Normaliser-aware merge of the S partial (m, l, u) of one query head
// (splits with l = 0 retained nothing and are left out).
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecParams p) {
  const int row = blockIdx.x;  // b * heads_q + h
  const int t = threadIdx.x;
  const float* m = p.part_m + (size_t)row * p.splits;
  const float* l = p.part_l + (size_t)row * p.splits;
  float M = -INFINITY;
  bool bad = false;  // a split met a length or page outside the cache
  for (int s = 0; s < p.splits; ++s) {
    if (l[s] > 0.f) M = fmaxf(M, m[s]);
    bad = bad || isnan(l[s]);
  }
  float lt = 0.f, u = 0.f;
  for (int s = 0; s < p.splits; ++s) {
    if (!(l[s] > 0.f)) continue;
    const float w = fast_exp2(m[s] - M);
    lt += w * l[s];
    u += w * p.part_u[((size_t)row * p.splits + s) * D + t];
  }
  p.o[(size_t)row * D + t] = to_bf16(bad ? NAN : u / lt);
  if (t == 0) p.lse[row] = bad ? NAN : (M + log2f(lt)) * kLn2;
}

template <int D, int GM>
hipError_t launch_d(const DecParams& p, bool test, hipStream_t stream) {
  dim3 grid((unsigned)(p.batch * p.heads_kv * p.splits)), block(64);
  const bool st = p.counters != nullptr || p.decisions != nullptr;
  // 128-key decisions matter to the test and to the recorded decisions; the
  // dense path without instrumentation computes the same either way
  const bool bk2 = p.kk == 2;
  if (test && st && bk2)
    hipLaunchKernelGGL((decode_split_kernel<D, GM, true, true, true>), grid, block, 0, stream, p);
  else if (test && st)
    hipLaunchKernelGGL((decode_split_kernel<D, GM, true, true, false>), grid, block, 0, stream, p);
  else if (test && bk2)
    hipLaunchKernelGGL((decode_split_kernel<D, GM, true, false, true>), grid, block, 0, stream, p);
  else if (test)
    hipLaunchKernelGGL((decode_split_kernel<D, GM, true, false, false>), grid, block, 0, stream, p);
  else if (st && bk2)
    hipLaunchKernelGGL((decode_split_kernel<D, GM, false, true, true>), grid, block, 0, stream, p);
  else if (st)
    hipLaunchKernelGGL((decode_split_kernel<D, GM, false, true, false>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, GM, false, false, false>), grid, block, 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(p.batch * p.heads_q), dim3(D), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dg(const DecParams& p, bool test, hipStream_t stream) {
  if (p.group <= 1) return launch_d<D, 1>(p, test, stream);
  if (p.group <= 2) return launch_d<D, 2>(p, test, stream);
  if (p.group <= 4) return launch_d<D, 4>(p, test, stream);
  return launch_d<D, 8>(p, test, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, bool test, hipStream_t stream) {
  DecParams p;
  p.q = (const __bf16*)a.q;
  p.k = (const __bf16*)a.k;
  p.v = (const __bf16*)a.v;
  p.o = (__bf16*)a.o;
  p.lse = a.lse;
  p.part_m = a.part_m;
  p.part_l = a.part_l;
  p.part_u = a.part_u;
  p.batch = a.batch;
  p.heads_q = a.heads_q;
  p.heads_kv = a.heads_kv;
  p.nk = a.nk;
  p.group = a.heads_q / a.heads_kv;
  p.splits = a.num_splits;
  p.tc = (a.nk + 63) / 64;
  p.kk = a.block_k / 64;
  p.tcd = (a.nk + a.block_k - 1) / a.block_k;
  // splits cut the decision tiles: ceil(tcd / S) of them, in 64-key tiles
  p.per = p.kk * ((p.tcd + a.num_splits - 1) / a.num_splits);
  p.c = a.scale * kLog2e;
  const float log2_tau = a.tau == 0.f ? -INFINITY : log2f(a.tau);
  p.thr = log2_tau - log2f((float)a.nk);
  p.log2_tau = log2_tau;
  p.table = a.block_table;
  p.lens = a.cache_lens;
  p.max_pages = p.tc;
  p.num_pages = a.num_pages;
  p.counters = a.counters;
  p.decisions = a.decisions;
  if (p.group > 8) return hipErrorNotSupported;
  return a.head_dim == 128 ? launch_dg<128>(p, test, stream) : launch_dg<64>(p, test, stream);
}

}  // namespace mala
