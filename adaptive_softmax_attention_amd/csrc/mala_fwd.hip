// MALA fused forward ("MassAlloc Attention: Let Attention Allocate Its Own Compute":
// Sec. 2.2 Eqs. 1-3, Appendix A Algorithm 1, and the forward part of
// Appendix A.1) and the dense FullAttn forward
// from the same template with the test compiled out.
//
// Work decomposition (gfx950):
//   * a pair of wave64s owns one 64-row decision block (query block i of
//     head h), 32 rows each; each wave ballots its rows and the pair's two
//     bits are combined through LDS at the barrier that already separates
//     score discovery from the V load, so the test of Eq. 3 costs no extra
//     synchronisation;
//   * a workgroup of 8 waves holds 4 blocks that share K/V tiles: 4 query
//     heads of one KV head (GQA), or 2 heads x 2 blocks, or 4 consecutive
//     query blocks of one head;
//   * scores are formed transposed, S^T = K Q^T (16x16x32 bf16 MFMA, fp32
//     accumulate), so each lane holds 16 keys of one query column: the row
//     max and row sum need only 2 cross-lane steps, and P^T is already in
//     the B-operand layout of O^T = V^T P^T;
//   * K and V tiles are copied asynchronously from global memory straight
//     into LDS rings (global_load_lds, row-major, swizzled); V^T operands are
//     read with the transposing LDS read, so nothing is staged in registers;
//   * software pipeline over the key blocks, visited from the diagonal down
//     (Sec. 2.2): K runs two tiles ahead; a tile's V is requested only after
//     the ballot says some block retains it, and is consumed one iteration
//     later: the running (m, l) update of a tile needs only its scores, so
//     the next tile's score discovery proceeds while V is in flight, and
//     O <- alpha O + P V is applied a step late in the same order;
//   * workgroups are issued longest-first (largest query block first).
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
  float c;         // softmax_scale * log2(e): raw score -> log2 units
  float log2_tau;  // log2(tau); -inf for tau = 0, +inf for tau = inf
  int group;       // heads_q / heads_kv
  int hpw, ipw;    // heads x query blocks per workgroup, hpw * ipw = 4
  int n_hg, n_ig;  // head groups per KV head, query-block groups
  int tr, tc;      // query / key tile counts
  unsigned long long* counters;
  uint8_t* decisions;
};

template <int D, bool kTest, bool kStats>
__global__ __launch_bounds__(512, 1) void fwd_kernel(FwdParams p) {
  constexpr int NDC = D / 32;         // 32-wide reduction chunks over d
  constexpr int NDS = D / 16;         // 16-row subtiles of O^T over d
  constexpr int KCH = D / 8;          // 16-byte chunks per K / V row
  constexpr int NT = 512;             // threads per workgroup
  constexpr int NQS = 2;              // 16-query subtiles per wave (32 rows)
  constexpr int CPT = 64 * KCH / NT;  // async 16-byte copies per thread per tile
  constexpr int RK = 3;               // K ring: current tile + 2 ahead
  constexpr int RV = 2;               // V ring

  __shared__ __attribute__((aligned(16))) __bf16 k_ring[RK][64 * D];
  __shared__ __attribute__((aligned(16))) __bf16 v_ring[RV][64 * D];
  __shared__ int flags[8];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;

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
  const int q0 = i * 64 + 32 * half;  // first row of this wave
  const int bq0 = i * 64;             // first row of the block
  const int jmax = valid ? (p.causal ? i : p.tc - 1) : -1;
  const int i_top = min(ig * p.ipw + p.ipw - 1, p.tr - 1);
  const int jtop = p.causal ? i_top : p.tc - 1;
  const int vrows = valid ? min(64, p.nq - bq0) : 0;

  const size_t qrow0 = (size_t)(b * p.heads_q + h) * p.nq;
  const __bf16* kbase = p.k + (size_t)(b * p.heads_kv + kvh) * p.nk * D;
  const __bf16* vbase = p.v + (size_t)(b * p.heads_kv + kvh) * p.nk * D;

  // ---- Q block in registers: B operand of S^T = K Q^T ----
  bf16x8 qr[NQS][NDC];
#pragma unroll
  for (int qs = 0; qs < NQS; ++qs) {
    const int qq = q0 + 16 * qs + l16;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      if (valid && qq < p.nq)
        qr[qs][dc] = *(const bf16x8*)(p.q + (qrow0 + qq) * D + 32 * dc + 8 * g4);
      else
        qr[qs][dc] = bf16x8{};
    }
  }

  // ---- running state per query column of this lane ----
  float m2[NQS], lsum[NQS], thr[NQS];
  floatx4 oacc[NDS][NQS];
#pragma unroll
  for (int qs = 0; qs < NQS; ++qs) {
    const int qq = q0 + 16 * qs + l16;
    m2[qs] = -INFINITY;
    lsum[qs] = 0.f;
    const float L = p.causal ? (float)(qq + 1) : (float)p.nk;  // visible keys
    thr[qs] = p.log2_tau - log2f(L);                            // log2(tau / L_q)
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) oacc[ds][qs] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- async tile copies (rows past the end re-read the last row; those
  //      keys are masked, so only finite values reach the products) ----
  auto issue_tile = [&](const __bf16* base, int j, __bf16* slot, bool tr_layout) {
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      const int s0 = x * NT + w * 64;  // first 16-byte slot of this wave
      const int s = s0 + lane;
      const int row = s / KCH, pc = s % KCH;
      const int sw = tr_layout ? (tr_swz(row) & (KCH - 1)) : (k_swz(row) & (KCH - 1));
      const int key = min(j * 64 + row, p.nk - 1);
      async_copy16(base + (size_t)key * D + (pc ^ sw) * 8, slot + s0 * 8);
    }
  };

  // pending post-score work of the previous tile (applied one step late)
  bool pend = false;
  bf16x8 pend_pb[2][NQS];
  float pend_alpha[NQS];
  bool v_prev = false;  // V of the previous tile was requested

  auto apply_pv = [&](const __bf16* vt) {
    // O^T <- alpha O^T + V^T P^T
#pragma unroll
    for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        oacc[ds][qs][0] *= pend_alpha[qs];
        oacc[ds][qs][1] *= pend_alpha[qs];
        oacc[ds][qs][2] *= pend_alpha[qs];
        oacc[ds][qs][3] *= pend_alpha[qs];
      }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        // lane addresses row k0 + l16/4, columns 16ds + 4(l16%4): the
        // transposing read returns V[k0 + e][16ds + l16], e = 0..3
        short4v t[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int row = 32 * kc + 8 * g4 + 4 * hh + (l16 >> 2);
          const int col = 16 * ds + 4 * (l16 & 3);
          const int ch = col >> 3;
          t[hh] = lds_read_tr4(vt + row * D + ((ch ^ (tr_swz(row) & (KCH - 1))) * 8) + (col & 7));
        }
        const bf16x8 a = join_tr(t[0], t[1]);
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs)
          oacc[ds][qs] = mfma16x16x32(a, pend_pb[kc][qs], oacc[ds][qs]);
      }
  };

  // prologue: K of the first two tiles
  issue_tile(kbase, jtop, k_ring[jtop % RK], false);
  if (jtop >= 1) issue_tile(kbase, jtop - 1, k_ring[(jtop - 1) % RK], false);

  for (int j = jtop; j >= 0; --j) {
    // K_j complete; V_{j+1} and K_{j-1} may still be in flight
    vmcnt_wait_le((v_prev ? CPT : 0) + (j >= 1 ? CPT : 0));
    lds_barrier();
    const __bf16* kt = k_ring[j % RK];

    const bool part = valid && j <= jmax;
    bool want = false;
    floatx4 s[4][NQS];
    float mt[NQS];
    if (part) {
      // score discovery, every legal tile
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) s[ks][qs] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          // MFMA row l16 of key subtile ks holds key 32(ks/2)+8(l16/4)+4(ks%2)+l16%4,
          // so output lane group g4 ends up with 8 consecutive keys per 32
          const int kr = 32 * (ks >> 1) + 8 * (l16 >> 2) + 4 * (ks & 1) + (l16 & 3);
          const int ch = 4 * dc + g4;
          const bf16x8 a = *(const bf16x8*)(kt + kr * D + ((ch ^ (k_swz(kr) & (KCH - 1))) * 8));
#pragma unroll
          for (int qs = 0; qs < NQS; ++qs) s[ks][qs] = mfma16x16x32(a, qr[qs][dc], s[ks][qs]);
        }
      }
      // causal mask at the diagonal and the ragged key tail
      const bool need_mask = (p.causal && j == i) || (j * 64 + 63 >= p.nk);
      if (need_mask) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = j * 64 + 32 * (ks >> 1) + 8 * g4 + 4 * (ks & 1) + r;
              const int qq = q0 + 16 * qs + l16;
              if (key >= p.nk || (p.causal && key > qq)) s[ks][qs][r] = -INFINITY;
            }
      }
      // tile row maxima
#pragma unroll
      for (int qs = 0; qs < NQS; ++qs) {
        float x = -INFINITY;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int r = 0; r < 4; ++r) x = fmaxf(x, s[ks][qs][r]);
        mt[qs] = group4_max(x);
      }
      if constexpr (kTest) {
        // Eq. 3 in log2 units: skip iff every valid row with a legal key has
        // rowmax*c - m - log2(l) < log2(tau/L); l = 0 counts as +inf
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) {
          const int qq = q0 + 16 * qs + l16;
          if (qq < p.nq && mt[qs] != -INFINITY) {
            if (lsum[qs] == 0.f) {
              want = true;
            } else {
              const float mg = mt[qs] * p.c - m2[qs] - fast_log2(lsum[qs]) - thr[qs];
              if (!(mg < 0.f)) want = true;
            }
          }
        }
        want = wave_any(want);
      } else {
        want = true;
      }
    }
    if (lane == 0) flags[w] = want ? 1 : 0;
    // V_{j+1} complete (K_{j-1} may stay in flight); flags visible
    if (v_prev) vmcnt_wait_le(j >= 1 ? CPT : 0);
    lds_barrier();
    // block decision = either half wants it; V is needed if any block retains
    const bool retain = part && (flags[2 * blk] | flags[2 * blk + 1]) != 0;
    int anyf = 0;
#pragma unroll
    for (int x = 0; x < 8; ++x) anyf |= flags[x];
    if (part && half == 0 && lane == 0) {
      if (kStats && p.counters) {
        atomicAdd(&p.counters[0], 1ull);
        if (retain) {
          atomicAdd(&p.counters[1], 1ull);
          atomicAdd(&p.counters[2], (unsigned long long)vrows * 64ull);
        }
      }
      if (kStats && p.decisions)
        p.decisions[((size_t)(b * p.heads_q + h) * p.tr + i) * p.tc + j] = retain ? 1 : 0;
    }
    // the previous tile's P V (its V arrived during this tile's scoring)
    if (pend) apply_pv(v_ring[(j + 1) % RV]);
    // request V_j only if some block retains tile j (skipped tiles never
    // touch V), then K two tiles ahead
    if (anyf) {
      issue_tile(vbase, j, v_ring[j % RV], true);
      if (kStats && tid == 0 && p.counters) atomicAdd(&p.counters[3], 1ull);
    }
    if (j >= 2) issue_tile(kbase, j - 2, k_ring[(j - 2) % RK], false);
    v_prev = anyf != 0;

    pend = retain;
    if (retain) {
      // online-softmax update of every valid row; the
      // O update for this tile is applied next iteration
#pragma unroll
      for (int qs = 0; qs < NQS; ++qs) {
        const float mn = fmaxf(m2[qs], mt[qs] * p.c);
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = fast_exp2(m2[qs] - mu);
        float rs = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pv = fast_exp2(s[ks][qs][r] * p.c - mu);
            s[ks][qs][r] = pv;
            rs += pv;
          }
        rs = group4_sum(rs);
        lsum[qs] = alpha * lsum[qs] + rs;
        m2[qs] = mn;
        pend_alpha[qs] = alpha;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          bf16x8 t;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            t[r] = to_bf16(s[2 * kc][qs][r]);
            t[4 + r] = to_bf16(s[2 * kc + 1][qs][r]);
          }
          pend_pb[kc][qs] = t;
        }
      }
    }
  }
  // the last tile's P V
  vmcnt_wait<0>();
  lds_barrier();
  if (pend) apply_pv(v_ring[0]);

  // ---- finalisation: O = O / l, LSE = m + log l ----
  if (valid) {
#pragma unroll
    for (int qs = 0; qs < NQS; ++qs) {
      const int qq = q0 + 16 * qs + l16;
      if (qq >= p.nq) continue;
      const float inv = 1.f / lsum[qs];
      __bf16* orow = p.o + (qrow0 + qq) * D;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        bf16x4 t;
        t[0] = to_bf16(oacc[ds][qs][0] * inv);
        t[1] = to_bf16(oacc[ds][qs][1] * inv);
        t[2] = to_bf16(oacc[ds][qs][2] * inv);
        t[3] = to_bf16(oacc[ds][qs][3] * inv);
        *(bf16x4*)(orow + 16 * ds + 4 * g4) = t;
      }
      if (g4 == 0) p.lse[qrow0 + qq] = (m2[qs] + log2f(lsum[qs])) * kLn2;
    }
  }
}

}  // namespace

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
  p.c = a.scale * kLog2e;
  p.log2_tau = a.tau == 0.f ? -INFINITY : log2f(a.tau);
  p.group = a.heads_q / a.heads_kv;
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
  p.tr = (a.nq + 63) / 64;
  p.tc = (a.nk + 63) / 64;
  p.n_hg = p.group / p.hpw;
  p.n_ig = (p.tr + p.ipw - 1) / p.ipw;
  p.counters = a.counters;
  p.decisions = a.decisions;
  const long long nblocks = (long long)p.n_ig * p.batch * p.heads_kv * p.n_hg;
  dim3 grid((unsigned)nblocks), block(512);
  // the instrumented variant is a separate instantiation, so the timed
  // kernel carries no counter code
  const bool st = p.counters != nullptr || p.decisions != nullptr;
  if (a.head_dim == 128) {
    if (test && st)
      hipLaunchKernelGGL((fwd_kernel<128, true, true>), grid, block, 0, stream, p);
    else if (test)
      hipLaunchKernelGGL((fwd_kernel<128, true, false>), grid, block, 0, stream, p);
    else if (st)
      hipLaunchKernelGGL((fwd_kernel<128, false, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_kernel<128, false, false>), grid, block, 0, stream, p);
  } else {
    if (test && st)
      hipLaunchKernelGGL((fwd_kernel<64, true, true>), grid, block, 0, stream, p);
    else if (test)
      hipLaunchKernelGGL((fwd_kernel<64, true, false>), grid, block, 0, stream, p);
    else if (st)
      hipLaunchKernelGGL((fwd_kernel<64, false, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_kernel<64, false, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mala
