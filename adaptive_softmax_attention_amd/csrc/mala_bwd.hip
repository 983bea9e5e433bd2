// MALA fused backward ("MassAlloc Attention: Let Attention Allocate Its Own Compute":
// Sec. 2.2 Eq. 4, Appendix A Algorithm 2, and the backward part of
// Appendix A.1) and the dense FullAttn backward
// from the same template with the test compiled out.
//
// Three kernels on the caller's stream:
//   1. bwd_pre:  D_q = rowsum(O o dO) in fp32 (from the
//                stored O) and a zero fill of the fp32 dQ accumulator (a fill
//                kernel rather than a memset, so the sequence can be captured
//                in a graph);
//   2. bwd_main: key-major traversal. A workgroup of 8 wave64s owns a pair of
//                64-key blocks (j0 = 2J, j1 = 2J + 1) of one KV head; each wave
//                owns a 16-key slice and keeps its dK, dV accumulators in
//                registers. It visits the G query heads of the group and the
//                query blocks from the diagonal up. Per tile:
//                S = Q K^T is recomputed (16x16x32 bf16 MFMA), the offline test
//                of Eq. 4 compares every legal s - z_q with log(tau/L_q) against
//                the forward's LSE (wave ballot, OR over the block's 4 waves at
//                the barrier that precedes the dO load); only a retained tile
//                loads dO and runs P = exp(s - z), dP = dO V^T,
//                dS = P o (dP - D), dV += P^T dO, dK += dS^T Q and
//                dQ += dS K. P and dS come out of the score MFMA already in the
//                A-operand layout of the dV / dK products; dS goes through LDS
//                so dQ contracts over both key blocks (128 keys) before the
//                fp32 atomic add into the accumulator;
//   3. bwd_dq:   dQ = bf16(scale * accumulator).
// Q and dO tiles are staged in LDS twice, row-major for the products that
// contract over d and transposed for those that contract over queries.
#include "mala_common.h"
#include "mala_internal.h"

namespace mala {
namespace {

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
  float* delta;
  float* dq_accum;
  int batch, heads_q, heads_kv, nq, nk, group;
  int causal;
  float scale;
  float c;         // scale * log2(e)
  float log2_tau;  // log2(tau); -inf for tau = 0, +inf for tau = inf
  int tr, tc, npair;
  unsigned long long* counters;
  uint8_t* decisions;
};

// ---------------------------------------------------------------- pre ----
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int LPR = D / 8;  // lanes per row (8 values each)
  const long long rows = (long long)p.batch * p.heads_q * p.nq;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = t / LPR;
  const int part = (int)(t % LPR);
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 a = *(const bf16x8*)(p.o + row * D + 8 * part);
    const bf16x8 b = *(const bf16x8*)(p.dout + row * D + 8 * part);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
    float* z = p.dq_accum + row * D + 8 * part;
    *(float4*)z = make_float4(0.f, 0.f, 0.f, 0.f);
    *(float4*)(z + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) p.delta[row] = acc;
}

// ---------------------------------------------------------------- dq -----
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdParams p) {
  const long long n = (long long)p.batch * p.heads_q * p.nq * D / 8;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const float4 a = *(const float4*)(p.dq_accum + 8 * t);
  const float4 b = *(const float4*)(p.dq_accum + 8 * t + 4);
  bf16x8 r;
  r[0] = to_bf16(a.x * p.scale);
  r[1] = to_bf16(a.y * p.scale);
  r[2] = to_bf16(a.z * p.scale);
  r[3] = to_bf16(a.w * p.scale);
  r[4] = to_bf16(b.x * p.scale);
  r[5] = to_bf16(b.y * p.scale);
  r[6] = to_bf16(b.z * p.scale);
  r[7] = to_bf16(b.w * p.scale);
  *(bf16x8*)(p.dq + 8 * t) = r;
}

// --------------------------------------------------------------- main ----
// LDS layouts (bf16): row-major tiles use 16-byte chunks XOR-swizzled by
// k_swz(row); transposed tiles [d][rows] use v_swz(d) on 128-byte rows, and
// the 256-byte-row tiles (K^T over 128 keys, dS over 128 keys) use ds_swz.
__device__ __forceinline__ int ds_swz(int row) { return (row & 7) ^ ((row >> 3) & 7); }

template <int D, bool kTest>
__global__ __launch_bounds__(512, 1) void bwd_main_kernel(BwdParams p) {
  constexpr int NT = 512;
  constexpr int NDC = D / 32;       // reduction chunks over d
  constexpr int NDS = D / 16;       // 16-column subtiles of d
  constexpr int KCH = D / 8;        // 16-byte chunks per row of d
  constexpr int QPT = 64 * KCH / NT;   // Q / dO rows staged per thread (2 or 1)
  constexpr int KTPT = 128 * KCH / NT;  // K rows staged per thread for K^T (4 or 2)
  constexpr int DQS = NDS / 2;      // d subtiles per wave in the dQ product

  __shared__ __attribute__((aligned(16))) __bf16 q_lds[64 * D];
  __shared__ __attribute__((aligned(16))) __bf16 qt_lds[D * 64];
  __shared__ __attribute__((aligned(16))) __bf16 do_lds[64 * D];
  __shared__ __attribute__((aligned(16))) __bf16 dot_lds[D * 64];
  __shared__ __attribute__((aligned(16))) __bf16 kt_lds[D * 128];
  __shared__ __attribute__((aligned(16))) __bf16 ds_lds[64 * 128];
  __shared__ __attribute__((aligned(16))) float z_lds[64];
  __shared__ __attribute__((aligned(16))) float t_lds[64];
  __shared__ __attribute__((aligned(16))) float d_lds[64];
  __shared__ int flags[8];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int kb = w >> 2, kw = w & 3;

  // ---- work item: key-block pair J of (b, kvh), longest first ----
  const int per = p.batch * p.heads_kv;
  const int J = (int)(blockIdx.x / per);
  const int bk = (int)(blockIdx.x % per);
  const int b = bk / p.heads_kv, kvh = bk % p.heads_kv;
  const int j0 = 2 * J;
  const int jw = j0 + kb;                 // this wave's key block
  const int key = 64 * jw + 16 * kw + l16;  // this lane's key (score column)
  const bool kb_valid = jw < p.tc;
  const __bf16* kbase = p.k + (size_t)bk * p.nk * D;
  const __bf16* vbase = p.v + (size_t)bk * p.nk * D;

  // K and V of this lane's key as B operands (fixed for the workgroup)
  bf16x8 kreg[NDC], vreg[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) {
    const bool ok = key < p.nk;
    kreg[dc] = ok ? *(const bf16x8*)(kbase + (size_t)key * D + 32 * dc + 8 * g4) : bf16x8{};
    vreg[dc] = ok ? *(const bf16x8*)(vbase + (size_t)key * D + 32 * dc + 8 * g4) : bf16x8{};
  }
  // K^T of both key blocks into LDS for the dQ product
  {
    const int ch = tid % KCH, kg = tid / KCH;
    bf16x8 kr[KTPT];
#pragma unroll
    for (int x = 0; x < KTPT; ++x) {
      const int kk = 64 * j0 + kg * KTPT + x;
      kr[x] = kk < p.nk ? *(const bf16x8*)(kbase + (size_t)kk * D + 8 * ch) : bf16x8{};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * ch + e;
      const int k0 = kg * KTPT;
      __bf16* dst = kt_lds + d * 128 + (((k0 >> 3) ^ (d & 15)) * 8) + (k0 & 7);
      if constexpr (KTPT == 4) {
        bf16x4 t4;
        t4[0] = kr[0][e];
        t4[1] = kr[1][e];
        t4[2] = kr[2][e];
        t4[3] = kr[3][e];
        *(bf16x4*)dst = t4;
      } else {
        typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
        bf16x2 t2;
        t2[0] = kr[0][e];
        t2[1] = kr[1][e];
        *(bf16x2*)dst = t2;
      }
    }
  }

  floatx4 dk_acc[NDS], dv_acc[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    dk_acc[ds] = floatx4{0.f, 0.f, 0.f, 0.f};
    dv_acc[ds] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- Q / dO staging: thread owns QPT rows x 8 columns of d ----
  const int sch = tid % KCH, sg = tid / KCH;  // column chunk, row group
  auto load_rows = [&](const __bf16* base, int i, bf16x8 (&r)[QPT]) {
#pragma unroll
    for (int x = 0; x < QPT; ++x) {
      const int qq = 64 * i + sg * QPT + x;
      r[x] = qq < p.nq ? *(const bf16x8*)(base + (size_t)qq * D + 8 * sch) : bf16x8{};
    }
  };
  auto store_rows = [&](const bf16x8 (&r)[QPT], __bf16* nat, __bf16* tr) {
#pragma unroll
    for (int x = 0; x < QPT; ++x) {
      const int row = sg * QPT + x;
      *(bf16x8*)(nat + row * D + ((sch ^ (k_swz(row) & (KCH - 1))) * 8)) = r[x];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * sch + e;
      const int r0 = sg * QPT;
      __bf16* dst = tr + d * 64 + (((r0 >> 3) ^ v_swz(d)) * 8) + (r0 & 7);
      if constexpr (QPT == 2) {
        typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
        bf16x2 t2;
        t2[0] = r[0][e];
        t2[1] = r[1][e];
        *(bf16x2*)dst = t2;
      } else {
        *dst = r[0][e];
      }
    }
  };

  const int i_first = p.causal ? j0 : 0;
  const int n_i = p.tr - i_first;
  const int n_items = n_i > 0 ? p.group * n_i : 0;
  // Q rows and the LSE of the next item are prefetched into registers one
  // item ahead (the LDS-only barriers leave those loads in flight)
  bf16x8 qreg[QPT];
  float lreg = 0.f;
  auto load_lse = [&](int h, int i) {
    const int qq = 64 * i + tid;
    lreg = (tid < 64 && qq < p.nq) ? p.lse[(size_t)(b * p.heads_q + h) * p.nq + qq] : 0.f;
  };
  if (n_items > 0) {
    const int h = kvh * p.group;
    load_rows(p.q + (size_t)(b * p.heads_q + h) * p.nq * D, i_first, qreg);
    load_lse(h, i_first);
  }

  for (int it = 0; it < n_items; ++it) {
    const int hh = it / n_i;
    const int i = i_first + it % n_i;
    const int h = kvh * p.group + hh;
    const size_t row0 = (size_t)(b * p.heads_q + h) * p.nq;

    lds_barrier();  // previous item's LDS reads complete
    store_rows(qreg, q_lds, qt_lds);
    if (tid < 64) {
      const int qq = 64 * i + tid;
      z_lds[tid] = lreg * kLog2e;
      const float L = p.causal ? (float)(qq + 1) : (float)p.nk;
      t_lds[tid] = p.log2_tau - log2f(L);  // log2(tau / L_q)
    }
    lds_barrier();  // Q_i, z, thresholds visible
    if (it + 1 < n_items) {
      const int hn = kvh * p.group + (it + 1) / n_i;
      const int in = i_first + (it + 1) % n_i;
      load_rows(p.q + (size_t)(b * p.heads_q + hn) * p.nq * D, in, qreg);
      load_lse(hn, in);
    }

    const bool part = kb_valid && (!p.causal || i >= jw);
    bool want = false;
    floatx4 s[4];
    if (part) {
      // S = Q_i K_j^T recomputed; MFMA row R of query
      // subtile qs holds query 32(qs/2) + 8(R/4) + 4(qs%2) + R%4
#pragma unroll
      for (int qs = 0; qs < 4; ++qs) s[qs] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
        for (int qs = 0; qs < 4; ++qs) {
          const int qr = 32 * (qs >> 1) + 8 * (l16 >> 2) + 4 * (qs & 1) + (l16 & 3);
          const int ch = 4 * dc + g4;
          const bf16x8 a = *(const bf16x8*)(q_lds + qr * D + ((ch ^ (k_swz(qr) & (KCH - 1))) * 8));
          s[qs] = mfma16x16x32(a, kreg[dc], s[qs]);
        }
      }
      // legality and the offline test of Eq. 4 (log2 units)
#pragma unroll
      for (int qs = 0; qs < 4; ++qs) {
        const int ql = 32 * (qs >> 1) + 8 * g4 + 4 * (qs & 1);  // first of 4 queries
        const float4 z4 = *(const float4*)(z_lds + ql);
        const float4 t4 = *(const float4*)(t_lds + ql);
        const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
        const float tt[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qq = 64 * i + ql + r;
          const bool legal = qq < p.nq && key < p.nk && (!p.causal || key <= qq);
          const float x = s[qs][r] * p.c - zz[r];  // log2 P
          s[qs][r] = legal ? x : -INFINITY;
          if constexpr (kTest) {
            if (legal && !(x < tt[r])) want = true;
          } else {
            if (legal) want = true;
          }
        }
      }
      want = wave_any(want);
    }
    if (lane == 0) flags[w] = want ? 1 : 0;
    lds_barrier();
    const bool ret0 = (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
    const bool ret1 = (flags[4] | flags[5] | flags[6] | flags[7]) != 0;
    const bool retain = part && (kb == 0 ? ret0 : ret1);
    if (kw == 0 && lane == 0 && part) {
      if (p.counters) {
        atomicAdd(&p.counters[0], 1ull);
        if (retain) {
          atomicAdd(&p.counters[1], 1ull);
          atomicAdd(&p.counters[2], (unsigned long long)min(64, p.nq - 64 * i) * 64ull);
        }
      }
      if (p.decisions)
        p.decisions[((size_t)(b * p.heads_q + h) * p.tr + i) * p.tc + jw] = retain ? 1 : 0;
    }
    if (!ret0 && !ret1) continue;  // both tiles skipped: dO never loaded

    // ---- retained: dO_i and D_i ----
    bf16x8 doreg[QPT];
    load_rows(p.dout + row0 * D, i, doreg);
    if (tid == 0 && p.counters) atomicAdd(&p.counters[3], 1ull);
    if (tid < 64) {
      const int qq = 64 * i + tid;
      d_lds[tid] = qq < p.nq ? p.delta[row0 + qq] : 0.f;
    }
    if (retain) {
#pragma unroll
      for (int qs = 0; qs < 4; ++qs)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[qs][r] = fast_exp2(s[qs][r]);  // P
    }
    store_rows(doreg, do_lds, dot_lds);
    lds_barrier();  // dO_i, dO_i^T, D_i visible

    if (retain) {
      // dP = dO V^T, same layout as S
      floatx4 dp[4];
#pragma unroll
      for (int qs = 0; qs < 4; ++qs) dp[qs] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
        for (int qs = 0; qs < 4; ++qs) {
          const int qr = 32 * (qs >> 1) + 8 * (l16 >> 2) + 4 * (qs & 1) + (l16 & 3);
          const int ch = 4 * dc + g4;
          const bf16x8 a = *(const bf16x8*)(do_lds + qr * D + ((ch ^ (k_swz(qr) & (KCH - 1))) * 8));
          dp[qs] = mfma16x16x32(a, vreg[dc], dp[qs]);
        }
      }
      // dS = P o (dP - D); pack P^T and dS^T as A operands
      bf16x8 pt[2], dst[2];
#pragma unroll
      for (int qs = 0; qs < 4; ++qs) {
        const int ql = 32 * (qs >> 1) + 8 * g4 + 4 * (qs & 1);
        const float4 d4 = *(const float4*)(d_lds + ql);
        const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = s[qs][r];
          const float dsv = pv * (dp[qs][r] - dd[r]);
          pt[qs >> 1][4 * (qs & 1) + r] = to_bf16(pv);
          dst[qs >> 1][4 * (qs & 1) + r] = to_bf16(dsv);
        }
      }
      // dV += P^T dO, dK += dS^T Q
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          const int d = 16 * ds + l16;
          const int ch = 4 * kc + g4;
          const bf16x8 bo = *(const bf16x8*)(dot_lds + d * 64 + ((ch ^ v_swz(d)) * 8));
          const bf16x8 bq = *(const bf16x8*)(qt_lds + d * 64 + ((ch ^ v_swz(d)) * 8));
          dv_acc[ds] = mfma16x16x32(pt[kc], bo, dv_acc[ds]);
          dk_acc[ds] = mfma16x16x32(dst[kc], bq, dk_acc[ds]);
        }
      // dS into LDS as [query][128 keys] for the dQ product
      const int kcol = 64 * kb + 16 * kw + l16;
#pragma unroll
      for (int qs = 0; qs < 4; ++qs)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ql = 32 * (qs >> 1) + 8 * g4 + 4 * (qs & 1) + r;
          ds_lds[ql * 128 + (((kcol >> 3) ^ ds_swz(ql)) * 8) + (kcol & 7)] =
              dst[qs >> 1][4 * (qs & 1) + r];
        }
    }
    lds_barrier();  // dS of both key blocks visible

    // dQ_i += dS K over the retained key blocks; wave w
    // computes queries 16(w%4).. and d columns (D/2)(w/4).. of the tile
    {
      const int qsd = w & 3, dh = w >> 2;
      floatx4 acc[DQS];
#pragma unroll
      for (int x = 0; x < DQS; ++x) acc[x] = floatx4{0.f, 0.f, 0.f, 0.f};
      const int qa = 16 * qsd + l16;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        if (!((kc < 2) ? ret0 : ret1)) continue;
        const int ch = 4 * kc + g4;
        const bf16x8 a = *(const bf16x8*)(ds_lds + qa * 128 + ((ch ^ ds_swz(qa)) * 8));
#pragma unroll
        for (int x = 0; x < DQS; ++x) {
          const int d = (D / 2) * dh + 16 * x + l16;
          const bf16x8 bkt = *(const bf16x8*)(kt_lds + d * 128 + ((ch ^ (d & 15)) * 8));
          acc[x] = mfma16x16x32(a, bkt, acc[x]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qq = 64 * i + 16 * qsd + 4 * g4 + r;
        if (qq >= p.nq) continue;
        float* dst_row = p.dq_accum + (row0 + qq) * D + (D / 2) * dh + l16;
#pragma unroll
        for (int x = 0; x < DQS; ++x) atomicAdd(dst_row + 16 * x, acc[x][r]);
      }
    }
  }

  // ---- dK_j = scale * sum, dV_j; rows = keys 4g4 + r ----
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int kk = 64 * jw + 16 * kw + 4 * g4 + r;
    if (!kb_valid || kk >= p.nk) continue;
    __bf16* dkr = p.dk + ((size_t)bk * p.nk + kk) * D;
    __bf16* dvr = p.dv + ((size_t)bk * p.nk + kk) * D;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      dkr[16 * ds + l16] = to_bf16(dk_acc[ds][r] * p.scale);
      dvr[16 * ds + l16] = to_bf16(dv_acc[ds][r]);
    }
  }
}

template <int D>
hipError_t launch_all(const BwdParams& p, bool test, hipStream_t stream) {
  const long long rows = (long long)p.batch * p.heads_q * p.nq;
  const long long pre_threads = rows * (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((pre_threads + 255) / 256)), dim3(256),
                     0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((long long)p.npair * p.batch * p.heads_kv)), block(512);
  if (test)
    hipLaunchKernelGGL((bwd_main_kernel<D, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((bwd_main_kernel<D, false>), grid, block, 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n8 = rows * D / 8;
  hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                     p);
  return hipGetLastError();
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
  p.delta = a.delta;
  p.dq_accum = a.dq_accum;
  p.batch = a.batch;
  p.heads_q = a.heads_q;
  p.heads_kv = a.heads_kv;
  p.nq = a.nq;
  p.nk = a.nk;
  p.group = a.heads_q / a.heads_kv;
  p.causal = a.causal;
  p.scale = a.scale;
  p.c = a.scale * kLog2e;
  p.log2_tau = a.tau == 0.f ? -INFINITY : log2f(a.tau);
  p.tr = (a.nq + 63) / 64;
  p.tc = (a.nk + 63) / 64;
  p.npair = (p.tc + 1) / 2;
  p.counters = a.counters;
  p.decisions = a.decisions;
  return a.head_dim == 128 ? launch_all<128>(p, test, stream) : launch_all<64>(p, test, stream);
}

}  // namespace mala
