// Internal launch interface between the C ABI (mala_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mala {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int batch, heads_q, heads_kv, nq, nk, head_dim;
  int causal;
  int block_q, block_k;  // decision tile, 64 or 128 each
  float scale;
  float tau;
  int spin;  // bound on the kernel's waits for one another (polls)
  unsigned long long* counters;
  uint8_t* decisions;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  void* workspace;  // bwd_workspace_bytes(): status word, row terms, decision map, partials
  int batch, heads_q, heads_kv, nq, nk, head_dim;
  int causal;
  int block_q, block_k;  // decision tile, 64 or 128 each
  float scale;
  float tau;
  int spin;  // bound on every wait of the scoring pass (polls)
  unsigned long long* counters;
  uint8_t* decisions;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* part_m;  // [B][Hq][S] fp32 (log2 domain)
  float* part_l;  // [B][Hq][S]
  float* part_u;  // [B][Hq][S][D]
  int batch, heads_q, heads_kv, nk, head_dim;
  int num_splits;
  int block_k;  // decision tile keys, 64 or 128
  float scale;
  float tau;
  unsigned long long* counters;
  uint8_t* decisions;
  // paged, variable-length cache (nullptr: contiguous caches of nk keys)
  const int32_t* block_table;  // [batch][ceil(nk / 64)]
  const int32_t* cache_lens;   // [batch]
  int num_pages;
};

// Each returns hipSuccess or the launch error. `test` selects the MALA rule
// (true) or the dense path (false).
hipError_t launch_fwd(const FwdArgs& a, bool test, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, bool test, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, bool test, hipStream_t stream);

// ---- backward workspace layout (shared by the size query and the launch) ----
constexpr int kRowInfo = 256;       // floats of row terms per 64-row block
constexpr size_t kBwdHeader = 256;  // bytes before the row terms: the int32 status word
constexpr int kSegMax = 8;          // dK/dV segments per pair of key blocks, at most
constexpr int kSlotsPerPair = 4;    // fp32 partial-sum slots per pair of key blocks

// Causal legal tiles: query block i reaches key blocks 0 .. min(tc - 1,
// i + cblk), so the decision map stores min(tc, i + cblk + 1) bytes for it;
// causal_row_start(i) is the number stored for the blocks before i (the
// lower triangle when nq = nk).
__host__ __device__ inline long long causal_row_start(long long i, long long tc, long long cblk) {
  const long long istar = tc - cblk - 1 > 0 ? tc - cblk - 1 : 0;  // blocks that reach every key block
  const long long m = i < istar ? i : istar;
  return m * (m - 1) / 2 + m * (cblk + 1) + (i - m) * tc;
}

// [header][row terms, B*Hq*Tr blocks][decision map][partial dK/dV: B*Hkv x
// kSlotsPerPair npair slots x 2 blocks x (dK, dV) x 64 x d fp32][int32 tables: kept items
// and segment entry per key block, npair pairs, npair * kSegMax work items,
// work count], with npair = Tc / 2 + 1.
inline size_t bwd_workspace_bytes(int batch, int heads_q, int heads_kv, int nq, int nk,
                                  int head_dim, int causal) {
  const size_t tr = (size_t)(nq + 63) / 64, tc = (size_t)(nk + 63) / 64;
  const size_t rowinfo = (size_t)batch * heads_q * tr * kRowInfo * sizeof(float);
  const long long off = causal ? (long long)nk - nq : 0;
  const size_t per_head =
      causal ? (size_t)causal_row_start((long long)tr, (long long)tc, (63 + off) / 64) : tr * tc;
  const size_t dmap = (size_t)batch * heads_q * per_head;
  const size_t npair = tc / 2 + 1;
  const size_t part =
      (size_t)batch * heads_kv * kSlotsPerPair * npair * 2 * 2 * 64 * head_dim * sizeof(float);
  const size_t tabs =
      (size_t)batch * heads_kv * (2 * tc + 2 * npair + npair * kSegMax + 1) * sizeof(int);
  return kBwdHeader + ((rowinfo + 255) & ~(size_t)255) + ((dmap + 255) & ~(size_t)255) + part +
         tabs;
}
size_t decode_workspace_bytes(int batch, int heads_q, int num_splits, int head_dim);

}  // namespace mala
