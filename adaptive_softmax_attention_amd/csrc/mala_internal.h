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
  void* workspace;  // bwd_workspace_bytes(): per-block row terms + decision map
  int batch, heads_q, heads_kv, nq, nk, head_dim;
  int causal;
  int block_q, block_k;  // decision tile, 64 or 128 each
  float scale;
  float tau;
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

size_t bwd_workspace_bytes(int batch, int heads_q, int heads_kv, int nq, int nk, int head_dim,
                           int causal);
size_t decode_workspace_bytes(int batch, int heads_q, int num_splits, int head_dim);

}  // namespace mala
