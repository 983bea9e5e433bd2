// C ABI of the MALA operator library: argument validation, workspace sizing
// and dispatch to the kernels. Every argument is checked on the host before
// the first HIP call, so each error path returns a status without touching
// the device.
#include <limits.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "mala.h"
#include "mala_internal.h"

namespace {

constexpr int64_t kMaxSeq = 1 << 24;       // keeps every index computation in range
constexpr int64_t kMaxGrid = (1ll << 31) - 1;

int check_shape(const mala_shape* s) {
  if (!s) return MALA_ERR_INVALID_ARG;
  if (s->batch < 1 || s->heads_q < 1 || s->heads_kv < 1 || s->seqlen_q < 1 || s->seqlen_k < 1 ||
      s->head_dim < 1)
    return MALA_ERR_INVALID_ARG;
  if (s->heads_q % s->heads_kv != 0) return MALA_ERR_INVALID_ARG;
  if (s->seqlen_q > kMaxSeq || s->seqlen_k > kMaxSeq) return MALA_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return MALA_ERR_UNSUPPORTED;
  // the largest tensor must stay addressable with 64-bit offsets and the
  // grids within range (checked generously)
  const long double elems = (long double)s->batch * s->heads_q * s->seqlen_q * s->head_dim;
  const long double kelems = (long double)s->batch * s->heads_kv * s->seqlen_k * s->head_dim;
  if (elems > 9.0e15L || kelems > 9.0e15L) return MALA_ERR_UNSUPPORTED;
  return MALA_OK;
}

int check_config(const mala_config* c, bool uses_tau) {
  if (!c) return MALA_ERR_INVALID_ARG;
  if (c->causal != 0 && c->causal != 1) return MALA_ERR_INVALID_ARG;
  if (c->block_q < 1 || c->block_k < 1) return MALA_ERR_INVALID_ARG;
  if ((c->block_q != 64 && c->block_q != 128) || (c->block_k != 64 && c->block_k != 128))
    return MALA_ERR_UNSUPPORTED;
  if (!(c->softmax_scale > 0.f) || isinf(c->softmax_scale)) return MALA_ERR_INVALID_ARG;
  if (uses_tau && (isnan(c->tau) || c->tau < 0.f)) return MALA_ERR_INVALID_ARG;
  return MALA_OK;
}

// Device check, cached per device ordinal: the kernels are built for gfx950.
int check_device() {
  static std::atomic<int> cache[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MALA_ERR_DEVICE;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 1) return MALA_OK;
    if (c == 2) return MALA_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MALA_ERR_DEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? MALA_OK : MALA_ERR_DEVICE;
}

int launch_status(hipError_t e) { return e == hipSuccess ? MALA_OK : MALA_ERR_LAUNCH; }

// Bound on the kernels' waits for one another, in polls: far beyond any
// legal schedule (a poll takes at least tens of cycles, so 2^22 of them
// last tens of milliseconds, against microseconds for a legal wait). The
// environment variable MALA_WAIT_BOUND overrides it for tests of the
// failure path (0 makes every wait give up at once); a malformed value is
// ignored.
int wait_bound() {
  constexpr int kDefault = 1 << 22;
  const char* s = getenv("MALA_WAIT_BOUND");
  if (!s || !*s) return kDefault;
  char* end = nullptr;
  const long long v = strtoll(s, &end, 10);
  if (!end || *end != '\0' || v < 0) return kDefault;
  return v > INT_MAX ? INT_MAX : (int)v;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---- device-resident scratch of mala_decode_noalloc -------------------------
// The split partials (m, l, u) of the allocation-free decode entry point live
// in this file-scope device array: each GPU the library runs on holds its own
// copy, at its own address, until the process ends. Host code never uses the
// array's name as an address (on the host it names a stand-in, not device
// memory); the address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
constexpr size_t kDecodeScratchBytes = 16u << 20;
constexpr int kMaxDevices = 64;
static __device__ __attribute__((aligned(256))) char scratch[kDecodeScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on the first call on
// that device).
int decode_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MALA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return MALA_ERR_DEVICE;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MALA_OK;
}

// The kernels move bf16 rows in 16-byte vectors and the workspace in float4
// words; lse, tables and lengths are read as 4-byte words, counters as
// 8-byte atomics.
bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

bool stats_aligned(const mala_stats* stats) {
  return !stats || !stats->counters || aligned(stats->counters, 8);
}

int fwd_common(const mala_shape* shape, const mala_config* cfg, const void* q, const void* k,
               const void* v, void* o, float* lse, const mala_stats* stats, void* stream,
               bool test) {
  int st = check_shape(shape);
  if (st) return st;
  st = check_config(cfg, test);
  if (st) return st;
  if (!q || !k || !v || !o || !lse) return MALA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !stats_aligned(stats))
    return MALA_ERR_INVALID_ARG;
  // causal queries align with the last keys; more queries than keys would
  // leave the first rows without a key
  if (cfg->causal && shape->seqlen_q > shape->seqlen_k) return MALA_ERR_UNSUPPORTED;
  const int64_t tr = (shape->seqlen_q + 63) / 64;
  if ((int64_t)shape->batch * shape->heads_q * ((tr + 3) / 4 + 1) > kMaxGrid)
    return MALA_ERR_UNSUPPORTED;
  st = check_device();
  if (st) return st;
  mala::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.batch = shape->batch;
  a.heads_q = shape->heads_q;
  a.heads_kv = shape->heads_kv;
  a.nq = shape->seqlen_q;
  a.nk = shape->seqlen_k;
  a.head_dim = shape->head_dim;
  a.causal = cfg->causal;
  a.block_q = cfg->block_q;
  a.block_k = cfg->block_k;
  a.scale = cfg->softmax_scale;
  a.tau = test ? cfg->tau : 0.f;
  a.spin = wait_bound();
  a.counters = stats ? stats->counters : nullptr;
  a.decisions = stats ? stats->decisions : nullptr;
  return launch_status(mala::launch_fwd(a, test, (hipStream_t)stream));
}

int bwd_common(const mala_shape* shape, const mala_config* cfg, const void* q, const void* k,
               const void* v, const void* o, const float* lse, const void* dout, void* dq,
               void* dk, void* dv, void* workspace, size_t workspace_bytes,
               const mala_stats* stats, void* stream, bool test) {
  int st = check_shape(shape);
  if (st) return st;
  st = check_config(cfg, test);
  if (st) return st;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return MALA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || !stats_aligned(stats))
    return MALA_ERR_INVALID_ARG;
  // causal queries align with the last keys; more queries than keys would
  // leave the first rows without a key
  if (cfg->causal && shape->seqlen_q > shape->seqlen_k) return MALA_ERR_UNSUPPORTED;
  const size_t need = mala_bwd_workspace_bytes(shape, cfg);
  if (!workspace || workspace_bytes < need) return MALA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return MALA_ERR_INVALID_ARG;
  const int64_t tc = (shape->seqlen_k + 63) / 64;
  const int64_t tr = (shape->seqlen_q + 63) / 64;
  // the dK/dV pass launches up to 8 segment workgroups per key block
  if ((int64_t)shape->batch * shape->heads_kv * tc * 8 > kMaxGrid) return MALA_ERR_UNSUPPORTED;
  if ((int64_t)shape->batch * shape->heads_q * ((tr + 3) / 4 + 1) > kMaxGrid)
    return MALA_ERR_UNSUPPORTED;
  // row-term pass: one 256-thread group per 16 (d = 64) or 8 (d = 128) padded rows
  if ((int64_t)shape->batch * shape->heads_q * tr * 64 * (shape->head_dim / 8) / 256 + 1 >
      kMaxGrid)
    return MALA_ERR_UNSUPPORTED;
  st = check_device();
  if (st) return st;
  mala::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.workspace = workspace;
  a.batch = shape->batch;
  a.heads_q = shape->heads_q;
  a.heads_kv = shape->heads_kv;
  a.nq = shape->seqlen_q;
  a.nk = shape->seqlen_k;
  a.head_dim = shape->head_dim;
  a.causal = cfg->causal;
  a.block_q = cfg->block_q;
  a.block_k = cfg->block_k;
  a.scale = cfg->softmax_scale;
  a.tau = test ? cfg->tau : 0.f;
  a.spin = wait_bound();
  a.counters = stats ? stats->counters : nullptr;
  a.decisions = stats ? stats->decisions : nullptr;
  return launch_status(mala::launch_bwd(a, test, (hipStream_t)stream));
}

// use_scratch: the partials go to the device-resident scratch array instead
// of a caller workspace (workspace / workspace_bytes are then ignored).
int decode_common(const mala_shape* shape, const mala_config* cfg, const void* q,
                  const void* k_cache, const void* v_cache, void* o, float* lse,
                  int32_t num_splits, void* workspace, size_t workspace_bytes,
                  const mala_stats* stats, void* stream, bool test,
                  const int32_t* block_table = nullptr, const int32_t* cache_lens = nullptr,
                  int32_t num_pages = 0, bool use_scratch = false) {
  int st = check_shape(shape);
  if (st) return st;
  st = check_config(cfg, test);
  if (st) return st;
  if (shape->seqlen_q != 1) return MALA_ERR_INVALID_ARG;
  if (!q || !k_cache || !v_cache || !o || !lse) return MALA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(block_table, 4) || !aligned(cache_lens, 4) ||
      !stats_aligned(stats))
    return MALA_ERR_INVALID_ARG;
  if (shape->heads_q / shape->heads_kv > 8) return MALA_ERR_UNSUPPORTED;
  if (num_splits < 1) return MALA_ERR_INVALID_ARG;
  const int64_t tc = (shape->seqlen_k + cfg->block_k - 1) / cfg->block_k;
  if (num_splits > tc) return MALA_ERR_INVALID_ARG;  // every split owns >= 1 decision tile
  const size_t need = mala_decode_workspace_bytes(shape, num_splits);
  if (use_scratch) {
    if (need > kDecodeScratchBytes) return MALA_ERR_WORKSPACE;
  } else {
    if (!workspace || workspace_bytes < need) return MALA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return MALA_ERR_INVALID_ARG;
  }
  if ((int64_t)shape->batch * shape->heads_kv * num_splits > kMaxGrid) return MALA_ERR_UNSUPPORTED;
  st = check_device();
  if (st) return st;
  if (use_scratch) {
    st = decode_scratch(&workspace);
    if (st) return st;
  }
  mala::DecodeArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.o = o;
  a.lse = lse;
  const size_t n = (size_t)shape->batch * shape->heads_q * num_splits;
  a.part_m = (float*)workspace;
  a.part_l = (float*)((char*)workspace + align256(n * sizeof(float)));
  a.part_u = (float*)((char*)workspace + 2 * align256(n * sizeof(float)));
  a.batch = shape->batch;
  a.heads_q = shape->heads_q;
  a.heads_kv = shape->heads_kv;
  a.nk = shape->seqlen_k;
  a.head_dim = shape->head_dim;
  a.num_splits = num_splits;
  a.block_k = cfg->block_k;
  a.scale = cfg->softmax_scale;
  a.tau = test ? cfg->tau : 0.f;
  a.counters = stats ? stats->counters : nullptr;
  a.decisions = stats ? stats->decisions : nullptr;
  a.block_table = block_table;
  a.cache_lens = cache_lens;
  a.num_pages = num_pages;
  return launch_status(mala::launch_decode(a, test, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int mala_fwd(const mala_shape* shape, const mala_config* cfg, const void* q, const void* k,
             const void* v, void* o, float* lse, const mala_stats* stats, void* stream) {
  return fwd_common(shape, cfg, q, k, v, o, lse, stats, stream, true);
}

int fullattn_fwd(const mala_shape* shape, const mala_config* cfg, const void* q, const void* k,
                 const void* v, void* o, float* lse, const mala_stats* stats, void* stream) {
  return fwd_common(shape, cfg, q, k, v, o, lse, stats, stream, false);
}

size_t mala_bwd_workspace_bytes(const mala_shape* shape, const mala_config* cfg) {
  if (check_shape(shape) || check_config(cfg, false)) return 0;
  return mala::bwd_workspace_bytes(shape->batch, shape->heads_q, shape->heads_kv,
                                   shape->seqlen_q, shape->seqlen_k, shape->head_dim,
                                   cfg->causal);
}

int mala_bwd(const mala_shape* shape, const mala_config* cfg, const void* q, const void* k,
             const void* v, const void* o, const float* lse, const void* dout, void* dq,
             void* dk, void* dv, void* workspace, size_t workspace_bytes,
             const mala_stats* stats, void* stream) {
  return bwd_common(shape, cfg, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                    stats, stream, true);
}

int fullattn_bwd(const mala_shape* shape, const mala_config* cfg, const void* q, const void* k,
                 const void* v, const void* o, const float* lse, const void* dout, void* dq,
                 void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 const mala_stats* stats, void* stream) {
  return bwd_common(shape, cfg, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                    stats, stream, false);
}

size_t mala_decode_workspace_bytes(const mala_shape* shape, int32_t num_splits) {
  if (check_shape(shape) || num_splits < 1) return 0;
  const size_t n = (size_t)shape->batch * shape->heads_q * num_splits;
  return 2 * align256(n * sizeof(float)) + align256(n * shape->head_dim * sizeof(float));
}

int32_t mala_decode_default_splits(const mala_shape* shape) {
  if (check_shape(shape)) return 1;
  // aim for >= 2048 (sequence, KV head, split) work items on 256 CUs,
  // with each split at least 8 key tiles long
  const int64_t tc = (shape->seqlen_k + 63) / 64;
  const int64_t pairs = (int64_t)shape->batch * shape->heads_kv;
  int64_t s = (2048 + pairs - 1) / pairs;
  if (s > tc / 8) s = tc / 8;
  if (s < 1) s = 1;
  if (s > 256) s = 256;
  return (int32_t)s;
}

int mala_decode(const mala_shape* shape, const mala_config* cfg, const void* q,
                const void* k_cache, const void* v_cache, void* o, float* lse,
                int32_t num_splits, void* workspace, size_t workspace_bytes,
                const mala_stats* stats, void* stream) {
  return decode_common(shape, cfg, q, k_cache, v_cache, o, lse, num_splits, workspace,
                       workspace_bytes, stats, stream, true);
}

int fullattn_decode(const mala_shape* shape, const mala_config* cfg, const void* q,
                    const void* k_cache, const void* v_cache, void* o, float* lse,
                    int32_t num_splits, void* workspace, size_t workspace_bytes,
                    const mala_stats* stats, void* stream) {
  return decode_common(shape, cfg, q, k_cache, v_cache, o, lse, num_splits, workspace,
                       workspace_bytes, stats, stream, false);
}

int mala_decode_noalloc(const mala_shape* shape, const mala_config* cfg, const void* q,
                        const void* k_cache, const void* v_cache, void* o, float* lse,
                        int32_t num_splits, const mala_stats* stats, void* stream) {
  return decode_common(shape, cfg, q, k_cache, v_cache, o, lse, num_splits, nullptr, 0, stats,
                       stream, true, nullptr, nullptr, 0, true);
}

int mala_decode_paged(const mala_shape* shape, const mala_config* cfg, const void* q,
                      const void* k_pages, const void* v_pages, const int32_t* block_table,
                      const int32_t* cache_lens, int32_t num_pages, void* o, float* lse,
                      int32_t num_splits, void* workspace, size_t workspace_bytes,
                      const mala_stats* stats, void* stream) {
  if (!block_table || !cache_lens || num_pages < 1) return MALA_ERR_INVALID_ARG;
  return decode_common(shape, cfg, q, k_pages, v_pages, o, lse, num_splits, workspace,
                       workspace_bytes, stats, stream, true, block_table, cache_lens, num_pages);
}

int fullattn_decode_paged(const mala_shape* shape, const mala_config* cfg, const void* q,
                          const void* k_pages, const void* v_pages, const int32_t* block_table,
                          const int32_t* cache_lens, int32_t num_pages, void* o, float* lse,
                          int32_t num_splits, void* workspace, size_t workspace_bytes,
                          const mala_stats* stats, void* stream) {
  if (!block_table || !cache_lens || num_pages < 1) return MALA_ERR_INVALID_ARG;
  return decode_common(shape, cfg, q, k_pages, v_pages, o, lse, num_splits, workspace,
                       workspace_bytes, stats, stream, false, block_table, cache_lens, num_pages);
}

const char* mala_status_string(int status) {
  switch (status) {
    case MALA_OK: return "success";
    case MALA_ERR_INVALID_ARG: return "invalid argument";
    case MALA_ERR_UNSUPPORTED: return "unsupported configuration (head_dim, tile size or size limit)";
    case MALA_ERR_WORKSPACE: return "workspace missing or too small";
    case MALA_ERR_DEVICE: return "no usable gfx950 HIP device";
    case MALA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
