// Shared device helpers for the MALA kernels (gfx950 / CDNA4).
//
// Matrix products use v_mfma_f32_16x16x32_bf16: D(16x16, fp32) += A(16x32,
// bf16) * B(32x16, bf16). Lane l of a wave64 supplies row (A) or column (B)
// l % 16 and eight consecutive reduction indices of group l / 16; it receives
// column l % 16 and rows 4*(l/16) + 0..3 of D. The kernels arrange both
// operands with the same reduction-index assignment, so any fixed hardware
// ordering of the eight values inside a lane yields the same contraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mala {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

__device__ __forceinline__ floatx4 mfma16x16x32(const bf16x8& a, const bf16x8& b,
                                                const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Cross-lane maximum / sum over the four lane groups (l, l^16, l^32, l^48)
// that hold the same query column of an MFMA result.
__device__ __forceinline__ float group4_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float group4_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ bool wave_any(bool p) { return __any(p); }

// Workgroup barrier for LDS traffic only. __syncthreads() also fences global
// memory at workgroup scope, which makes every wave drain its outstanding
// global loads (s_waitcnt vmcnt(0)) at each barrier and so defeats register
// prefetching. None of these kernels communicates through global memory
// within a launch, so waiting for this wave's LDS operations
// (lgkmcnt(0), with vmcnt and expcnt left at their maxima) before s_barrier
// is sufficient; the signal fence keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Round-to-nearest-even fp32 -> bf16 pair (the compiler emits the native
// conversion on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }

// --- LDS swizzles -----------------------------------------------------------
// K tile in LDS: [64 keys][D] bf16, 16-byte chunks XOR-swizzled per key so
// that the eight lanes of one read phase (keys 0-3 and 8-11 of a 16-key
// group, same column chunk) hit distinct bank groups.
__device__ __forceinline__ int k_swz(int key) {
  return (key & 3) | ((key & 8) >> 1) | ((key & 4) << 1);
}
// V^T tile in LDS: [D][64 keys] bf16 (128 B rows of eight 16-byte chunks).
__device__ __forceinline__ int v_swz(int d) { return (d ^ (d >> 3)) & 7; }

}  // namespace mala
