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

// v_mfma_f32_32x32x16_bf16: D(32x32, fp32) += A(32x16) * B(16x32). Lane l
// supplies row (A) or column (B) l % 32 with reduction indices
// 8(l/32) .. 8(l/32)+7, and receives column l % 32 of D in 16 registers:
// register 4i + r holds row 8i + 4(l/32) + r. One wave reaches close to the
// matrix-core peak with this shape on its own (the 16x16x32 shape needs two
// waves per SIMD for that), and it leaves room for independent vector work
// between consecutive products.
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
__device__ __forceinline__ floatx16 mfma32x32x16(const bf16x8& a, const bf16x8& b,
                                                 const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Maximum / sum of x over the lane pair (l, l ^ 32), which hold the two
// 16-row halves of one column of a 32x32 MFMA result. v_permlane32_swap
// exchanges the two 32-lane halves between its operands, so both returned
// values are the pair seen from either side; a symmetric reduction of the
// two is correct whichever half ends up in which.
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// --- asynchronous global -> LDS copies ---------------------------------------
// global_load_lds_dwordx4: each lane's 16 bytes land at M0 + 16 * lane
// (lane-contiguous); the global address per lane is free, so a swizzled LDS
// layout is produced by choosing which chunk each lane fetches. The copy
// counts in vmcnt; vmcnt_wait<N>() waits until at most N vector-memory
// operations of this wave are outstanding (loads complete in issue order).
// The copy is issued as inline assembly: the compiler then neither treats it
// as an LDS store (it would otherwise drain vmcnt before every later LDS
// read, since it cannot tell ring slots apart) nor counts it, which only
// strengthens the waits it emits for its own loads. All ordering between the
// copies and the LDS reads of their data is explicit: vmcnt_wait followed by
// lds_barrier. The compiler treats M0 as a reserved register and does not
// honour it as a clobber of inline assembly; the copies are safe because no
// instruction the compiler generates in these kernels uses M0 (the generated
// assembly is checked by tests/test_isa_checks.py).

// LDS byte address of a __shared__ object (a 32-bit constant for the
// compiler; no generic-pointer arithmetic or null checks).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}
// Copy with a wave-uniform 64-bit base (SGPR pair), a 32-bit per-lane byte
// offset (no per-lane 64-bit address arithmetic) and the LDS destination as
// a byte address (no generic-pointer conversion).
__device__ __forceinline__ void async_copy16_sa(const void* sbase, uint32_t voff, uint32_t lds_byte) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_byte);
  // readfirstlane returns a signed int: go through uint32_t so that the low
  // half is zero-extended (a sign-extended low half would corrupt the high
  // half of the address)
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sb), "s"(lds)
      : "memory", "m0");
}

// Copy from a per-lane 64-bit address to an LDS byte address.
__device__ __forceinline__ void async_copy16_a(const void* gsrc, uint32_t lds_byte) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gsrc), "s"(lds)
      : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void vmcnt_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (7 << 4) | (0xF << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// vmcnt wait with a run-time (wave-uniform) count: waits for the largest
// supported count <= n (waiting for more than needed is always safe).
__device__ __forceinline__ void vmcnt_wait_le(int n) {
  switch (n < 0 ? 0 : (n > 48 ? 48 : n)) {
    case 0: vmcnt_wait<0>(); break;
    case 1: vmcnt_wait<1>(); break;
    case 2: vmcnt_wait<2>(); break;
    case 3: vmcnt_wait<3>(); break;
    case 4: vmcnt_wait<4>(); break;
    case 5: vmcnt_wait<5>(); break;
    case 6: vmcnt_wait<6>(); break;
    case 7: vmcnt_wait<7>(); break;
    case 8: vmcnt_wait<8>(); break;
    case 9: vmcnt_wait<9>(); break;
    case 10: vmcnt_wait<10>(); break;
    case 11: vmcnt_wait<11>(); break;
    case 12: vmcnt_wait<12>(); break;
    case 13: vmcnt_wait<13>(); break;
    case 14: vmcnt_wait<14>(); break;
    case 15: vmcnt_wait<15>(); break;
    case 16: vmcnt_wait<16>(); break;
    case 17: vmcnt_wait<17>(); break;
    case 18: vmcnt_wait<18>(); break;
    case 19: vmcnt_wait<19>(); break;
    case 20: vmcnt_wait<20>(); break;
    case 21: vmcnt_wait<21>(); break;
    case 22: vmcnt_wait<22>(); break;
    case 23: vmcnt_wait<23>(); break;
    case 24: vmcnt_wait<24>(); break;
    case 25: vmcnt_wait<25>(); break;
    case 26: vmcnt_wait<26>(); break;
    case 27: vmcnt_wait<27>(); break;
    case 28: vmcnt_wait<28>(); break;
    case 29: vmcnt_wait<29>(); break;
    case 30: vmcnt_wait<30>(); break;
    case 31: vmcnt_wait<31>(); break;
    case 32: vmcnt_wait<32>(); break;
    case 33: vmcnt_wait<33>(); break;
    case 34: vmcnt_wait<34>(); break;
    case 35: vmcnt_wait<35>(); break;
    case 36: vmcnt_wait<36>(); break;
    case 37: vmcnt_wait<37>(); break;
    case 38: vmcnt_wait<38>(); break;
    case 39: vmcnt_wait<39>(); break;
    case 40: vmcnt_wait<40>(); break;
    case 41: vmcnt_wait<41>(); break;
    case 42: vmcnt_wait<42>(); break;
    case 43: vmcnt_wait<43>(); break;
    case 44: vmcnt_wait<44>(); break;
    case 45: vmcnt_wait<45>(); break;
    case 46: vmcnt_wait<46>(); break;
    case 47: vmcnt_wait<47>(); break;
    default: vmcnt_wait<48>(); break;
  }
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte rows addressed by lanes 4e + i/4 (e = 0..3). Lane j
// addressing row k0 + j/4, columns n0 + 4(j%4) .. +3 of a row-major [k][n]
// bf16 tile therefore gives lane i the column n0 + i for rows k0 .. k0+3:
// the transposed MFMA operand, read straight from the natural layout.
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short short4v;
__device__ __forceinline__ short4v lds_read_tr4(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v*)(p));
}
// Two transposed 4-element reads joined into one MFMA operand. The join is a
// whole-vector shuffle plus one bit cast: inserting the 16-bit values into a
// bf16 vector element by element produced wrong operands at -O3.
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short short8v;
__device__ __forceinline__ bf16x8 join_tr(const short4v& lo, const short4v& hi) {
  const short8v v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// --- LDS swizzles -----------------------------------------------------------
// Tiles of the 32x32 products ([64 rows][D] bf16, 16-byte chunks XORed per
// row). K-type tiles are read row-major by 32 consecutive rows per
// instruction (one chunk each); their swizzle makes any 16 consecutive rows
// hit distinct 16-byte bank groups. V-type tiles are read with the
// transposing read, 4 consecutive rows x 16 columns per 16-lane group and 4
// chunks across a 32-lane phase; their swizzle keeps those 4 rows on distinct
// bank groups for 32- and 64-bank phases.
template <int D>
__device__ __forceinline__ int kswz32(int row) {
  if constexpr (D == 128) return row & 15;
  else return (row & 7) ^ ((row >> 3) & 1);
}
template <int D>
__device__ __forceinline__ int vswz32(int row) {
  if constexpr (D == 128) return (6 * (row & 1)) ^ (10 * ((row >> 1) & 1));
  else return 2 * (row & 3);
}

// Tiles read both ways with the 32x32 shapes (the Q and dO tiles of the
// dK/dV pass): row-major operand reads of 32 consecutive rows (one chunk
// each) and the transposing reads of the V-type pattern above. Chunk bits
// 2-3 and 1-2 follow row bits 0-1 one to one (distinct bank groups for the
// transposing reads with 64 and 32 banks), and the whole XOR is one to one on
// row bits 0-3 (distinct groups for 16 consecutive rows of the row-major
// reads).
template <int D>
__device__ __forceinline__ int qswz32(int row) {
  if constexpr (D == 128)
    return (6 * (row & 1)) ^ (10 * ((row >> 1) & 1)) ^ ((row >> 2) & 1) ^ (8 * ((row >> 3) & 1));
  else
    return (2 * (row & 1)) ^ (4 * ((row >> 1) & 1)) ^ ((row >> 2) & 1) ^ (2 * ((row >> 3) & 1));
}

// Tiles of the 16x16 products read both ways (the K and V tiles of the dQ
// pass): row-major operand reads whose 16 rows per lane group are the
// permuted set 32a + 8(R/4) + 4c + R%4 (R = 0..15, one chunk per lane group),
// and transposing reads of 4 consecutive rows x 16 columns per 16-lane group.
// Measured on gfx950 (bank-conflict counter, each access kind alone): the
// transposing reads go in 32-lane phases over 64 banks, and a 16-byte read
// serves, per half wave, the lanes whose bits 2-4 have equal parity
// together. For d = 128 chunk bits 1-3 follow row bits 0, 1, 3; for d = 64
// chunk bits 1-2 follow row bits 1, 3. Both access kinds are then free of
// bank conflicts.
template <int D>
__device__ __forceinline__ int dqswz(int row) {
  if constexpr (D == 128)
    return ((row & 3) << 1) | (((row >> 3) & 1) << 3);
  else
    return (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2);
}

}  // namespace mala
