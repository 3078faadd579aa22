// tern_device.h -- device helpers shared by the HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tern_internal.h"

namespace tern {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Pointers reach the kernels through descriptors in memory, so the compiler
// cannot see that they are global; say so, to get global_load instead of
// flat_load.
template <typename T>
using gptr = const T __attribute__((address_space(1)))*;

// Packed weights are read exactly once per launch: stream them past the
// caches with a non-temporal 16-byte load (global_load_dwordx4 ... nt).
__device__ __forceinline__ u32x4 load_weights16(const uint8_t* p) {
  return __builtin_nontemporal_load((gptr<u32x4>)(p));
}

// Activations and metadata are re-read by many waves: ordinary loads.
__device__ __forceinline__ u32x4 load16(const void* p) { return *(gptr<u32x4>)(p); }

template <typename T>
__device__ __forceinline__ T load_g(const T* p) {
  return *(gptr<T>)(p);
}

template <typename T>
__device__ __forceinline__ void store_g(T* p, T v) {
  *(T __attribute__((address_space(1)))*)(p) = v;
}

// Raw buffer resource over `bytes` bytes at `base` (stride 0, gfx9 format
// word).  A buffer store whose offset lies outside the range is dropped by
// the hardware, so a wave can issue a store on every lane and let the range
// check mask it: no branch around the store, and the store is always in
// the instruction stream (loads issued after it can then be waited for
// without also waiting for it).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kDropOffset = 0x80000000u;  // beyond any range used here

__device__ __forceinline__ void buffer_store_u32(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}

// Range-checked loads (a load outside the range returns zero and touches no
// memory).  The whole offset is the per-lane one: the range check covers it.
// Weights use the non-temporal policy, as load_weights16.
constexpr int kCpolNT = 2;
__device__ __forceinline__ u32x4 buffer_load_weights16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCpolNT));
}
__device__ __forceinline__ uint32_t buffer_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// ---- cross-lane exchange within a wave64 -------------------------------
// dpp_partner<D>(v) returns v from a partner lane at "distance" D inside the
// same 16-lane DPP row: for D = 8 the lane l ^ 8 (row_ror:8), for D = 4 the
// mirror lane 7 - (l & 7) of the same 8-lane half (row_half_mirror), for
// D = 2 and 1 the lane l ^ D (quad_perm).  Each pairs every lane whose bit D
// is clear with one whose bit D is set, which is all a butterfly needs.
template <int D>
__device__ __forceinline__ uint32_t dpp_partner(uint32_t v) {
  static_assert(D == 8 || D == 4 || D == 2 || D == 1, "DPP distance");
  constexpr int ctrl = D == 8 ? 0x128 : D == 4 ? 0x141 : D == 2 ? 0x4E : 0xB1;
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, 0xF, 0xF, false);
}

// Sum of v over the pair (lane, partner at distance D); every lane gets it.
template <int D>
__device__ __forceinline__ uint32_t pair_sum(uint32_t v) {
  if constexpr (D == 32) {
    // v_permlane32_swap: upper half of the first operand <-> lower half of
    // the second; with both operands v the two results are v and v^32.
    auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return p[0] + p[1];
  } else if constexpr (D == 16) {
    auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return p[0] + p[1];
  } else {
    return v + dpp_partner<D>(v);
  }
}

// Transposed butterfly step: lanes with bit D clear keep a + partner's a,
// lanes with bit D set keep b + partner's b.
template <int D>
__device__ __forceinline__ uint32_t pair_split(uint32_t a, uint32_t b, int lane) {
  if constexpr (D == 32) {
    // after the swap: first = (a_lo | b_lo), second = (a_hi | b_hi)
    auto p = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    return p[0] + p[1];
  } else if constexpr (D == 16) {
    auto p = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    return p[0] + p[1];
  } else {
    const bool hi = (lane & D) != 0;
    const uint32_t keep = hi ? b : a;
    const uint32_t send = hi ? a : b;
    return keep + dpp_partner<D>(send);
  }
}

// Reduce NV per-lane values over groups of LPR lanes (aligned, LPR a power of
// two <= 64, NV a power of two <= LPR).  Returns, in every lane, the group
// total of value index  vidx(lane) = sum_i bit(lane, LPR/2 >> i) << i  for
// i < log2(NV); all lanes of a group that share those bits hold the same
// total.
template <int LPR, int NV>
__device__ __forceinline__ uint32_t reduce_split(uint32_t (&v)[NV], int lane) {
  static_assert(NV >= 1 && NV <= LPR && (NV & (NV - 1)) == 0, "NV");
  if constexpr (NV > 1) {
    constexpr int D = LPR / 2;
#pragma unroll
    for (int k = 0; k < NV / 2; ++k) v[k] = pair_split<D>(v[2 * k], v[2 * k + 1], lane);
    // the surviving NV/2 values now differ between the two halves; recurse
    // inside each half
    uint32_t (&w)[NV / 2] = *reinterpret_cast<uint32_t(*)[NV / 2]>(&v[0]);
    return reduce_split<LPR / 2, NV / 2>(w, lane);
  } else {
    uint32_t x = v[0];
    if constexpr (LPR >= 64) x = pair_sum<32>(x);
    if constexpr (LPR >= 32) x = pair_sum<16>(x);
    if constexpr (LPR >= 16) x = pair_sum<8>(x);
    if constexpr (LPR >= 8) x = pair_sum<4>(x);
    if constexpr (LPR >= 4) x = pair_sum<2>(x);
    if constexpr (LPR >= 2) x = pair_sum<1>(x);
    return x;
  }
}

// Value index held by `lane` after reduce_split<LPR, NV>.
template <int LPR, int NV>
__device__ __forceinline__ int split_index(int lane) {
  int idx = 0;
#pragma unroll
  for (int i = 0, d = LPR / 2; (1 << i) < NV; ++i, d >>= 1) idx |= ((lane & d) ? 1 : 0) << i;
  return idx;
}

// Plain sum over an aligned group of LPR lanes, returned in every lane.
template <int LPR>
__device__ __forceinline__ uint32_t group_sum(uint32_t x) {
  uint32_t v[1] = {x};
  return reduce_split<LPR, 1>(v, 0);
}

// Wait for the wave's LDS accesses; no memory access moves across it.
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// y = (s_row * acc) * s_act with two round-to-nearest products.
// z * rowsum (or (z + 128) * rowsum) as a full-rate 24-bit multiply: the
// 32-bit integer multiply is a quarter-rate instruction.  The product is
// exact while both factors fit 24 signed bits, which the call preconditions
// give: |z| <= 255, and a row or block sum of ternary weights is at most K <=
// TERN_MAX_K < 2^23 in magnitude.
__device__ __forceinline__ uint32_t mul_zr(int32_t z, int32_t r) { return (uint32_t)__mul24(z, r); }

__device__ __forceinline__ float epilogue(float s_row, int32_t acc, float s_act) {
  return __fmul_rn(__fmul_rn(s_row, (float)acc), s_act);
}

// run + s * a with the product and the sum each rounded to nearest: HIP's
// __fmul_rn / __fadd_rn are the plain operators, which the compiler would
// otherwise fuse into one FMA (one rounding instead of two).
__device__ __forceinline__ float add_product_rn(float run, float s, float a) {
#pragma clang fp contract(off)
  return run + s * a;
}

}  // namespace tern
