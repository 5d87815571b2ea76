// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int WAVE = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// Round to nearest even; NaN stays a quiet NaN (a select, not a branch).
__device__ __forceinline__ uint16_t f2bf(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return uint16_t((u & 0x7fffffffu) > 0x7f800000u ? (u >> 16) | 0x40u : r);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (lo in the low half) with gfx950's conversion
// instruction (v_cvt_pk_bf16_f32): round to nearest even, NaN quiet.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const floatx2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) { return __shfl_xor(v, mask, WAVE); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = __shfl_xor(uint32_t(v), mask, WAVE);
  uint32_t hi = __shfl_xor(uint32_t(v >> 32), mask, WAVE);
  return (uint64_t(hi) << 32) | lo;
}

// Reductions over aligned groups of G <= 16 lanes with DPP inside a row of
// 16 lanes: quad swaps (lane ^ 1, lane ^ 2), then the half-row mirror (lane i
// <-> 7 - i) and the row mirror (i <-> 15 - i), which pair each partial with
// one from the other half once the halves are uniform.  Every lane of a group
// ends with the same result (each step combines two equal-order partials), no
// LDS crossbar round trips.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return uint64_t(dpp_u32<CTRL>(uint32_t(v))) | (uint64_t(dpp_u32<CTRL>(uint32_t(v >> 32))) << 32);
}
template <int G>
__device__ __forceinline__ float row_max(float v) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "group of 2..16 lanes");
  v = fmaxf(v, dpp_f32<0xB1>(v));
  if constexpr (G >= 4) v = fmaxf(v, dpp_f32<0x4E>(v));
  if constexpr (G >= 8) v = fmaxf(v, dpp_f32<0x141>(v));
  if constexpr (G >= 16) v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}
template <int G>
__device__ __forceinline__ float row_sum(float v) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "group of 2..16 lanes");
  v += dpp_f32<0xB1>(v);
  if constexpr (G >= 4) v += dpp_f32<0x4E>(v);
  if constexpr (G >= 8) v += dpp_f32<0x141>(v);
  if constexpr (G >= 16) v += dpp_f32<0x140>(v);
  return v;
}
template <int G>
__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "group of 2..16 lanes");
  uint64_t o = dpp_u64<0xB1>(v);
  v = o > v ? o : v;
  if constexpr (G >= 4) { o = dpp_u64<0x4E>(v); v = o > v ? o : v; }
  if constexpr (G >= 8) { o = dpp_u64<0x141>(v); v = o > v ? o : v; }
  if constexpr (G >= 16) { o = dpp_u64<0x140>(v); v = o > v ? o : v; }
  return v;
}

// Reductions over aligned groups of G lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}
template <int G>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

// Total order key of a selection score: larger score -> larger key, -0 == +0,
// NaN below everything (key 0).
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0u;
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The 32-bit finalizer of MurmurHash3 (Appleby, public domain): a bijection
// of the 32-bit integers with full avalanche.
__host__ __device__ __forceinline__ uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

// ---------------------------------------------------------------- 16-byte memory ops
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
