// Pieces shared by the grouped-GEMM kernels (fp32 and bf16).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

struct TileCoord {
  int grp, row0, M, m0, n0;
};

// Tile `tile` of a grouped GEMM whose per-group tile prefix is ts[0..G]
// (ts[g] = tiles of the groups before g, m-tiles fastest within a group).
// Empty groups own no tile, so the owner is the largest g with ts[g] <= tile.
__device__ __forceinline__ void locate_tile(const int32_t* ts, const int32_t* offsets, int G,
                                            int tile, int BM, int BN, TileCoord& tc) {
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ts[mid] <= tile) lo = mid; else hi = mid;
  }
  const int local = tile - ts[lo];
  const int row0 = offsets[lo];
  const int M = offsets[lo + 1] - row0;
  const int mt = int(cdiv(M, BM));
  tc.grp = lo;
  tc.row0 = row0;
  tc.M = M;
  tc.m0 = (local % mt) * BM;
  tc.n0 = (local / mt) * BN;
}

__device__ __forceinline__ float gelu_erf(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
}
__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }
// d/dv silu(v) = sigma(v) * (1 + v * (1 - sigma(v)))
__device__ __forceinline__ float dsilu(float v) {
  const float s = 1.0f / (1.0f + expf(-v));
  return s * (1.0f + v * (1.0f - s));
}
// d/dv gelu(v) = Phi(v) + v * phi(v) for the exact erf GELU
__device__ __forceinline__ float dgelu_erf(float v) {
  return 0.5f * (1.0f + erff(v * 0.70710678118654752f)) +
         v * 0.39894228040143268f * expf(-0.5f * v * v);
}
// Cheaper forms for epilogues whose results are rounded to bf16 (relative
// step 2^-9): hardware 2^x and reciprocal (about 1 ulp each) and erf from
// Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26:
// erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
// t = 1 / (1 + p x) for x >= 0, |error| <= 1.5e-7.  GELU's exp(-v^2/2) is the
// same exponential, so gelu' costs one more multiply-add.
__device__ __forceinline__ float exp_fast(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }
// 1 - erf(|x|) = poly(t) * e with e = exp(-x^2) supplied by the caller
__device__ __forceinline__ float erfc_poly(float ax) {
  const float t = rcp_fast(fmaf(0.3275911f, ax, 1.0f));
  float p = 1.061405429f;
  p = fmaf(p, t, -1.453152027f);
  p = fmaf(p, t, 1.421413741f);
  p = fmaf(p, t, -0.284496736f);
  p = fmaf(p, t, 0.254829592f);
  return p * t;
}
// Phi(v) = (1 + erf(v / sqrt 2)) / 2 and the Gaussian factor exp(-v^2/2)
__device__ __forceinline__ float phi_cdf(float v, float& e) {
  const float x = v * 0.70710678118654752f;
  e = exp_fast(-x * x);
  const float q = 0.5f * erfc_poly(fabsf(x)) * e;   // (1 - erf|x|) / 2
  return v >= 0.0f ? 1.0f - q : q;
}
__device__ __forceinline__ float gelu_fast(float v) {
  float e;
  return v * phi_cdf(v, e);
}
__device__ __forceinline__ float dgelu_fast(float v) {
  float e;
  const float c = phi_cdf(v, e);
  return fmaf(v * 0.39894228040143268f, e, c);
}
__device__ __forceinline__ float silu_fast(float v) { return v * rcp_fast(1.0f + exp_fast(-v)); }
__device__ __forceinline__ float dsilu_fast(float v) {
  const float s = rcp_fast(1.0f + exp_fast(-v));
  return s * fmaf(v, 1.0f - s, 1.0f);
}

__device__ __forceinline__ float4 unpack_bf4(uint2 u) {
  return make_float4(bf2f(uint16_t(u.x & 0xffffu)), bf2f(uint16_t(u.x >> 16)),
                     bf2f(uint16_t(u.y & 0xffffu)), bf2f(uint16_t(u.y >> 16)));
}

// Operands are read through raw buffer descriptors (base and size in scalar
// registers): each load instruction carries a 32-bit per-lane offset, and the
// K advance is a scalar offset or a rebased descriptor, so no 64-bit address
// arithmetic runs per stage.  Loads at or beyond the descriptor's size return
// zeros (K rows past the end of a group in the weight-gradient mode).  These
// loads count on vmcnt only, so the waits for LDS reads never wait for them
// (the global-to-LDS form also counts on lgkmcnt).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // dword 3: a raw (untyped, unswizzled) buffer on CDNA
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), int(bytes), 0x00020000);
}
__device__ __forceinline__ uint32_t clamp_bytes(int64_t b) {
  return b <= 0 ? 0u : (b >= int64_t(0xffffffff) ? 0xffffffffu : uint32_t(b));
}

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ...
// lds): lane l writes lds_wave_base + 16*l; the LDS pointer must be
// wave-uniform.  (A plain function: the builtin called from a lambda inside a
// kernel template breaks the host-side instantiation.)
__device__ __forceinline__ void lds_load16(rsrc_t r, uint32_t voff, uint32_t soff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)(lds_wave_base), 16, voff, soff, 0, 0);
}
// 4 bytes per lane: lane l writes the dword at lds_wave_base + 4*l.
__device__ __forceinline__ void lds_load4(rsrc_t r, uint32_t voff, uint32_t soff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)(lds_wave_base), 4, voff, soff, 0, 0);
}

// Wait until at most N of this wave's vector-memory loads are outstanding
// (s_waitcnt vmcnt(N); expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding load); LDS accesses are not moved across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace moe
