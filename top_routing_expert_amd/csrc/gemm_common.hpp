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
__device__ __forceinline__ float4 unpack_bf4(uint2 u) {
  return make_float4(bf2f(uint16_t(u.x & 0xffffu)), bf2f(uint16_t(u.x >> 16)),
                     bf2f(uint16_t(u.y & 0xffffu)), bf2f(uint16_t(u.y >> 16)));
}

}  // namespace moe
