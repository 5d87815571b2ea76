// Counter-based draws for the stochastic routers: the standard-normal noise
// of noisy top-k gating ("Mixture of Experts Explained", "What is sparsity?",
// the H(x) equation) and the per-token uniform of GShard's random second
// expert ("Mixture of Experts Explained", "MoEs and Transformers").
//
// Generator: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011), keyed by (seed, 0).  Stream s
// (0 = normals, 1 = uniforms) of a call with offset o draws block b from
// counter (b, o, s, 0); element j takes word j % 4 of block j / 4.  A uniform
// is a word's top 24 bits times 2^-24 (exact in fp32, in [0, 1)).  Normals
// come in pairs from words (0, 1) and (2, 3) of a block by the Box-Muller
// transform: r = sqrt(-2 ln(1 - u)), (r cos 2 pi v, r sin 2 pi v).
//
// One lane per Philox block: the whole draw is 20 64-bit multiplies and a
// handful of transcendentals per 4 outputs, so the kernel is bound by its
// 16-byte stores.
#include "../../include/moe.h"
#include "common.hpp"

namespace moe {
namespace {

constexpr uint64_t PHILOX_M0 = 0xD2E7470EE14C6C93ull, PHILOX_M1 = 0xCA5A826395121157ull;
constexpr uint64_t PHILOX_W0 = 0x9E3779B97F4A7C15ull, PHILOX_W1 = 0xBB67AE8584CAA73Bull;

struct Words { uint64_t w[4]; };

__device__ __forceinline__ Words philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                               uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(PHILOX_M0, c0), lo0 = PHILOX_M0 * c0;
    const uint64_t hi1 = __umul64hi(PHILOX_M1, c2), lo1 = PHILOX_M1 * c2;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += PHILOX_W0;
    k1 += PHILOX_W1;
  }
  return Words{{c0, c1, c2, c3}};
}

__device__ __forceinline__ float uniform24(uint64_t w) {
  return float(uint32_t(w >> 40)) * 0x1p-24f;   // exact: a 24-bit integer times 2^-24
}

__device__ __forceinline__ float2 box_muller(uint64_t wu, uint64_t wv) {
  const float u = uniform24(wu), v = uniform24(wv);
  // ln(1 - u) with 1 - u in (0, 1]; log1p keeps full relative accuracy near u = 0
  const float r = sqrtf(-2.0f * log1pf(-u));
  float s, c;
  sincospif(2.0f * v, &s, &c);   // 2v exact; sin/cos of pi * 2v
  return make_float2(r * c, r * s);
}

__global__ void __launch_bounds__(256)
router_draws_kernel(uint64_t seed, uint64_t offset, int64_t n_noise, float* __restrict__ noise,
                    bool noise_vec, int64_t n_uni, float* __restrict__ uniform) {
  const int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (noise && 4 * b < n_noise) {
    const Words q = philox4x64_10(uint64_t(b), offset, 0, 0, seed, 0);
    const float2 z01 = box_muller(q.w[0], q.w[1]);
    const float2 z23 = box_muller(q.w[2], q.w[3]);
    const int64_t j = 4 * b;
    if (noise_vec && j + 4 <= n_noise) {
      *reinterpret_cast<float4*>(noise + j) = make_float4(z01.x, z01.y, z23.x, z23.y);
    } else {
      const float z[4] = {z01.x, z01.y, z23.x, z23.y};
      for (int i = 0; i < 4 && j + i < n_noise; ++i) noise[j + i] = z[i];
    }
  }
  if (uniform && 4 * b < n_uni) {
    const Words q = philox4x64_10(uint64_t(b), offset, 1, 0, seed, 0);
    const int64_t j = 4 * b;
    for (int i = 0; i < 4 && j + i < n_uni; ++i) uniform[j + i] = uniform24(q.w[i]);
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_router_draws(const moe_dims* d, uint64_t seed, uint64_t offset, float* noise,
                                float* uniform, void* stream) {
  if (!d || d->T < 0 || d->E < 1) return MOE_ERR_INVALID_ARG;
  if (d->T > (int64_t(1) << 40) / d->E) return MOE_ERR_UNSUPPORTED;
  const int64_t n_noise = noise ? d->T * d->E : 0, n_uni = uniform ? d->T : 0;
  const int64_t lanes = cdiv(n_noise > n_uni ? n_noise : n_uni, 4);
  if (lanes == 0) return MOE_OK;
  const int64_t blocks = cdiv(lanes, 256);
  if (blocks > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  const bool vec = (reinterpret_cast<uintptr_t>(noise) & 15u) == 0;
  hipLaunchKernelGGL(router_draws_kernel, dim3(unsigned(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), seed, offset, n_noise, noise, vec, n_uni,
                     uniform);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
