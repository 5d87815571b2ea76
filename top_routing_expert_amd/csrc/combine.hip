// Weighted unpermute-combine of the sparse MoE layer for gfx950, and the
// fixed-step selection-bias update.
//
// y[t] = sum over kept slots j (slot order) of gate[t,j] * o[row_of_slot[t,j]]
// + shared[t] ("Mixture of Experts Explained", "What is sparsity?": the
// gate-weighted sum of expert outputs; dropped slots add nothing, the token
// travels on through the caller's residual, "MoEs and Transformers").
#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace moe {

// One wave per token; each lane owns 4 consecutive floats per 256-float slab.
// A token's slot rows are the same for the whole wave, so each slot row is
// read through its own buffer descriptor (an empty one for a dropped slot,
// whose loads return zeros): the loads of all KM slots of a slab go out
// together with no branch, instead of one load round trip per slot.  The
// slot sum keeps its fixed order and skips dropped slots.
template <int KM>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o,
                                                      const int32_t* __restrict__ row_of_slot,
                                                      const float* __restrict__ gate,
                                                      const float* __restrict__ shared, int T,
                                                      int k, int d, float* __restrict__ y) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;
  // lane j fetches slot j's row and gate; every lane then takes them as scalars
  const int my_row = l < k ? row_of_slot[int64_t(t) * k + l] : -1;
  const float my_g = l < k ? gate[int64_t(t) * k + l] : 0.0f;
  int rows[KM];
  float gs[KM];
  rsrc_t rs[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    rows[j] = __builtin_amdgcn_readlane(my_row, j);
    gs[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_g), j));
    rs[j] = make_rsrc(rows[j] >= 0 ? o + int64_t(rows[j]) * d : o, rows[j] >= 0 ? uint32_t(d) * 4 : 0u);
  }
  const int nv = d >> 2;
  for (int c = l; c < nv; c += 64) {
    floatx4 v[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      v[j] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs[j], uint32_t(c) * 16, 0, 0));
    float4 acc = shared ? reinterpret_cast<const float4*>(shared + int64_t(t) * d)[c]
                        : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (rows[j] < 0) continue;
      acc.x = fmaf(gs[j], v[j][0], acc.x);
      acc.y = fmaf(gs[j], v[j][1], acc.y);
      acc.z = fmaf(gs[j], v[j][2], acc.z);
      acc.w = fmaf(gs[j], v[j][3], acc.w);
    }
    reinterpret_cast<float4*>(y + int64_t(t) * d)[c] = acc;
  }
}

// bias[e] += gamma * sign(target - counts[e]), sign(0) = 0 (handbook news
// digest, "confirmed": the fixed-step loss-free bias update).
__global__ void bias_update_kernel(const int32_t* __restrict__ counts, float* __restrict__ bias,
                                   int E, float target, float gamma) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const float c = float(counts[e]);
  const float sgn = target > c ? 1.0f : (target < c ? -1.0f : 0.0f);
  bias[e] = bias[e] + gamma * sgn;
}

// out[i] = v[i] for i < n (n <= 4): tiny device-side constants (group offsets).
__global__ void fill_i32_kernel(int32_t* out, int n, int32_t v0, int32_t v1, int32_t v2, int32_t v3) {
  const int i = threadIdx.x;
  if (i < n) out[i] = i == 0 ? v0 : i == 1 ? v1 : i == 2 ? v2 : v3;
}

// out[i] = min(i * step, cap), i = 0..n-1 (row offsets of equal chunks)
__global__ void fill_seq_i32_kernel(int32_t* out, int n, int32_t step, int32_t cap) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = int32_t(min(int64_t(i) * step, int64_t(cap)));
}

// Several fill_seq tables in one launch: block y fills table y.
__global__ void fill_seqs_kernel(SeqFills f) {
  const int y = blockIdx.y;
  if (y >= f.count) return;
  for (int i = threadIdx.x; i < f.n[y]; i += blockDim.x)
    f.out[y][i] = int32_t(min(int64_t(i) * f.step[y], int64_t(f.cap[y])));
}

hipError_t launch_fill_seqs(const SeqFills& f, hipStream_t st) {
  if (f.count <= 0) return hipSuccess;
  if (f.count > 8) return hipErrorInvalidValue;
  fill_seqs_kernel<<<dim3(1, unsigned(f.count)), dim3(256), 0, st>>>(f);
  return hipGetLastError();
}

__global__ void zero_i32_kernel(int32_t* out, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = 0;
}

hipError_t launch_fill_seq_i32(int32_t* out, int n, int32_t step, int32_t cap, hipStream_t st) {
  fill_seq_i32_kernel<<<dim3(unsigned(cdiv(n, 256))), dim3(256), 0, st>>>(out, n, step, cap);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* out, int n, int32_t v0, int32_t v1, int32_t v2, int32_t v3,
                           hipStream_t st) {
  fill_i32_kernel<<<dim3(1), dim3(64), 0, st>>>(out, n, v0, v1, v2, v3);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int32_t* out, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  zero_i32_kernel<<<dim3(unsigned(cdiv(n, 256))), dim3(256), 0, st>>>(out, n);
  return hipGetLastError();
}

hipError_t launch_combine(const float* o, const int32_t* row_of_slot, const float* gate,
                          const float* shared, int T, int k, int d, float* y, hipStream_t st) {
  const dim3 grid(unsigned(cdiv(T, 4))), block(256);
  if (k <= 1) combine_kernel<1><<<grid, block, 0, st>>>(o, row_of_slot, gate, shared, T, k, d, y);
  else if (k <= 2) combine_kernel<2><<<grid, block, 0, st>>>(o, row_of_slot, gate, shared, T, k, d, y);
  else if (k <= 4) combine_kernel<4><<<grid, block, 0, st>>>(o, row_of_slot, gate, shared, T, k, d, y);
  else if (k <= 8) combine_kernel<8><<<grid, block, 0, st>>>(o, row_of_slot, gate, shared, T, k, d, y);
  else combine_kernel<16><<<grid, block, 0, st>>>(o, row_of_slot, gate, shared, T, k, d, y);
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts, float* bias, int E, float target,
                              float gamma, hipStream_t st) {
  bias_update_kernel<<<dim3(unsigned(cdiv(E, 256))), dim3(256), 0, st>>>(counts, bias, E, target,
                                                                          gamma);
  return hipGetLastError();
}

}  // namespace moe
