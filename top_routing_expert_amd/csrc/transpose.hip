// Transposes used by the backward pass of the MoE layer (gfx950).
//
// The weight-gradient GEMMs reduce over the rows of each expert, and the
// data-gradient GEMMs multiply by the weights in the other orientation.  The
// MFMA operands want the reduction index contiguous, so the backward first
// writes transposed copies:
//   * batched transpose: out[b][c][r] = in[b][r][c] (weights [E][n][d] -> [E][d][n]);
//   * group-padded transpose of expert-contiguous rows: for group g with rows
//     offsets[g]..offsets[g+1]-1, out_g[c][m] = in[offsets[g] + m][c] for
//     m < M_g and 0 up to Kp_g = M_g rounded up to 64; group g starts at
//     element C * koff_g, koff_g = sum of Kp over the groups before g.
// Both go through a 64x64 LDS tile so reads and writes are row-contiguous.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int TT = 64;   // tile edge

template <typename T>
__device__ __forceinline__ void tile_copy(const T* __restrict__ in, int64_t in_ld, int rows_valid,
                                          int cols_valid, T* __restrict__ out, int64_t out_ld,
                                          int out_rows_valid, int out_cols_valid, T (*s)[TT + 1]) {
  // in: tile origin, rows_valid x cols_valid readable; out: transposed origin
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;   // 64 x 4 threads
#pragma unroll 4
  for (int r = ty; r < TT; r += 4)
    s[r][tx] = (r < rows_valid && tx < cols_valid) ? in[int64_t(r) * in_ld + tx] : T(0);
  __syncthreads();
#pragma unroll 4
  for (int c = ty; c < TT; c += 4)
    if (c < out_rows_valid && tx < out_cols_valid) out[int64_t(c) * out_ld + tx] = s[tx][c];
}

template <typename T>
__global__ __launch_bounds__(256) void batched_transpose_kernel(const T* __restrict__ in, int R,
                                                                int Cc, T* __restrict__ out) {
  __shared__ T s[TT][TT + 1];
  const int64_t b = blockIdx.z;
  const int r0 = blockIdx.y * TT, c0 = blockIdx.x * TT;
  const T* src = in + b * R * int64_t(Cc) + int64_t(r0) * Cc + c0;
  T* dst = out + b * R * int64_t(Cc) + int64_t(c0) * R + r0;
  const int rv = min(TT, R - r0), cv = min(TT, Cc - c0);
  tile_copy<T>(src, Cc, rv, cv, dst, R, cv, rv, s);
}

// Exclusive scan over groups of Kp = roundup(M_g, 64) into ks[0..G] (LDS, 257
// entries), 256 threads, G <= 256.  Returns ks[G].
__device__ __forceinline__ int32_t scan_padded(const int32_t* offsets, int G, int32_t* ks) {
  const int tid = threadIdx.x;
  ks[tid + 1] = tid < G ? ((offsets[tid + 1] - offsets[tid] + 63) & ~63) : 0;
  if (tid == 0) ks[0] = 0;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int32_t v = tid >= o ? ks[tid + 1 - o] : 0;
    __syncthreads();
    ks[tid + 1] += v;
    __syncthreads();
  }
  return ks[G];
}

// grid.x over column tiles, grid.y over 64-row tiles of the padded row space.
template <typename T>
__global__ __launch_bounds__(256) void group_transpose_kernel(const T* __restrict__ in, int Cc,
                                                              const int32_t* __restrict__ offsets,
                                                              int G, T* __restrict__ out) {
  __shared__ T s[TT][TT + 1];
  __shared__ int32_t ks[257];
  const int32_t total = scan_padded(offsets, G, ks);
  const int p0 = blockIdx.y * TT;           // padded row of this tile
  if (p0 >= total) return;
  int lo = 0, hi = G;                        // group with ks[g] <= p0 < ks[g+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ks[mid] <= p0) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int m0 = p0 - ks[g];                 // row inside the group
  const int Mg = offsets[g + 1] - offsets[g];
  const int Kp = ks[g + 1] - ks[g];
  const int c0 = blockIdx.x * TT;
  const T* src = in + int64_t(offsets[g] + m0) * Cc + c0;
  T* dst = out + int64_t(Cc) * ks[g] + int64_t(c0) * Kp + m0;
  const int rv = max(0, min(TT, Mg - m0)), cv = min(TT, Cc - c0);
  // rows past M_g are read as 0 and written (the padding must be zero)
  tile_copy<T>(src, Cc, rv, cv, dst, Kp, cv, TT, s);
}

hipError_t launch_batched_transpose(const void* in, int batch, int R, int Cc, int elem_bytes,
                                    void* out, hipStream_t st) {
  const dim3 grid(unsigned(cdiv(Cc, TT)), unsigned(cdiv(R, TT)), unsigned(batch));
  if (elem_bytes == 2)
    batched_transpose_kernel<uint16_t><<<grid, dim3(256), 0, st>>>(
        static_cast<const uint16_t*>(in), R, Cc, static_cast<uint16_t*>(out));
  else
    batched_transpose_kernel<float><<<grid, dim3(256), 0, st>>>(static_cast<const float*>(in), R,
                                                                Cc, static_cast<float*>(out));
  return hipGetLastError();
}

hipError_t launch_group_transpose(const void* in, int Cc, const int32_t* offsets, int G,
                                  int64_t max_rows, int elem_bytes, void* out, hipStream_t st) {
  const int64_t padded = cdiv(max_rows, TT) * TT + int64_t(TT) * G;
  const dim3 grid(unsigned(cdiv(Cc, TT)), unsigned(padded / TT));
  if (elem_bytes == 2)
    group_transpose_kernel<uint16_t><<<grid, dim3(256), 0, st>>>(
        static_cast<const uint16_t*>(in), Cc, offsets, G, static_cast<uint16_t*>(out));
  else
    group_transpose_kernel<float><<<grid, dim3(256), 0, st>>>(static_cast<const float*>(in), Cc,
                                                              offsets, G, static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace moe
