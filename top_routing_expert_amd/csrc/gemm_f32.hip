// Grouped expert GEMM, fp32 FMA version (fp32 layers), for gfx950.
//
// Same contract as the bf16 MFMA kernel (the three operand layouts, forward
// and backward epilogues), fp32 storage throughout.  A one-block
// planner writes the per-group tile prefix of the row mode; each workgroup
// locates its tile by binary search.
#include "gemm_common.hpp"

namespace moe {

constexpr int F32_BM = 64, F32_BN = 64, F32_BK = 16;

// tile_start[g] = sum over groups before g of ceil(M_g / BM) * NT.
__global__ __launch_bounds__(256) void gemm_plan_kernel(const int32_t* __restrict__ offsets, int G,
                                                        int BM, int NT,
                                                        int32_t* __restrict__ tile_start) {
  __shared__ int32_t s[256];
  int32_t carry = 0;
  for (int base = 0; base < G; base += 256) {
    const int gi = base + threadIdx.x;
    const int32_t mine = gi < G ? int32_t(cdiv(offsets[gi + 1] - offsets[gi], BM)) * NT : 0;
    s[threadIdx.x] = mine;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int32_t v = threadIdx.x >= o ? s[threadIdx.x - o] : 0;
      __syncthreads();
      s[threadIdx.x] += v;
      __syncthreads();
    }
    if (gi < G) tile_start[gi] = carry + s[threadIdx.x] - mine;
    carry += s[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) tile_start[G] = carry;
}

// 256 threads, 64x64 tile per panel, each thread a 4x4 micro-tile.  NP = 2 for
// SwiGLU (gate rows n0.., up rows up_off+n0..).  MODE as for the bf16 kernel:
// GM_NT reads B [g][n, K], GM_NN reads B [g][K, n], GM_KGROUP reduces over the
// rows of each group with A [rows, M_fixed] and B [rows, N].
template <int EPI, int NP, int MODE>
__global__ __launch_bounds__(256) void gg_f32_kernel(GemmArgs g) {
  __shared__ float As[F32_BK][F32_BM + 4];
  __shared__ float Bs[NP][F32_BK][F32_BN + 4];
  TileCoord tc;
  int K;
  const float* A;
  const float* B;
  float* out = static_cast<float*>(g.out);
  if constexpr (MODE == GM_KGROUP) {
    const int MT = int(cdiv(g.M_fixed, F32_BM)), NT = int(cdiv(g.N, F32_BN));
    const int tile = blockIdx.x;
    tc.grp = tile / (MT * NT);
    const int local = tile - tc.grp * MT * NT;
    tc.m0 = (local % MT) * F32_BM;
    tc.n0 = (local / MT) * F32_BN;
    tc.row0 = 0;
    tc.M = g.M_fixed;
    const int32_t r0 = g.offsets[tc.grp];
    K = g.offsets[tc.grp + 1] - r0;
    A = static_cast<const float*>(g.A) + int64_t(r0) * g.M_fixed;
    B = static_cast<const float*>(g.B) + int64_t(r0) * g.N;
    out += int64_t(tc.grp) * g.M_fixed * g.N;
  } else {
    const int32_t* ts = g.tile_start;
    if (int(blockIdx.x) >= ts[g.G]) return;
    locate_tile(ts, g.offsets, g.G, blockIdx.x, F32_BM, F32_BN, tc);
    K = g.K;
    A = static_cast<const float*>(g.A);
    B = static_cast<const float*>(g.B) + int64_t(tc.grp) * g.b_group_stride;
  }
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[NP][4][4];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[p][i][j] = 0.0f;
  // K-contiguous operands: thread loads row lrow, k = lk..lk+3.  K-major
  // operands: thread loads k row kr, columns kc..kc+3 (coalesced along the row).
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const int kr = tid >> 4, kc = (tid & 15) * 4;
  for (int k0 = 0; k0 < K; k0 += F32_BK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (MODE == GM_KGROUP) {
        const int kk = k0 + kr, m = tc.m0 + kc + q;
        As[kr][kc + q] = (kk < K && m < tc.M) ? A[int64_t(kk) * g.M_fixed + m] : 0.0f;
      } else {
        const int kk = k0 + lk + q, mr = tc.m0 + lrow;
        As[lk + q][lrow] = (mr < tc.M && kk < K) ? A[int64_t(tc.row0 + mr) * K + kk] : 0.0f;
      }
      if constexpr (MODE == GM_NT) {
        const int kk = k0 + lk + q;
        const bool nok = tc.n0 + lrow < g.N && kk < K;
#pragma unroll
        for (int p = 0; p < NP; ++p)
          Bs[p][lk + q][lrow] = nok ? B[int64_t(p * g.up_off + tc.n0 + lrow) * K + kk] : 0.0f;
      } else {
        const int kk = k0 + kr, n = tc.n0 + kc + q;
        Bs[0][kr][kc + q] = (kk < K && n < g.N) ? B[int64_t(kk) * g.N + n] : 0.0f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < F32_BK; ++kk) {
      float av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float bv = Bs[p][kk][tx * 4 + j];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[p][i][j] = fmaf(av[i], bv, acc[p][i][j]);
        }
    }
    __syncthreads();
  }
  float* hs = static_cast<float*>(g.h_save);
  const float* hin = static_cast<const float*>(g.h_in);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mr = tc.m0 + ty * 4 + i;
    if (mr >= tc.M) continue;
    const int64_t row = tc.row0 + mr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = tc.n0 + tx * 4 + j;
      if (n >= g.N) continue;
      const float v0 = acc[0][i][j];
      if constexpr (EPI == EPI_STORE_F32) {
        out[row * g.N + n] = v0;
      } else if constexpr (EPI == EPI_GELU) {
        if (hs) hs[row * g.n_b + n] = v0;
        out[row * g.N + n] = gelu_erf(v0);
      } else if constexpr (EPI == EPI_SWIGLU) {
        const float v1 = acc[NP - 1][i][j];
        if (hs) {
          hs[row * g.n_b + n] = v0;
          hs[row * g.n_b + g.up_off + n] = v1;
        }
        out[row * g.N + n] = silu(v0) * v1;
      } else if constexpr (EPI == EPI_SWIGLU_BWD) {
        const float hg = hin[row * g.n_b + n], hu = hin[row * g.n_b + g.up_off + n];
        out[row * g.n_b + n] = v0 * hu * dsilu(hg);
        out[row * g.n_b + g.up_off + n] = v0 * silu(hg);
      } else {
        out[row * g.n_b + n] = v0 * dgelu_erf(hin[row * g.n_b + n]);
      }
    }
  }
}

template <int EPI, int NP, int MODE>
static void launch_rows(const GemmArgs& g, unsigned grid, hipStream_t st) {
  gg_f32_kernel<EPI, NP, MODE><<<dim3(grid), dim3(256), 0, st>>>(g);
}

hipError_t launch_grouped_gemm_f32(const GemmArgs& g, hipStream_t st) {
  if (g.ldb && g.ldb != g.N) return hipErrorInvalidValue;   // B row stride: N only
  if (g.G == 0) return hipSuccess;
  const int NT = int(cdiv(g.N, F32_BN));
  if (g.mode == GM_KGROUP) {
    if (g.epi != EPI_STORE_F32) return hipErrorInvalidValue;
    const unsigned grid = unsigned(int64_t(g.G) * cdiv(g.M_fixed, F32_BM) * NT);
    gg_f32_kernel<EPI_STORE_F32, 1, GM_KGROUP><<<dim3(grid), dim3(256), 0, st>>>(g);
    return hipGetLastError();
  }
  gemm_plan_kernel<<<dim3(1), dim3(256), 0, st>>>(g.offsets, g.G, F32_BM, NT, g.tile_start);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned grid = unsigned((cdiv(g.max_rows, F32_BM) + g.G) * NT);
  if (grid == 0) return hipSuccess;
  if (g.mode == GM_NN) {
    switch (g.epi) {
      case EPI_STORE_F32: launch_rows<EPI_STORE_F32, 1, GM_NN>(g, grid, st); break;
      case EPI_SWIGLU_BWD: launch_rows<EPI_SWIGLU_BWD, 1, GM_NN>(g, grid, st); break;
      case EPI_GELU_BWD: launch_rows<EPI_GELU_BWD, 1, GM_NN>(g, grid, st); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (g.epi) {
    case EPI_STORE_F32: launch_rows<EPI_STORE_F32, 1, GM_NT>(g, grid, st); break;
    case EPI_GELU: launch_rows<EPI_GELU, 1, GM_NT>(g, grid, st); break;
    case EPI_SWIGLU: launch_rows<EPI_SWIGLU, 2, GM_NT>(g, grid, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
