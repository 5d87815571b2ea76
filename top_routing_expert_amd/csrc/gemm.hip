// Grouped expert GEMM of the sparse MoE layer for gfx950.
//
// Rows of each expert are contiguous ("Mixture of Experts Explained", "Making
// MoEs go brrr": uneven per-expert batches want grouped, not branchy,
// computation).  out[rows of g] = epilogue(A[rows of g] . B[g]^T), B in the
// [out, in] layout.  The row counts live on the device: a one-block planner
// turns offsets into a prefix of tile counts and every workgroup finds its
// (group, m-tile, n-tile) by binary search, so no host synchronisation is
// needed.  Epilogues: fp32 store (down projection), exact GELU, or SwiGLU with
// the gate and up projections computed by the same workgroup from one A tile.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int BF_BM = 128, BF_BN = 128, BF_BK = 64;   // bf16 MFMA tile
constexpr int F32_BM = 64, F32_BN = 64, F32_BK = 16;  // fp32 FMA tile

int64_t gemm_tile_bound(int64_t max_rows, int G, int N, bool bf16) {
  const int bm = bf16 ? BF_BM : F32_BM, bn = bf16 ? BF_BN : F32_BN;
  return (cdiv(max_rows, bm) + G) * cdiv(N, bn);
}

// tile_start[g] = sum over groups before g of ceil(M_g / BM) * (N / BN).
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

struct TileCoord {
  int grp, row0, M, m0, n0;
};

// Largest group whose first tile is <= tile (empty groups own no tile).
__device__ __forceinline__ bool find_tile(const GemmArgs& g, int tile, int BM, int BN,
                                          TileCoord& tc) {
  const int32_t* ts = g.tile_start;
  if (tile >= ts[g.G]) return false;
  int lo = 0, hi = g.G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ts[mid] <= tile) lo = mid; else hi = mid;
  }
  const int local = tile - ts[lo];
  const int row0 = g.offsets[lo];
  const int M = g.offsets[lo + 1] - row0;
  const int mt = int(cdiv(M, BM));
  tc.grp = lo;
  tc.row0 = row0;
  tc.M = M;
  tc.m0 = (local % mt) * BM;
  tc.n0 = (local / mt) * BN;
  return true;
}

__device__ __forceinline__ float gelu_erf(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }
__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.  256 threads = 4 waves in a 2x2 grid, each wave a 64x64
// sub-tile of every panel (2x2 MFMA 32x32x16 blocks).  NP = 2 for SwiGLU: the
// gate rows n0.. and the up rows up_off+n0.. are two B panels sharing A.
// LDS tiles are [row][64 k] with the eight 16-byte chunks of a row XOR-swizzled
// by (row & 7), double buffered; global loads for step k+1 are in flight
// while step k multiplies.
template <int EPI, int NP>
__global__ __launch_bounds__(256) void gg_bf16_kernel(GemmArgs g) {
  __shared__ uint4 lds[2 * (1 + NP) * BF_BM * BF_BK / 8];
  TileCoord tc;
  if (!find_tile(g, blockIdx.x, BF_BM, BF_BN, tc)) return;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wm = w >> 1, wn = w & 1;
  const int K = g.K;
  const uint16_t* A = static_cast<const uint16_t*>(g.A);
  const uint16_t* B = static_cast<const uint16_t*>(g.B) + int64_t(tc.grp) * g.b_group_stride;

  constexpr int TILE16 = BF_BM * BF_BK / 8;  // uint4 per tile
  auto As = [&](int buf) { return lds + buf * (1 + NP) * TILE16; };
  auto Bs = [&](int buf, int p) { return lds + buf * (1 + NP) * TILE16 + (1 + p) * TILE16; };

  // global -> register staging: thread covers chunk c of rows r, r+32, r+64, r+96
  const int lc = tid & 7, lr = tid >> 3;
  const uint16_t* a_src[4];
  bool a_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mr = tc.m0 + lr + 32 * i;
    a_ok[i] = mr < tc.M;
    a_src[i] = A + int64_t(tc.row0 + (a_ok[i] ? mr : 0)) * K + 8 * lc;
  }
  const uint16_t* b_src[NP][4];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      b_src[p][i] = B + int64_t(p * g.up_off + tc.n0 + lr + 32 * i) * K + 8 * lc;

  uint4 ra[4], rb[NP][4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = a_ok[i] ? ld16(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) rb[p][i] = ld16(b_src[p][i] + k0);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lr + 32 * i;
      const int slot = row * 8 + (lc ^ (row & 7));
      As(buf)[slot] = ra[i];
#pragma unroll
      for (int p = 0; p < NP; ++p) Bs(buf, p)[slot] = rb[p][i];
    }
  };

  floatx16 acc[NP][2][2];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[p][mi][ni][r] = 0.0f;

  const int fr = l & 31, fg = l >> 5;
  const int KT = K / BF_BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BF_BK);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + fg;
      bf16x8 af[2], bfr[NP][2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int row = wm * 64 + mi * 32 + fr;
        af[mi] = __builtin_bit_cast(bf16x8, As(buf)[row * 8 + (ch ^ (row & 7))]);
      }
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int row = wn * 64 + ni * 32 + fr;
          bfr[p][ni] = __builtin_bit_cast(bf16x8, Bs(buf, p)[row * 8 + (ch ^ (row & 7))]);
        }
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[p][mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[p][ni],
                                                                     acc[p][mi][ni], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  Accumulator register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32 of its 32x32 block.
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mr = tc.m0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * fg + (r & 3);
        if (mr >= tc.M) continue;
        const int64_t row = tc.row0 + mr;
        const int n = tc.n0 + wn * 64 + ni * 32 + fr;
        const float v0 = acc[0][mi][ni][r];
        if constexpr (EPI == EPI_STORE_F32) {
          static_cast<float*>(g.out)[row * g.N + n] = v0;
        } else if constexpr (EPI == EPI_GELU) {
          if (g.h_save) static_cast<uint16_t*>(g.h_save)[row * g.n_b + n] = f2bf(v0);
          static_cast<uint16_t*>(g.out)[row * g.N + n] = f2bf(gelu_erf(v0));
        } else {
          const float v1 = acc[NP - 1][mi][ni][r];
          if (g.h_save) {
            static_cast<uint16_t*>(g.h_save)[row * g.n_b + n] = f2bf(v0);
            static_cast<uint16_t*>(g.h_save)[row * g.n_b + g.up_off + n] = f2bf(v1);
          }
          static_cast<uint16_t*>(g.out)[row * g.N + n] = f2bf(silu(v0) * v1);
        }
      }
}

// ---------------------------------------------------------------------------
// fp32 FMA kernel with the same planning and epilogues (fp32 storage).
// 256 threads, 64x64 tile per panel, each thread a 4x4 micro-tile.
template <int EPI, int NP>
__global__ __launch_bounds__(256) void gg_f32_kernel(GemmArgs g) {
  __shared__ float As[F32_BK][F32_BM + 4];
  __shared__ float Bs[NP][F32_BK][F32_BN + 4];
  TileCoord tc;
  if (!find_tile(g, blockIdx.x, F32_BM, F32_BN, tc)) return;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int K = g.K;
  const float* A = static_cast<const float*>(g.A);
  const float* B = static_cast<const float*>(g.B) + int64_t(tc.grp) * g.b_group_stride;
  float acc[NP][4][4];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[p][i][j] = 0.0f;
  // load mapping: 64 rows x 16 k = 1024 values, 4 per thread: row = tid/4, k = 4*(tid%4)..+3
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  for (int k0 = 0; k0 < K; k0 += F32_BK) {
    const int mr = tc.m0 + lrow;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kk = k0 + lk + q;
      As[lk + q][lrow] = (mr < tc.M && kk < K) ? A[int64_t(tc.row0 + mr) * K + kk] : 0.0f;
      const bool nok = tc.n0 + lrow < g.N && kk < K;
#pragma unroll
      for (int p = 0; p < NP; ++p)
        Bs[p][lk + q][lrow] = nok ? B[int64_t(p * g.up_off + tc.n0 + lrow) * K + kk] : 0.0f;
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
      float* out = static_cast<float*>(g.out);
      float* hs = static_cast<float*>(g.h_save);
      if constexpr (EPI == EPI_STORE_F32) {
        out[row * g.N + n] = v0;
      } else if constexpr (EPI == EPI_GELU) {
        if (hs) hs[row * g.n_b + n] = v0;
        out[row * g.N + n] = gelu_erf(v0);
      } else {
        const float v1 = acc[NP - 1][i][j];
        if (hs) {
          hs[row * g.n_b + n] = v0;
          hs[row * g.n_b + g.up_off + n] = v1;
        }
        out[row * g.N + n] = silu(v0) * v1;
      }
    }
  }
}

// ---------------------------------------------------------------------------
static hipError_t plan(const GemmArgs& g, int BM, int BN, hipStream_t st) {
  gemm_plan_kernel<<<dim3(1), dim3(256), 0, st>>>(g.offsets, g.G, BM, int(cdiv(g.N, BN)),
                                                  g.tile_start);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_bf16(const GemmArgs& g, hipStream_t st) {
  hipError_t e = plan(g, BF_BM, BF_BN, st);
  if (e != hipSuccess) return e;
  const unsigned grid = unsigned(gemm_tile_bound(g.max_rows, g.G, g.N, true));
  if (grid == 0) return hipSuccess;
  switch (g.epi) {
    case EPI_STORE_F32: gg_bf16_kernel<EPI_STORE_F32, 1><<<dim3(grid), dim3(256), 0, st>>>(g); break;
    case EPI_GELU: gg_bf16_kernel<EPI_GELU, 1><<<dim3(grid), dim3(256), 0, st>>>(g); break;
    case EPI_SWIGLU: gg_bf16_kernel<EPI_SWIGLU, 2><<<dim3(grid), dim3(256), 0, st>>>(g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_f32(const GemmArgs& g, hipStream_t st) {
  hipError_t e = plan(g, F32_BM, F32_BN, st);
  if (e != hipSuccess) return e;
  const unsigned grid = unsigned(gemm_tile_bound(g.max_rows, g.G, g.N, false));
  if (grid == 0) return hipSuccess;
  switch (g.epi) {
    case EPI_STORE_F32: gg_f32_kernel<EPI_STORE_F32, 1><<<dim3(grid), dim3(256), 0, st>>>(g); break;
    case EPI_GELU: gg_f32_kernel<EPI_GELU, 1><<<dim3(grid), dim3(256), 0, st>>>(g); break;
    case EPI_SWIGLU: gg_f32_kernel<EPI_SWIGLU, 2><<<dim3(grid), dim3(256), 0, st>>>(g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
