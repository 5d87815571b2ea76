// Grouped expert GEMM on bf16 MFMA for gfx950 (the expert FFN of the MoE
// layer: "Mixture of Experts Explained", "Making MoEs go brrr" — experts run
// as grouped, not branchy, computation over expert-contiguous rows).
//
// out[rows of g] = epilogue(A[rows of g] . B[g]^T), A [rows, K] and B [g][n, K]
// both K-contiguous (B in the [out, in] layout), fp32 accumulation.
//
// Design for CDNA4:
//  * 256 threads = 4 waves in a 2x2 grid; each wave owns a (BM/2) x (BN/2)
//    sub-tile of every panel as (BM/64) x (BN/64) blocks of
//    v_mfma_f32_32x32x16_bf16.  With BM = BN = 256 a wave issues 16 MFMAs per
//    8 LDS fragment reads, half the LDS bytes per MFMA of a 64x64 wave tile.
//  * Global -> LDS with global_load_lds_dwordx4 (no staging registers): each
//    wave instruction fills 1 KB = 8 tile rows of 64 bf16.  The eight 16-byte
//    chunks of a row are XOR-swizzled by swz(row) = (row & 7) ^ ((row >> 3) & 1),
//    which keeps a fragment read conflict-free whether the LDS serves 8 lanes
//    (128 B) or 16 lanes (256 B) per pass; the swizzle is applied on the source
//    address a lane loads, since the LDS slot is fixed by the lane.
//    Two K stages of 64 are double buffered: the loads of stage k+1 are in
//    flight while stage k multiplies.
//  * The tile plan (per-group prefix of tile counts) is computed by every
//    workgroup from the device-resident row offsets: no planner launch and no
//    host synchronisation.  Rows past a group's end are clamped to its last
//    row on load and never stored.
//  * Workgroups are dealt round-robin to the 8 XCDs; block b takes logical
//    tile (b % 8) * ceil(tiles / 8) + b / 8, so each XCD works through a
//    contiguous run of tiles (same expert, consecutive n-tiles, m-tiles
//    fastest) and its L2 holds the shared A rows and weight panels.
//  * NP = 2 (SwiGLU): the gate rows n0.. and up rows up_off+n0.. of W13 are
//    two B panels multiplied against one A tile; the epilogue forms
//    silu(gate) * up directly.
#include "gemm_common.hpp"

namespace moe {

constexpr int GB_BK = 64;

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane l writes lds_wave_base + 16*l; the LDS pointer must be wave-uniform.  (A
// plain function: the builtin called from a lambda inside a kernel template
// breaks the host-side instantiation.)
__device__ __forceinline__ void lds_load16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 0);
}

// Row mode: ts[g] = tiles of the groups before g (ceil(M_g/BM) * N/BN each).
// K mode: ts[g] = padded rows of the groups before g (koff_g); the tile count
// is G * (M_fixed/BM) * (N/BN).  Returns the number of tiles.
template <int BM, int BN, int KG>
__device__ __forceinline__ int32_t plan_tiles(const GemmArgs& g, int32_t* ts) {
  const int tid = threadIdx.x;
  const int NT = g.N / BN;
  if constexpr (KG) {
    ts[tid + 1] = tid < g.G ? ((g.offsets[tid + 1] - g.offsets[tid] + 63) & ~63) : 0;
  } else {
    ts[tid + 1] = tid < g.G ? int32_t(cdiv(g.offsets[tid + 1] - g.offsets[tid], BM)) * NT : 0;
  }
  if (tid == 0) ts[0] = 0;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int32_t v = tid >= o ? ts[tid + 1 - o] : 0;
    __syncthreads();
    ts[tid + 1] += v;
    __syncthreads();
  }
  if constexpr (KG) return g.G * (g.M_fixed / BM) * NT;
  return ts[g.G];
}

template <int BM, int BN, int NP, int EPI, int KG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gg_bf16_kernel(GemmArgs g) {
  constexpr int ROWS = BM + NP * BN;     // 128-byte LDS rows per stage
  constexpr int STAGE = ROWS * 8;        // uint4 per stage
  constexpr int MI = BM / 64, NI = BN / 64;
  constexpr int A_INS = BM / 32, B_INS = BN / 32;  // load instructions per wave per panel
  // Two stages of (BM + NP*BN) rows x 128 bytes: up to 128 KB, dynamic LDS.
  extern __shared__ uint4 lds[];
  __shared__ int32_t ts[257];

  const int32_t total = plan_tiles<BM, BN, KG>(g, ts);
  const int per = (total + 7) >> 3;
  const int bid = blockIdx.x;
  const int tile = (bid & 7) * per + (bid >> 3);
  if ((bid >> 3) >= per || tile >= total) return;
  TileCoord tc;
  int K;                                     // reduction length of this tile
  const uint16_t* A;
  const uint16_t* B;
  if constexpr (KG) {
    const int MT = g.M_fixed / BM;
    const int tpg = MT * (g.N / BN);
    tc.grp = tile / tpg;
    const int local = tile - tc.grp * tpg;
    tc.m0 = (local % MT) * BM;
    tc.n0 = (local / MT) * BN;
    tc.row0 = 0;
    tc.M = g.M_fixed;
    K = ts[tc.grp + 1] - ts[tc.grp];
    A = static_cast<const uint16_t*>(g.A) + int64_t(g.M_fixed) * ts[tc.grp];
    B = static_cast<const uint16_t*>(g.B) + int64_t(g.N) * ts[tc.grp];
  } else {
    locate_tile(ts, g.offsets, g.G, tile, BM, BN, tc);
    K = g.K;
    A = static_cast<const uint16_t*>(g.A);
    B = static_cast<const uint16_t*>(g.B) + int64_t(tc.grp) * g.b_group_stride;
  }

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wm = w >> 1, wn = w & 1;

  // Lane l of a load instruction fills LDS slot l of an 8-row group: row l/8,
  // physical chunk l%8, which holds logical chunk (l%8) ^ swz(row).  Every
  // 8-row group this wave fills starts at a row with (row >> 3) & 1 == w & 1.
  const int lrow = l >> 3;
  const int lchunk = (l & 7) ^ lrow ^ (w & 1);
  const uint16_t* a_src[A_INS];
#pragma unroll
  for (int i = 0; i < A_INS; ++i) {
    const int mr = min(tc.m0 + 8 * (w + 4 * i) + lrow, tc.M - 1);
    a_src[i] = A + int64_t(tc.row0 + mr) * K + 8 * lchunk;
  }
  const uint16_t* b_src[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p)
    b_src[p] = B + int64_t(p * g.up_off + tc.n0 + 8 * w + lrow) * K + 8 * lchunk;
  const int64_t b_step = int64_t(32) * K;   // 32 rows between a wave's B instructions

  auto issue = [&](int stage, int k0) {
    uint4* base = lds + stage * STAGE;
#pragma unroll
    for (int i = 0; i < A_INS; ++i) lds_load16(a_src[i] + k0, base + (w + 4 * i) * 64);
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int i = 0; i < B_INS; ++i)
        lds_load16(b_src[p] + i * b_step + k0, base + (BM + p * BN) * 8 + (w + 4 * i) * 64);
  };

  floatx16 acc[NP][MI][NI];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[p][mi][ni][r] = 0.0f;

  const int fr = l & 31, fg = l >> 5;
  const int KT = K / GB_BK;
  // Each tile walks the K stages starting at its own offset (tile mod KT):
  // concurrent tiles read different K columns, which spreads their requests
  // over the L2 channels instead of having every CU hit the same channel with
  // the same power-of-two row stride.  The sum order depends only on the tile.
  const int krot = KT > 0 ? tile % KT : 0;
  if (KT > 0) issue(0, krot * GB_BK);
  __syncthreads();
  // Fragments of K-step s+1 are read from LDS while the MFMAs of step s run.
  bf16x8 af[2][MI], bfr[2][NP][NI];
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) {
      const int kn = kt + 1 + krot;
      issue(cur ^ 1, (kn < KT ? kn : kn - KT) * GB_BK);
    }
    const uint4* As = lds + cur * STAGE;
#pragma unroll
    for (int s = 0; s <= 4; ++s) {
      if (s < 4) {
        const int pc = (2 * s + fg) ^ (fr & 7) ^ ((fr >> 3) & 1);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          af[s & 1][mi] = __builtin_bit_cast(bf16x8, As[(wm * (BM / 2) + mi * 32 + fr) * 8 + pc]);
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            bfr[s & 1][p][ni] = __builtin_bit_cast(
                bf16x8, As[(BM + p * BN + wn * (BN / 2) + ni * 32 + fr) * 8 + pc]);
      }
      if (s > 0) {
        const int q = (s - 1) & 1;
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
              acc[p][mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  af[q][mi], bfr[q][p][ni], acc[p][mi][ni], 0, 0, 0);
      }
      // Keep this order in the schedule: the LDS reads of step s, then the
      // MFMAs of step s-1 (otherwise the scheduler sinks every read next to
      // its use and each MFMA group waits on LDS latency).
      if (s < 4) __builtin_amdgcn_sched_group_barrier(0x100, MI + NP * NI, 0);
      if (s > 0) __builtin_amdgcn_sched_group_barrier(0x008, NP * MI * NI, 0);
    }
    __syncthreads();
  }

  // Epilogue through LDS (free after the last barrier).  Per 32-row block mi,
  // each wave writes its accumulators (register r of lane l holds row
  // 8*(r/4) + 4*(l/32) + r%4, column l%32 of a 32x32 block) into its own
  // [NP][32][BN/2 + 4] fp32 region, then reads rows back four columns per lane
  // and stores 16 bytes (fp32) or 8 bytes (bf16) per lane, row-contiguous.
  constexpr int CST = BN / 2 + 4;
  constexpr int LPR = (BN / 2) / 4;   // lanes per row
  constexpr int RPI = 64 / LPR;       // rows per read-back step
  float* cw = reinterpret_cast<float*>(lds) + w * (NP * 32 * CST);
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          cw[(p * 32 + 8 * (r >> 2) + 4 * fg + (r & 3)) * CST + ni * 32 + fr] = acc[p][mi][ni][r];
    __syncthreads();
    const int c4 = (l % LPR) * 4;
    const int n = tc.n0 + wn * (BN / 2) + c4;
#pragma unroll 4
    for (int it = 0; it < 32 / RPI; ++it) {
      const int rl = it * RPI + l / LPR;
      const int mr = tc.m0 + wm * (BM / 2) + mi * 32 + rl;
      if (mr < tc.M) {
        const int64_t row = tc.row0 + mr;
        const float4 v0 = *reinterpret_cast<const float4*>(cw + rl * CST + c4);
        if constexpr (EPI == EPI_STORE_F32) {
          float* outp = static_cast<float*>(g.out) + (KG ? int64_t(tc.grp) * g.M_fixed * g.N : 0);
          *reinterpret_cast<float4*>(outp + row * g.N + n) = v0;
        } else if constexpr (EPI == EPI_SWIGLU_BWD) {
          // v0 = dA[row, n..n+3]; h_in row = [gate | up]; out row = [dgate | dup]
          const uint16_t* hr = static_cast<const uint16_t*>(g.h_in) + row * g.n_b;
          const float4 hg = unpack_bf4(*reinterpret_cast<const uint2*>(hr + n));
          const float4 hu = unpack_bf4(*reinterpret_cast<const uint2*>(hr + g.up_off + n));
          uint16_t* orow = static_cast<uint16_t*>(g.out) + row * g.n_b;
          *reinterpret_cast<uint2*>(orow + n) =
              make_uint2(pack_bf2(v0.x * hu.x * dsilu(hg.x), v0.y * hu.y * dsilu(hg.y)),
                         pack_bf2(v0.z * hu.z * dsilu(hg.z), v0.w * hu.w * dsilu(hg.w)));
          *reinterpret_cast<uint2*>(orow + g.up_off + n) =
              make_uint2(pack_bf2(v0.x * silu(hg.x), v0.y * silu(hg.y)),
                         pack_bf2(v0.z * silu(hg.z), v0.w * silu(hg.w)));
        } else if constexpr (EPI == EPI_GELU_BWD) {
          const float4 h = unpack_bf4(
              *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(g.h_in) + row * g.n_b + n));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.out) + row * g.n_b + n) =
              make_uint2(pack_bf2(v0.x * dgelu_erf(h.x), v0.y * dgelu_erf(h.y)),
                         pack_bf2(v0.z * dgelu_erf(h.z), v0.w * dgelu_erf(h.w)));
        } else if constexpr (EPI == EPI_GELU) {
          if (g.h_save)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.h_save) + row * g.n_b + n) =
                make_uint2(pack_bf2(v0.x, v0.y), pack_bf2(v0.z, v0.w));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.out) + row * g.N + n) =
              make_uint2(pack_bf2(gelu_erf(v0.x), gelu_erf(v0.y)),
                         pack_bf2(gelu_erf(v0.z), gelu_erf(v0.w)));
        } else {
          const float4 v1 = *reinterpret_cast<const float4*>(cw + (32 + rl) * CST + c4);
          if (g.h_save) {
            uint16_t* hs = static_cast<uint16_t*>(g.h_save) + row * g.n_b;
            *reinterpret_cast<uint2*>(hs + n) = make_uint2(pack_bf2(v0.x, v0.y), pack_bf2(v0.z, v0.w));
            *reinterpret_cast<uint2*>(hs + g.up_off + n) =
                make_uint2(pack_bf2(v1.x, v1.y), pack_bf2(v1.z, v1.w));
          }
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.out) + row * g.N + n) =
              make_uint2(pack_bf2(silu(v0.x) * v1.x, silu(v0.y) * v1.y),
                         pack_bf2(silu(v0.z) * v1.z, silu(v0.w) * v1.w));
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
template <int BM, int BN, int NP, int EPI, int KG>
void launch_cfg(const GemmArgs& g, hipStream_t st) {
  const int64_t bound = KG ? int64_t(g.G) * (g.M_fixed / BM) * (g.N / BN)
                           : (cdiv(g.max_rows, BM) + g.G) * (g.N / BN);
  const unsigned grid = unsigned(cdiv(bound, 8) * 8);
  constexpr size_t lds_bytes = size_t(2) * (BM + NP * BN) * 128;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gg_bf16_kernel<BM, BN, NP, EPI, KG>),
      hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_bytes));
  (void)attr;
  gg_bf16_kernel<BM, BN, NP, EPI, KG><<<dim3(grid), dim3(256), lds_bytes, st>>>(g);
}

template <int EPI>
static void launch_rows_np1(const GemmArgs& g, bool bm256, bool bn256, hipStream_t st) {
  if (bm256) {
    if (bn256) launch_cfg<256, 256, 1, EPI, 0>(g, st); else launch_cfg<256, 128, 1, EPI, 0>(g, st);
  } else {
    if (bn256) launch_cfg<128, 256, 1, EPI, 0>(g, st); else launch_cfg<128, 128, 1, EPI, 0>(g, st);
  }
}

// Tile shape (row mode): 256-row tiles when groups average at least 192 rows
// (fewer re-reads of each weight panel), else 128; 256-column tiles when that
// still gives a tile per CU, else 128.  K mode: 256 x 256 when the output
// dimensions allow it.
hipError_t launch_grouped_gemm_bf16(const GemmArgs& g, hipStream_t st) {
  if (g.G == 0) return hipSuccess;
  if (g.kgroup) {
    if (g.epi != EPI_STORE_F32) return hipErrorInvalidValue;
    const bool m256 = g.M_fixed % 256 == 0, n256 = g.N % 256 == 0;
    if (m256 && n256) launch_cfg<256, 256, 1, EPI_STORE_F32, 1>(g, st);
    else if (m256) launch_cfg<256, 128, 1, EPI_STORE_F32, 1>(g, st);
    else if (n256) launch_cfg<128, 256, 1, EPI_STORE_F32, 1>(g, st);
    else launch_cfg<128, 128, 1, EPI_STORE_F32, 1>(g, st);
    return hipGetLastError();
  }
  if (g.max_rows == 0) return hipSuccess;
  const int64_t avg = g.max_rows / g.G;
  const bool bm256 = avg >= 192;
  const int64_t mt = cdiv(g.max_rows, bm256 ? 256 : 128);
  const bool bn256 = (g.N % 256 == 0) && mt * (g.N / 256) >= 256;
  switch (g.epi) {
    case EPI_STORE_F32: launch_rows_np1<EPI_STORE_F32>(g, bm256, bn256, st); break;
    case EPI_GELU: launch_rows_np1<EPI_GELU>(g, bm256, bn256, st); break;
    case EPI_SWIGLU_BWD: launch_rows_np1<EPI_SWIGLU_BWD>(g, bm256, bn256, st); break;
    case EPI_GELU_BWD: launch_rows_np1<EPI_GELU_BWD>(g, bm256, bn256, st); break;
    case EPI_SWIGLU:
      if (bm256) launch_cfg<256, 128, 2, EPI_SWIGLU, 0>(g, st);
      else launch_cfg<128, 128, 2, EPI_SWIGLU, 0>(g, st);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
