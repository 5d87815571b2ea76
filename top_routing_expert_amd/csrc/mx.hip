// MXFP4 routed experts for inference on gfx950 (Ultimate MoE Training Handbook
// news: Kimi K3 quantises its routed experts to MXFP4), with the OCP
// Microscaling formats: FP4 E2M1 weights with one E8M0 scale per 32 k, FP8 E4M3
// activations with one E8M0 scale per 64 k.
//
// Quantisers: a block's shared exponent is floor(log2(max|v|)) minus the
// element type's largest exponent (2 for E2M1, 8 for E4M3), the scale code
// that exponent + 127 clamped to [0, 254]; elements are v * 2^-X rounded to the
// nearest grid value, ties to even, saturating at 6 (E2M1) or 448 (E4M3).
//
// Grouped GEMM on v_mfma_scale_f32_32x32x64_f8f6f4 (A FP8, B FP4).  Lane
// layout of one instruction (checked with an in-bounds probe): B lane (n, h)
// holds the 32 FP4 values k = 32h .. 32h+31 of one 64-k step (16 bytes, low
// nibble first) and multiplies them by its own scale byte; A lane (m, h) pairs
// its bytes 0..15 with B lanes h = 0 and bytes 16..31 with B lanes h = 1, so A
// lane (m, h) holds the activation bytes [16h, 16h+16) and [32+16h, 32+16h+16)
// of the step, under one scale for all 64 k.
//
// Layouts, k-block-major so that one 64-k step of a tile is one contiguous
// run (1 KB per wave load instruction, whole cache lines; row-major codes
// would give 64-byte activation and 32-byte weight pieces per row):
// activations codes [K/64][row_stride][64] bytes, scales [K/64][row_stride];
// weights codes [G][K/64][N][32] bytes (two E2M1 per byte, low nibble = even
// k), scales [G][K/32][N].  The scales travel through the same global->LDS
// ring as the codes (one uniform load instruction per wave per stage).
#include "gemm_common.hpp"

namespace moe {

typedef int v8i32_t __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- element codes
// 2^k as a float, -126 <= k <= 127 (multiplying by it rounds like ldexpf).
__device__ __forceinline__ float pow2f(int k) { return __uint_as_float(uint32_t(127 + k) << 23); }
// v * 2^k for -127 <= k <= 127 (the one exponent below the normal range by ldexpf)
__device__ __forceinline__ float scale_pow2(float v, int k) {
  return k >= -126 ? v * pow2f(k) : ldexpf(v, k);
}

// Nearest value of a sign-magnitude grid (mbits mantissa bits, smallest normal
// exponent emin, subnormals below), ties to even, saturating at maxmag.
__device__ __forceinline__ uint32_t grid_code(float v, int mbits, int emin, float maxmag, int bias,
                                              int sign_bit) {
  const uint32_t sgn = (__float_as_uint(v) >> 31) << sign_bit;
  const float a = fminf(fabsf(v), maxmag);
  // binade of a from its exponent field (zero and fp32 subnormals fall below
  // emin and are clamped to it, as every value under 2^emin is)
  int e = int((__float_as_uint(a) >> 23) & 0xffu) - 127;
  e = e < emin ? emin : e;
  const float q = rintf(a * pow2f(mbits - e));   // exact scaling by a power of two
  const float half = float(1 << mbits), lim = float(2 << mbits);
  uint32_t code;
  if (a >= ldexpf(1.0f, emin)) {
    code = q >= lim ? uint32_t(e + 1 + bias) << mbits
                    : (uint32_t(e + bias) << mbits) | uint32_t(q - half);
  } else {
    code = q >= half ? (1u << mbits) : uint32_t(q);
  }
  return code | sgn;
}
__device__ __forceinline__ uint32_t e2m1_code(float v) { return grid_code(v, 1, 0, 6.0f, 1, 3); }
// Four E4M3 codes (byte i from v_i) of values already scaled into their block's
// range: the sign bit of v_i over the code of min(|v_i|, 448), which the
// hardware conversion produces (round to nearest even, subnormals below 2^-6);
// it equals the grid rule above, grid_code(v, 3, -6, 448, 7, 7), on every
// non-negative fp32 up to 448 (checked exhaustively on the device).  A NaN
// saturates to 448 with its sign, as in the grid rule.
__device__ __forceinline__ uint32_t e4m3_pack4(float v0, float v1, float v2, float v3) {
  uint32_t w = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(fminf(fabsf(v0), 448.0f),
                                                        fminf(fabsf(v1), 448.0f), 0, false));
  w = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(fminf(fabsf(v2), 448.0f), fminf(fabsf(v3), 448.0f),
                                               int(w), true));
  const uint32_t sg = ((__float_as_uint(v0) >> 31) << 7) | ((__float_as_uint(v1) >> 31) << 15) |
                      ((__float_as_uint(v2) >> 31) << 23) | (__float_as_uint(v3) & 0x80000000u);
  return w | sg;
}

// E8M0 scale code of a block with largest magnitude amax (emax of the element type).
__device__ __forceinline__ int scale_code(float amax, int emax) {
  if (!(amax > 0.0f)) return 0;
  const int c = ilogbf(amax) - emax + 127;
  return c < 0 ? 0 : (c > 254 ? 254 : c);
}

// Eight consecutive elements (one 16-byte bf16 load or two fp32 loads).
__device__ __forceinline__ void load8(const void* p, int64_t i, bool bf16, float* v) {
  if (bf16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  } else {
    const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Each thread quantises eight consecutive elements of a row; the LANES threads
// of one block (32 / 8 = 4 for FP4, 64 / 8 = 8 for FP8) are adjacent lanes and
// combine their maxima with butterfly shuffles.  Loads and code stores are then
// contiguous across the wave.  Blocks never straddle rows (K is a multiple of
// the block size), so the threads of a block are all in range or all out.
template <int LANES>
__device__ __forceinline__ float block_amax(const float* v, bool live) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = live ? m : 0.0f;
#pragma unroll
  for (int o = 1; o < LANES; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  return m;
}

// w [rows, K] (rows = G*N, row r = (g, n)) -> codes [G][K/64][N][32] (low
// nibble first), scales [G][K/32][N].
__global__ __launch_bounds__(256) void mx4_quantize_kernel(const void* __restrict__ w, bool bf16,
                                                           int64_t rows, int K, int N,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  const int per_row = K / 8;
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool live = t < rows * per_row;
  const int64_t r = live ? t / per_row : 0;
  const int c8 = live ? int(t - r * per_row) : 0;
  float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (live) load8(w, r * K + int64_t(c8) * 8, bf16, v);
  const int sc = scale_code(block_amax<4>(v, live), 2);
  if (!live) return;
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) packed |= e2m1_code(scale_pow2(v[i], 127 - sc)) << (4 * i);
  const int64_t g = r / N, n = r - g * N;
  *reinterpret_cast<uint32_t*>(codes + ((g * (K / 64) + c8 / 8) * N + n) * 32 + (c8 % 8) * 4) = packed;
  if ((c8 & 3) == 0) scales[(g * (K / 32) + c8 / 4) * N + n] = uint8_t(sc);
}

// x [rows, K] -> codes [K/64][stride][64], scales[kb * stride + r].
__global__ __launch_bounds__(256) void mx8_quantize_kernel(const void* __restrict__ x, bool bf16,
                                                           int64_t rows, int K, int64_t stride,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  // One wave per (8 rows, one 64-element k-block): lane = 8 * (row in the
  // group) + (8-element slice), so a wave reads 128 contiguous bytes of each
  // of its rows and writes 512 contiguous bytes of codes (8 rows of the block).
  const int KB = K / 64;
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t wv = t >> 6;
  const int lane = int(t & 63);
  const int64_t r = (wv / KB) * 8 + (lane >> 3);
  const int kb = int(wv % KB), q = lane & 7;
  const bool live = r < rows;
  float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (live) load8(x, r * K + int64_t(kb) * 64 + q * 8, bf16, v);
  const int sc = scale_code(block_amax<8>(v, live), 8);
  if (!live) return;
  const int k = 127 - sc;
  const uint32_t p[2] = {e4m3_pack4(scale_pow2(v[0], k), scale_pow2(v[1], k), scale_pow2(v[2], k), scale_pow2(v[3], k)),
                         e4m3_pack4(scale_pow2(v[4], k), scale_pow2(v[5], k), scale_pow2(v[6], k), scale_pow2(v[7], k))};
  *reinterpret_cast<uint2*>(codes + (int64_t(kb) * stride + r) * 64 + q * 8) = make_uint2(p[0], p[1]);
  if (q == 0) scales[int64_t(kb) * stride + r] = uint8_t(sc);
}

// ---------------------------------------------------------------- grouped GEMM
constexpr int MX_BN = 256;       // tile columns: 4 waves along n, 64 columns each
constexpr int MX_NS = 6;         // ring slots, one 64-k stage each

template <int N>
__device__ __forceinline__ void mx_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void mx_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Chunk swizzles (16-byte chunks): A rows of 64 bytes (4 chunks), B rows of 32
// bytes (2 chunks); conflict-free for 8- and 16-lane LDS passes.
__device__ __forceinline__ int swz_a(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }
__device__ __forceinline__ int swz_b(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }

struct MxArgs {
  const uint8_t* A;        // [K/64][a_stride][64] FP8 codes
  const uint8_t* As;       // [K/64, a_stride] scales
  int64_t a_stride;
  const uint8_t* B;        // [G][K/64][nb_rows][32] FP4 codes
  const uint8_t* Bs;       // [G, K/32, nb_rows] scales
  int nb_rows;             // rows of each group's B (n_up for the up projection, d for down)
  const int32_t* offsets;
  int G;
  int64_t max_rows;
  int N, K, up_off, epi;
  float* out;              // STORE: [rows, N] fp32
  uint8_t* aq;             // act epilogues: [N/64][aq_stride][64] FP8 codes
  uint8_t* aqs;            // [N/64, aq_stride] scales
  int64_t aq_stride;
};

// 512 threads = 8 waves (2 along m x 4 along n), tile BM x 256, each wave
// (BM/2) x 64 as (BM/64) x 2 blocks of 32x32.  NP = 2: gate and up panels.
template <int BM, int NP, int EPI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gg_mx_kernel(MxArgs g) {
  constexpr int BN = MX_BN, WV = 8;
  constexpr int MI = BM / 64, NI = 2;
  constexpr int A_BYTES = BM * 64, B_BYTES = NP * BN * 32;
  // scale region: A scales as 128 dwords from a 4-byte-aligned start (up to
  // BM + 3 bytes used), B scales NP * 2 runs of 256 bytes; an LDS-DMA load of
  // 4 bytes puts lane l's dword at +4l
  constexpr int AS_BYTES = 512, BS_BYTES = NP * 2 * BN;
  constexpr int PAD_BYTES = 256;            // target of the padding scale loads
  constexpr int STAGE = A_BYTES + B_BYTES + AS_BYTES + BS_BYTES + PAD_BYTES;
  constexpr int A_INS = A_BYTES / 1024 / WV, B_INS = B_BYTES / 1024 / WV;
  static_assert(A_INS >= 1 && B_INS >= 1, "tile too small");
  static_assert(BM + 3 <= AS_BYTES, "A scale run");
  constexpr int INS = A_INS + B_INS + 1;     // + one scale load per wave
  extern __shared__ uint4 lds_u4[];
  char* lds = reinterpret_cast<char*>(lds_u4);
  __shared__ int32_t ts[257];

  // tile plan: ts[g] = tiles before group g (ceil(M_g / BM) * N / BN each)
  {
    const int tid = threadIdx.x;
    const bool scan = tid < 256;
    const int NTt = g.N / BN;
    if (scan) ts[tid + 1] = tid < g.G ? int32_t(cdiv(g.offsets[tid + 1] - g.offsets[tid], BM)) * NTt : 0;
    if (tid == 0) ts[0] = 0;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int32_t v = scan && tid >= o ? ts[tid + 1 - o] : 0;
      __syncthreads();
      if (scan) ts[tid + 1] += v;
      __syncthreads();
    }
  }
  const int32_t total = ts[g.G];
  const int per = (total + 7) >> 3;
  const int bid = blockIdx.x;
  const int tile = (bid & 7) * per + (bid >> 3);
  if ((bid >> 3) >= per || tile >= total) return;
  TileCoord tc;
  locate_tile(ts, g.offsets, g.G, tile, BM, BN, tc);
  const int K = g.K, KS = K / 64;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wm = w >> 2, wn = w & 3;

  // ---- load sources (instruction q = w + 8i of each region): per-lane byte
  // offsets within each stage's buffer descriptors (rebased per 64-k stage)
  uint32_t a_off[A_INS];
#pragma unroll
  for (int i = 0; i < A_INS; ++i) {
    const int row = 16 * (w + WV * i) + (l >> 2);
    const int c = (l & 3) ^ swz_a(row);
    const int mr = min(tc.m0 + row, tc.M - 1);
    a_off[i] = uint32_t((int64_t(tc.row0) + mr) * 64 + 16 * c);
  }
  uint32_t b_off[B_INS];
  const uint8_t* Bg = g.B + int64_t(tc.grp) * g.nb_rows * (K / 2);
#pragma unroll
  for (int i = 0; i < B_INS; ++i) {
    const int row = 32 * (w + WV * i) + (l >> 1);          // 0 .. NP*BN-1
    const int p = row / BN, col = row % BN;
    const int c = (l & 1) ^ swz_b(row);
    b_off[i] = uint32_t((p * g.up_off + tc.n0 + col) * 32 + 16 * c);
  }
  // scale loads (4 bytes per lane): waves 0 and 1 bring the A scales of the
  // tile's rows from the aligned start a4 (a_off = misalignment); the next
  // NP*2 waves bring the B scales (one 256-column run of scale row 2s + h of
  // panel p); the rest issue a load outside an empty descriptor, which
  // writes zeros to the padding and keeps every wave's load count equal.
  const int nA = 2, nB = NP * 2;
  const int64_t a_first = int64_t(tc.row0) + tc.m0;
  const int64_t a4 = a_first & ~int64_t(3);
  const int a_off_s = int(a_first - a4);
  const int64_t a_last = (g.a_stride & ~int64_t(3)) - 4;   // last whole dword of a scale row
  const uint8_t* Bsg = g.Bs + int64_t(tc.grp) * (K / 32) * g.nb_rows;
  const int64_t a_kstep = g.a_stride * 64, b_kstep = int64_t(g.nb_rows) * 32;   // bytes per 64-k block
  const int sj = w - nA;
  const uint32_t s_off = w < nA ? uint32_t(min(a4 + 256 * w + 4 * l, a_last))
                         : w < nA + nB ? uint32_t((sj & 1) * g.nb_rows + (sj >> 1) * g.up_off + tc.n0 + 4 * l)
                                       : 0u;
  auto issue = [&](char* base, int ks) {
    const rsrc_t ra = make_rsrc(g.A + a_kstep * ks, clamp_bytes(a_kstep));
#pragma unroll
    for (int i = 0; i < A_INS; ++i) lds_load16(ra, a_off[i], 0, base + (w + WV * i) * 1024);
    const rsrc_t rb = make_rsrc(Bg + b_kstep * ks, clamp_bytes(b_kstep));
#pragma unroll
    for (int i = 0; i < B_INS; ++i) lds_load16(rb, b_off[i], 0, base + A_BYTES + (w + WV * i) * 1024);
    char* sb = base + A_BYTES + B_BYTES;
    if (w < nA)
      lds_load4(make_rsrc(g.As + int64_t(ks) * g.a_stride, clamp_bytes(g.a_stride)), s_off, 0,
                sb + 256 * w);
    else if (w < nA + nB)
      lds_load4(make_rsrc(Bsg + int64_t(2 * ks) * g.nb_rows, clamp_bytes(2 * int64_t(g.nb_rows))),
                s_off, 0, sb + AS_BYTES + 256 * sj);
    else
      lds_load4(make_rsrc(g.As, 0), 0, 0, sb + AS_BYTES + BS_BYTES);
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

  const int fr = l & 31, fh = l >> 5;
  const int krot = KS > 0 ? tile % KS : 0;
  auto kidx = [&](int j) { const int kn = j + krot; return kn < KS ? kn : kn - KS; };
  // Ring of MX_NS = 6 slots (stage s in slot s % 6) walked in steps of two
  // 64-k stages: one wait and one barrier per 128 k, the next two stages
  // issued into the slots the previous step released, four stages in flight.
  // K is a multiple of 256, so KS is even.
  auto compute = [&](const char* base) {
    const char* Ab = base;
    const char* Bb = base + A_BYTES;
    const uint8_t* Sa = reinterpret_cast<const uint8_t*>(base + A_BYTES + B_BYTES);
    const uint8_t* Sb = Sa + AS_BYTES;
    v8i32_t af[MI];
    int sa[MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = wm * (BM / 2) + mi * 32 + fr;
      const int z = swz_a(row);
      const uint4 lo = *reinterpret_cast<const uint4*>(Ab + row * 64 + 16 * (fh ^ z));
      const uint4 hi = *reinterpret_cast<const uint4*>(Ab + row * 64 + 16 * ((2 + fh) ^ z));
      af[mi] = v8i32_t{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      sa[mi] = Sa[a_off_s + row];
    }
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int col = wn * 64 + ni * 32 + fr;
        const int row = p * BN + col;
        const uint4 bv = *reinterpret_cast<const uint4*>(Bb + row * 32 + 16 * (fh ^ swz_b(row)));
        const v8i32_t bf = v8i32_t{int(bv.x), int(bv.y), int(bv.z), int(bv.w), 0, 0, 0, 0};
        const int sb = Sb[(2 * p + fh) * 256 + col];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          acc[p][mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[mi], bf, acc[p][mi][ni], 0, 4, 0, sa[mi], 0, sb);
      }
  };
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (j < KS) issue(lds + j * STAGE, kidx(j));
  for (int kt = 0; kt < KS; kt += 2) {
    // stages kt, kt+1 have landed once at most the loads of the stages issued
    // after them are outstanding (loads complete in order)
    if (min(KS, kt + 4) - (kt + 2) >= 2) mx_wait_vmcnt<2 * INS>();
    else mx_wait_vmcnt<0>();
    mx_barrier();
    // The slots written and the slots read never overlap; passing them as
    // restrict parameters of one inlined call lets the compiler read this
    // step's fragments without waiting for the loads just issued.
    auto step = [&](char* __restrict__ w0, char* __restrict__ w1, const char* __restrict__ r0,
                    const char* __restrict__ r1) {
      if (kt + 4 < KS) issue(w0, kidx(kt + 4));
      if (kt + 5 < KS) issue(w1, kidx(kt + 5));
      compute(r0);
      compute(r1);
    };
    step(lds + ((kt + 4) % MX_NS) * STAGE, lds + ((kt + 5) % MX_NS) * STAGE,
         lds + (kt % MX_NS) * STAGE, lds + ((kt + 1) % MX_NS) * STAGE);
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();

  // ---- epilogue through LDS: per 32-row block mi, each wave writes its
  // [NP][32][64 + 4] fp32 region, then 16 lanes per row read 4 columns each.
  constexpr int CST = 64 + 4;
  float* cw = reinterpret_cast<float*>(lds) + w * (NP * 32 * CST);
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          cw[(p * 32 + 8 * (r >> 2) + 4 * fh + (r & 3)) * CST + ni * 32 + fr] = acc[p][mi][ni][r];
    __syncthreads();
    const int c4 = (l & 15) * 4;
    const int n = tc.n0 + wn * 64 + c4;
#pragma unroll 2
    for (int it = 0; it < 8; ++it) {
      const int rl = it * 4 + (l >> 4);
      const int mr = tc.m0 + wm * (BM / 2) + mi * 32 + rl;
      const bool ok = mr < tc.M;
      const int64_t row = int64_t(tc.row0) + mr;
      const float4 v0 = *reinterpret_cast<const float4*>(cw + rl * CST + c4);
      if constexpr (EPI == EPI_STORE_F32) {
        if (ok) *reinterpret_cast<float4*>(g.out + row * g.N + n) = v0;
      } else {
        float a[4];
        if constexpr (EPI == EPI_SWIGLU) {
          const float4 v1 = *reinterpret_cast<const float4*>(cw + (32 + rl) * CST + c4);
          a[0] = silu_fast(v0.x) * v1.x; a[1] = silu_fast(v0.y) * v1.y;
          a[2] = silu_fast(v0.z) * v1.z; a[3] = silu_fast(v0.w) * v1.w;
        } else {
          a[0] = gelu_fast(v0.x); a[1] = gelu_fast(v0.y); a[2] = gelu_fast(v0.z); a[3] = gelu_fast(v0.w);
        }
        // FP8 quantisation of the 64-column block held by these 16 lanes
        float amax = fmaxf(fmaxf(fabsf(a[0]), fabsf(a[1])), fmaxf(fabsf(a[2]), fabsf(a[3])));
        amax = group_max<16>(amax);
        const int sc = scale_code(amax, 8);
        const int k = 127 - sc;
        const uint32_t pk = e4m3_pack4(scale_pow2(a[0], k), scale_pow2(a[1], k), scale_pow2(a[2], k),
                                       scale_pow2(a[3], k));
        if (ok) {
          *reinterpret_cast<uint32_t*>(g.aq + (int64_t(n / 64) * g.aq_stride + row) * 64 + (n % 64)) = pk;
          if ((l & 15) == 0) g.aqs[int64_t(n / 64) * g.aq_stride + row] = uint8_t(sc);
        }
      }
    }
    __syncthreads();
  }
}

template <int BM, int NP, int EPI>
void launch_mx_cfg(const MxArgs& g, hipStream_t st) {
  const int64_t bound = (cdiv(g.max_rows, BM) + g.G) * (g.N / MX_BN);
  const unsigned grid = unsigned(cdiv(bound, 8) * 8);
  constexpr size_t stage = size_t(BM) * 64 + size_t(NP) * MX_BN * 32 + 512 + size_t(NP) * 2 * MX_BN + 256;
  constexpr size_t epi = size_t(8) * NP * 32 * (64 + 4) * 4;   // the fp32 epilogue staging
  constexpr size_t lds_bytes = MX_NS * stage > epi ? MX_NS * stage : epi;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gg_mx_kernel<BM, NP, EPI>),
      hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_bytes));
  (void)attr;
  gg_mx_kernel<BM, NP, EPI><<<dim3(grid), dim3(512), lds_bytes, st>>>(g);
}

hipError_t launch_mx_quantize_weights(const void* w, bool bf16, int64_t rows, int K, int N,
                                      uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const int64_t nt = rows * (K / 8);
  if (nt == 0) return hipSuccess;
  mx4_quantize_kernel<<<unsigned(cdiv(nt, 256)), 256, 0, st>>>(w, bf16, rows, K, N, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_quantize_act(const void* x, bool bf16, int64_t rows, int K, int64_t stride,
                                  uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const int64_t nt = cdiv(rows, 8) * (K / 64) * 64;   // one wave per 8 rows x 64 k
  if (nt == 0) return hipSuccess;
  mx8_quantize_kernel<<<unsigned(cdiv(nt, 256)), 256, 0, st>>>(x, bf16, rows, K, stride, codes,
                                                               scales);
  return hipGetLastError();
}

// Up projection with the activation and FP8 quantisation fused, then the down
// projection to fp32.  xq/xs: the rows' FP8 codes and scales; aq/aqs: buffers
// for the quantised activation [max_rows, F], [F/64, a_stride].
hipError_t launch_mx_ffn(const uint8_t* xq, const uint8_t* xs, int64_t x_stride,
                         const int32_t* offsets, int G, int64_t max_rows, int d, int F, int act,
                         const uint8_t* W13q, const uint8_t* W13s, const uint8_t* W2q,
                         const uint8_t* W2s, uint8_t* aq, uint8_t* aqs, int64_t a_stride,
                         float* out, hipStream_t st) {
  if (G == 0 || max_rows == 0) return hipSuccess;
  const bool swiglu = act == 0;
  MxArgs u{};
  u.A = xq; u.As = xs; u.a_stride = x_stride;
  u.B = W13q; u.Bs = W13s; u.nb_rows = swiglu ? 2 * F : F;
  u.offsets = offsets; u.G = G; u.max_rows = max_rows;
  u.N = F; u.K = d; u.up_off = swiglu ? F : 0;
  u.aq = aq; u.aqs = aqs; u.aq_stride = a_stride;
  const bool bm256 = max_rows / G >= 192;
  if (swiglu) {
    u.epi = EPI_SWIGLU;
    launch_mx_cfg<128, 2, EPI_SWIGLU>(u, st);
  } else {
    u.epi = EPI_GELU;
    if (bm256) launch_mx_cfg<256, 1, EPI_GELU>(u, st); else launch_mx_cfg<128, 1, EPI_GELU>(u, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MxArgs dn{};
  dn.A = aq; dn.As = aqs; dn.a_stride = a_stride;
  dn.B = W2q; dn.Bs = W2s; dn.nb_rows = d;
  dn.offsets = offsets; dn.G = G; dn.max_rows = max_rows;
  dn.N = d; dn.K = F; dn.up_off = 0; dn.epi = EPI_STORE_F32; dn.out = out;
  // the down projection keeps 256-row tiles only while they give two tiles per
  // CU: with fewer, 128-row tiles stream the long K better (32 experts x 245
  // rows, d = 1024, F = 4096: 50 vs 69 us)
  const bool dn256 = bm256 && cdiv(max_rows, 256) * (d / MX_BN) >= 512;
  if (dn256) launch_mx_cfg<256, 1, EPI_STORE_F32>(dn, st); else launch_mx_cfg<128, 1, EPI_STORE_F32>(dn, st);
  return hipGetLastError();
}

}  // namespace moe
