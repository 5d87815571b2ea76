// Grouped expert GEMM on bf16 MFMA for gfx950 (the expert FFN of the MoE
// layer and its backward: "Mixture of Experts Explained", "Making MoEs go
// brrr" — experts run as grouped, not branchy, computation over
// expert-contiguous rows).
//
// Three operand layouts (GemmArgs::mode), fp32 accumulation:
//  * GM_NT (forward): out[rows of g] = epi(A[rows] . B[g]^T), A [rows, K] and
//    B [g][n, K] both K-contiguous (B in the [out, in] weight layout).
//  * GM_NN (data gradients): out[rows of g] = epi(A[rows] . B[g]), B [g][K, n]:
//    the same weights read as stored, K-major.
//  * GM_KGROUP (weight gradients): out[g] = A_g^T . B_g, reduced over the M_g
//    rows of group g; A [rows, M_fixed] and B [rows, N] are the saved
//    activations as stored (K-major), out [g][M_fixed, N] fp32.
//
// Design for CDNA4:
//  * 512 threads = 8 waves in a 2x4 grid (two waves per SIMD); each wave owns
//    a (BM/2) x (BN/4) sub-tile of every panel as (BM/64) x (BN/128) blocks of
//    v_mfma_f32_32x32x16_bf16.  With BM = BN = 256 a wave issues 8 MFMAs per
//    6 operand fragments.
//  * Global -> LDS with buffer_load_dwordx4 ... lds (no staging registers):
//    each wave instruction fills 1 KB of LDS from a raw buffer descriptor and
//    a 32-bit per-lane offset.  A ring of K stages of 64 (as many as fit
//    144 KB, at most 4): the next stages' loads, issued as one burst after
//    each stage's barrier, are in flight while a stage multiplies.
//  * A stage's loads and its fragment reads sit in one inlined call whose
//    write and read slots are restrict pointers: the compiler then knows the
//    LDS-DMA writes cannot alias the fragment reads and does not wait for the
//    loads before reading fragments.
//  * A K-contiguous operand is staged as rows of 64 k (128 B) whose eight
//    16-byte chunks are XOR-swizzled by (row & 7) ^ ((row >> 3) & 1); an MFMA
//    fragment is one 16-byte LDS read per lane, conflict-free whether the LDS
//    serves 8 or 16 lanes per pass.
//  * A K-major operand is staged as 64 rows of k, each holding the tile's X
//    columns (2*X bytes).  The 32-byte segments of row r are XOR-swizzled by
//    kswz(r) = (r & 3) ^ ((r & 3) << 1) (0, 3, 6, 5); a fragment is two LDS
//    transpose reads (ds_read_b64_tr_b16) per lane, which hand each lane four
//    consecutive k of one column.  Each 16-lane read touches four rows at four
//    distinct 32-byte bank groups, and the two 16-lane groups of a 32-lane
//    pass at eight: no bank conflicts with 128- or 256-byte passes.
//  * The tile plan (per-group prefix of tile counts) is computed by every
//    workgroup from the device-resident row offsets: no planner launch and no
//    host synchronisation.  Rows past a group's end are clamped to its last
//    row on load and never stored; K rows past a group's end (weight
//    gradients) read as zeros (beyond the buffer descriptor's size).
//  * Workgroups are dealt round-robin to the 8 XCDs; block b takes logical
//    tile (b % 8) * ceil(tiles / 8) + b / 8, so each XCD works through a
//    contiguous run of tiles (same expert, consecutive n-tiles, m-tiles
//    fastest) and its L2 holds the shared A rows and weight panels.
//  * Long reductions with an fp32 store: when the tiles leave a last round
//    that fills at most half of the compute units, those tiles are cut into
//    K segments run by extra workgroups after the whole tiles, and a second
//    kernel adds their partial sums in segment order.
//  * NP = 2 (SwiGLU forward): the gate rows n0.. and up rows up_off+n0.. of
//    W13 are two B panels multiplied against one A tile; the epilogue forms
//    silu(gate) * up directly.
//  * The epilogue stages the accumulators through LDS (row-contiguous 16-lane
//    stores), applies GELU / SwiGLU or their backward with hardware 2^x and
//    reciprocal and the bf16 conversion instruction, and writes bf16 or fp32
//    with non-temporal stores.
#include <atomic>

#include "gemm_common.hpp"

namespace moe {

constexpr int GB_BK = 64;
constexpr int GB_WAVES = 8;   // waves per workgroup (one workgroup per CU)

// Epilogue outputs written with non-temporal stores (streamed to memory
// without being kept in the caches), one bit per output kind.  Every output of
// these GEMMs is either read back much later (h, the weight gradients) or
// streamed once by the next kernel; streaming them all measured fastest (32
// experts x 256 rows, d = 1024, F = 4096: weight gradient 175 -> 155 us, down
// projection 90 -> 80 us, random operands).
enum : int {
  GB_NT_WGRAD = 1,    // fp32 weight gradients (K-grouped mode)
  GB_NT_HSAVE = 2,    // saved pre-activations h (read back only in the backward)
  GB_NT_FWD_F32 = 4,  // fp32 forward outputs (the expert outputs o)
  GB_NT_FWD_ACT = 8,  // bf16 activations a (the down projection's input)
  GB_NT_DGRAD = 16,   // data-gradient outputs
};
constexpr int GB_NT = GB_NT_WGRAD | GB_NT_HSAVE | GB_NT_FWD_F32 | GB_NT_FWD_ACT | GB_NT_DGRAD;

typedef unsigned uintx2 __attribute__((ext_vector_type(2)));
template <bool NT>
__device__ __forceinline__ void st_f4(float* p, float4 v) {
  if constexpr (NT) __builtin_nontemporal_store(floatx4{v.x, v.y, v.z, v.w}, reinterpret_cast<floatx4*>(p));
  else *reinterpret_cast<float4*>(p) = v;
}
template <bool NT>
__device__ __forceinline__ void st_u2(uint16_t* p, uint2 v) {
  if constexpr (NT) __builtin_nontemporal_store(uintx2{v.x, v.y}, reinterpret_cast<uintx2*>(p));
  else *reinterpret_cast<uint2*>(p) = v;
}

// Four activations of one row as bf16: hi = bf16(a) in rows of out_ld (or N)
// elements, and with lo_off the remainders lo = bf16(a - hi) at lo_off + n
// (a - hi is exact in fp32; hi + lo carries a to about 16 significant bits).
template <bool NT>
__device__ __forceinline__ void store_act(const GemmArgs& g, int64_t row, int n, float4 a) {
  const uint32_t h01 = pack_bf2(a.x, a.y), h23 = pack_bf2(a.z, a.w);
  uint16_t* orow = static_cast<uint16_t*>(g.out) + row * (g.out_ld ? g.out_ld : g.N);
  st_u2<NT>(orow + n, make_uint2(h01, h23));
  if (g.lo_off) {
    const float l0 = a.x - __uint_as_float(h01 << 16), l1 = a.y - __uint_as_float(h01 & 0xffff0000u);
    const float l2 = a.z - __uint_as_float(h23 << 16), l3 = a.w - __uint_as_float(h23 & 0xffff0000u);
    st_u2<NT>(orow + g.lo_off + n, make_uint2(pack_bf2(l0, l1), pack_bf2(l2, l3)));
  }
}

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// LDS transpose read of 16-bit data: within each 16-lane group, lane b+i
// receives element i%4 of the four values addressed by lane b+4q+i/4, for
// q = 0..3.  When lane b+4q+t points at row r0+q, columns c0+4t.. of a [k][x]
// tile, lane b+i receives column c0+i of rows r0..r0+3.
__device__ __forceinline__ bf16x8 lds_read_tr_pair(const char* p0, const char* p1) {
  const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p0));
  const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Ring depth: as many 64-deep K stages as fit in 144 KB of LDS, at most 4.
__host__ __device__ constexpr int gb_stages(int BM, int BN, int NP) {
  return (BM + NP * BN) * 128 <= 32768 ? 4 : ((BM + NP * BN) * 128 <= 49152 ? 3 : 2);
}

// Segment swizzle of K-major rows: distinct in the low two bits and in bits
// 1..2 over any four consecutive rows.
__device__ __forceinline__ int kswz(int r) { return (r & 3) ^ ((r & 3) << 1); }

// K-major staging: lane l of load instruction q fills row q*(512/X) + l/(X/8)
// (a k row of X columns, 2*X bytes), physical 16-byte chunk p = l % (X/8),
// which holds logical chunk 2*((p >> 1) ^ kswz(row)) + (p & 1).
template <int X>
__device__ __forceinline__ void kmajor_slot(int q, int l, int& row, int& col) {
  row = q * (512 / X) + l / (X / 8);
  const int p = l % (X / 8);
  col = 8 * (2 * ((p >> 1) ^ kswz(row)) + (p & 1));
}

// Row-grouped modes: ts[g] = tiles of the groups before g (ceil(M_g/BM) * N/BN
// each), an inclusive scan by the first 256 threads (G <= 256).  Returns the
// number of tiles.
template <int BM, int BN>
__device__ __forceinline__ int32_t plan_tiles(const GemmArgs& g, int32_t* ts) {
  const int tid = threadIdx.x;
  const bool scan = tid < 256;
  const int NT = g.N / BN;
  if (scan) ts[tid + 1] = tid < g.G ? int32_t(cdiv(g.offsets[tid + 1] - g.offsets[tid], BM)) * NT : 0;
  if (tid == 0) ts[0] = 0;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int32_t v = scan && tid >= o ? ts[tid + 1 - o] : 0;
    __syncthreads();
    if (scan) ts[tid + 1] += v;
    __syncthreads();
  }
  return ts[g.G];
}

template <int BM, int BN, int NP, int EPI, int MODE, int WV>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(WV / 4, WV / 4)))
void gg_bf16_kernel(GemmArgs g) {
  constexpr bool AK = MODE == GM_KGROUP;    // A staged K-major
  constexpr bool BKM = MODE != GM_NT;       // B staged K-major
  static_assert(NP == 1 || MODE == GM_NT, "two B panels only in the forward layout");
  static_assert(BM >= 128 && BN >= 128, "K-major staging needs at least 8 segments per row");
  static_assert(WV == 4 || WV == 8, "4 or 8 waves");
  constexpr int NWN = WV / 2;            // waves along n (2 along m)
  constexpr int WTN = BN / NWN;          // wave tile width
  constexpr int ROWS = BM + NP * BN;     // 128-byte LDS rows per stage
  constexpr int STAGE = ROWS * 8;        // uint4 per stage
  constexpr int MI = BM / 64, NI = WTN / 32;
  constexpr int A_INS = BM / (8 * WV), B_INS = BN / (8 * WV);  // load instructions per wave per panel
  static_assert(NI >= 1 && A_INS >= 1 && B_INS >= 1, "tile too small for the wave count");
  constexpr int NS = gb_stages(BM, BN, NP);
  constexpr int INS = A_INS + NP * B_INS;   // load instructions per wave per stage
  // NS stages of (BM + NP*BN) x 128 bytes (at most 144 KB), dynamic LDS.
  extern __shared__ uint4 lds[];
  __shared__ int32_t ts[257];

  int32_t total;
  int tile;
  // K segments of a split tile: this block's segment (-1: a whole tile), the
  // segment count, and the number of whole tiles (split tiles follow them).
  int seg = -1, nseg = 1, whole = 0;
  if constexpr (MODE == GM_KGROUP) {
    // A tile's work grows with its group's rows, so groups are taken heaviest
    // first (ts[r] = the group of rank r by rows, descending, ties to the
    // lower index; G <= 256) and tiles go round-robin over the XCDs in that
    // order: the longest tiles start first and spread over the whole chip.
    const int tid = threadIdx.x;
    const int32_t mine = tid < g.G ? g.offsets[tid + 1] - g.offsets[tid] : -1;
    if (tid < 256) ts[tid] = mine;
    __syncthreads();
    int rank = 0;
    if (tid < g.G)
      for (int h = 0; h < g.G; ++h) {
        const int32_t o = ts[h];
        rank += (o > mine) || (o == mine && h < tid);
      }
    __syncthreads();
    if (tid < g.G) ts[rank] = tid;
    __syncthreads();
    total = g.G * (g.M_fixed / BM) * (g.N / BN);
    tile = blockIdx.x;
    if (tile >= total) return;
  } else {
    total = plan_tiles<BM, BN>(g, ts);
    whole = total;
    if (EPI == EPI_STORE_F32 && g.sk_part) {
      // A last round of at most half the concurrent workgroups would leave
      // most compute units idle while it runs: its tiles are split along K
      // into S segments (S * tiles <= sk_cus), all of which run at once.
      const int tail = total % g.sk_cus;
      if (tail > 0 && 2 * tail <= g.sk_cus) {
        nseg = min(4, g.sk_cus / tail);
        whole = total - tail;
      }
      // (every thread of block 0 stores the same two values: no branch on
      // the thread index, so the tile's values stay wave-uniform)
      if (blockIdx.x == 0) {
        g.sk_tab[0] = total - whole;
        g.sk_tab[1] = nseg;
      }
    }
    const int bid = blockIdx.x;
    if (!g.sk_part || bid < g.sk_grid0) {
      const int per = (whole + 7) >> 3;
      tile = (bid & 7) * per + (bid >> 3);
      if ((bid >> 3) >= per || tile >= whole) return;
    } else {
      // blocks past sk_grid0: segment sidx % S of split tile sidx / S
      const int sidx = bid - g.sk_grid0;
      if (sidx >= (total - whole) * nseg) return;
      tile = whole + sidx / nseg;
      seg = sidx % nseg;
    }
  }
  // Row stride of a K-major B: [rows, ldb] in the K-grouped mode, [K, N] otherwise.
  const int64_t ldb = (MODE == GM_KGROUP && g.ldb) ? g.ldb : int64_t(g.N);
  // K-contiguous B (forward layout): row stride, the K period when B wraps
  const int64_t ldbk = (MODE == GM_NT && g.b_kwrap) ? int64_t(g.b_kwrap) : int64_t(g.K);
  TileCoord tc;
  int K;                                     // reduction length of this tile
  const uint16_t* A;
  const uint16_t* B;
  if constexpr (MODE == GM_KGROUP) {
    const int MT = g.M_fixed / BM;
    const int tpg = MT * (g.N / BN);
    tc.grp = ts[tile / tpg];
    const int local = tile % tpg;
    tc.m0 = (local % MT) * BM;
    tc.n0 = (local / MT) * BN;
    tc.row0 = 0;                             // output rows of group grp
    tc.M = g.M_fixed;
    const int32_t r0 = g.offsets[tc.grp];
    K = g.offsets[tc.grp + 1] - r0;
    A = static_cast<const uint16_t*>(g.A) + int64_t(r0) * g.M_fixed;
    B = static_cast<const uint16_t*>(g.B) + int64_t(r0) * ldb;
  } else {
    locate_tile(ts, g.offsets, g.G, tile, BM, BN, tc);
    K = g.K;
    if (seg == 0) {
      int32_t* e = g.sk_tab + 2 + 3 * (tile - whole);
      e[0] = tc.row0 + tc.m0;
      e[1] = tc.n0;
      e[2] = min(tc.M - tc.m0, BM);
    }
    A = static_cast<const uint16_t*>(g.A);
    B = static_cast<const uint16_t*>(g.B) + int64_t(tc.grp) * g.b_group_stride;
  }

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wm = w / NWN, wn = w % NWN;

  // ---- load sources.  Instruction i of wave w fills the 1 KB LDS block
  // q = w + WV*i of its panel.  K-contiguous: lane l fills slot l of the
  // 8-row group q: row l/8, physical chunk l%8, which holds logical chunk
  // (l%8) ^ swz(row); the group starts at a row with (row >> 3) & 1 == w & 1.
  const int lrow = l >> 3;
  const int lchunk = (l & 7) ^ lrow ^ (w & 1);
  // Per-lane byte offsets of each load instruction, relative to the tile's
  // (row modes) or the stage's (K-major operands) descriptor base.
  uint32_t a_off[A_INS];
#pragma unroll
  for (int i = 0; i < A_INS; ++i) {
    if constexpr (AK) {
      int row, col;
      kmajor_slot<BM>(w + WV * i, l, row, col);
      a_off[i] = uint32_t((int64_t(row) * g.M_fixed + tc.m0 + col) * 2);
    } else {
      const int mr = min(tc.m0 + 8 * (w + WV * i) + lrow, tc.M - 1) - tc.m0;
      a_off[i] = uint32_t((int64_t(mr) * K + 8 * lchunk) * 2);
    }
  }
  constexpr int NBS = BKM ? B_INS : NP * B_INS;
  uint32_t b_off[NBS];
#pragma unroll
  for (int i = 0; i < NBS; ++i) {
    if constexpr (BKM) {
      int row, col;
      kmajor_slot<BN>(w + WV * i, l, row, col);
      b_off[i] = uint32_t((int64_t(row) * ldb + tc.n0 + col) * 2);
    } else {
      const int p = i / B_INS, ii = i % B_INS;
      b_off[i] = uint32_t((int64_t(p * g.up_off + 8 * (w + WV * ii) + lrow) * ldbk + 8 * lchunk) * 2);
    }
  }
  // Row modes: descriptors fixed per tile (A from the tile's first row, B from
  // the group's weights at the tile's first column), K advanced by the scalar
  // offset.  K-major operands: rebased per stage at row k0, sized to the rows
  // left in the group.
  const uint16_t* a_tile = AK ? A : A + int64_t(tc.row0 + tc.m0) * K;
  const uint16_t* b_tile = BKM ? B : B + int64_t(tc.n0) * ldbk;
  const rsrc_t a_rs = make_rsrc(a_tile, 0xffffffffu);
  const rsrc_t b_rs = make_rsrc(b_tile, 0xffffffffu);

  // Issue a stage's loads.
  auto issue = [&](uint4* base, int k0) {
    if constexpr (AK) {
      const rsrc_t r = make_rsrc(A + int64_t(k0) * g.M_fixed,
                                 clamp_bytes(int64_t(K - k0) * g.M_fixed * 2));
#pragma unroll
      for (int i = 0; i < A_INS; ++i) lds_load16(r, a_off[i], 0, base + (w + WV * i) * 64);
    } else {
#pragma unroll
      for (int i = 0; i < A_INS; ++i)
        lds_load16(a_rs, a_off[i], uint32_t(k0) * 2, base + (w + WV * i) * 64);
    }
    uint4* bbase = base + BM * 8;
    if constexpr (BKM) {
      const int64_t rows_left = MODE == GM_KGROUP ? int64_t(K - k0) : int64_t(0x7fffffff);
      const rsrc_t r = make_rsrc(B + int64_t(k0) * ldb, clamp_bytes(rows_left * ldb * 2));
#pragma unroll
      for (int i = 0; i < B_INS; ++i) lds_load16(r, b_off[i], 0, bbase + (w + WV * i) * 64);
    } else {
      // column of B's stage: k0, or k0 mod the K period when B wraps (K = 2 * period)
      const int kb = (g.b_kwrap && k0 >= g.b_kwrap) ? k0 - g.b_kwrap : k0;
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int i = 0; i < B_INS; ++i)
          lds_load16(b_rs, b_off[p * B_INS + i], uint32_t(kb) * 2,
                     bbase + p * BN * 8 + (w + WV * i) * 64);
    }
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

  // ---- fragment addressing.  K-contiguous: lane l reads row fr = l%32,
  // logical chunk 2s + fg (k = 16s + 8fg ..).  K-major: in 16-lane group gq,
  // lane j reads row 16s + 8(gq >> 1) + 4h + j/4 at column xf + 16(gq & 1) + 4(j%4)
  // for h = 0, 1; the segment (xf/16) ^ (gq & 1) ^ kswz(j/4) holds it.
  const int fr = l & 31, fg = l >> 5;
  const int gq = l >> 4, jq = l & 15;
  const int t32 = 32 * ((gq & 1) ^ kswz(jq >> 2));
  int a_xo[MI], b_xo[NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) a_xo[mi] = (2 * (wm * (BM / 2) + mi * 32)) ^ t32;
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) b_xo[ni] = (2 * (wn * WTN + ni * 32)) ^ t32;
  const int a_lane = (8 * (gq >> 1) + (jq >> 2)) * (2 * BM) + 8 * (jq & 3);
  const int b_lane = (8 * (gq >> 1) + (jq >> 2)) * (2 * BN) + 8 * (jq & 3);

  // K steps [k_lo, k_lo + NK) of this block: all of them, or its segment's.
  const int KT0 = int(cdiv(K, GB_BK));
  const int k_lo = seg >= 0 ? seg * KT0 / nseg : 0;
  const int KT = seg >= 0 ? (seg + 1) * KT0 / nseg - k_lo : KT0;
  // A wave whose half of the tile lies wholly past its group's last row (the
  // last row tile of a group with few rows) skips its fragment reads and
  // MFMAs; it still issues its share of every stage's loads and meets every
  // barrier, and its zero accumulators are never stored.
  const bool live = tc.m0 + wm * (BM / 2) < tc.M;
  // Each tile walks the K stages starting at its own offset (tile mod KT):
  // concurrent tiles read different K columns, which spreads their requests
  // over the L2 channels instead of having every CU hit the same channel with
  // the same power-of-two row stride.  The sum order depends only on the tile.
  const int krot = KT > 0 ? tile % KT : 0;
  auto kcol = [&](int j) {
    const int kn = j + krot;
    return (k_lo + (kn < KT ? kn : kn - KT)) * GB_BK;
  };
  // NS-stage ring: the loads of K steps kt+1 .. kt+NS-2 are in flight while
  // step kt multiplies, and step kt+NS-1 is issued into the slot step kt-1
  // has just released.
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < KT) issue(lds + j * STAGE, kcol(j));
  // Fragments of K-step s+1 are read from LDS while the MFMAs of step s run.
  constexpr int DS_PER_STEP = MI * (AK ? 2 : 1) + NP * NI * (BKM ? 2 : 1);
  bf16x8 af[2][MI], bfr[2][NP][NI];
  int cur = 0, nxt = NS - 1;
  for (int kt = 0; kt < KT; ++kt) {
    // This wave's loads of step kt have landed once no more than the loads of
    // the steps issued after it are outstanding (loads complete in order).
    const int after = min(NS - 2, KT - 1 - kt);
    if (NS >= 4 && after >= 2) wait_vmcnt<(NS >= 4 ? 2 : 0) * INS>();
    else if (NS >= 3 && after >= 1) wait_vmcnt<(NS >= 3 ? 1 : 0) * INS>();
    else wait_vmcnt<0>();
    // Every wave's loads of step kt have landed and every wave has finished
    // reading step kt-1 (its MFMAs were issued before this point).
    lds_barrier();
    const bool more = kt + NS - 1 < KT;
    const int knext = more ? kcol(kt + NS - 1) : 0;
    // One stage: the next stage's loads into slot `wslot` and this stage's
    // fragment reads from slot `rslot`.  The two slots never overlap; passing
    // them as restrict parameters of one inlined call tells the compiler so,
    // and it then no longer waits for the loads just issued before reading
    // fragments (which it did before every transposed LDS read).
    auto stage = [&](uint4* __restrict__ wslot, const uint4* __restrict__ rslot) {
      // The next stage's loads go out as one burst right after the barrier,
      // giving them the whole stage to land (spreading them over the
      // sub-steps measured 2-4% slower once the loads were buffer loads).
      if (more) issue(wslot, knext);
      const uint4* As = rslot;
      const char* Ab = reinterpret_cast<const char*>(As);
      const char* Bb = Ab + BM * 128;
      if (live)
#pragma unroll
      for (int s = 0; s <= 4; ++s) {
        if (s < 4) {
          const int pc = (2 * s + fg) ^ (fr & 7) ^ ((fr >> 3) & 1);
#pragma unroll
          for (int mi = 0; mi < MI; ++mi) {
            if constexpr (AK) {
              const char* p = Ab + a_lane + a_xo[mi] + 16 * s * (2 * BM);
              af[s & 1][mi] = lds_read_tr_pair(p, p + 4 * (2 * BM));
            } else {
              af[s & 1][mi] = __builtin_bit_cast(bf16x8, As[(wm * (BM / 2) + mi * 32 + fr) * 8 + pc]);
            }
          }
#pragma unroll
          for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
              if constexpr (BKM) {
                const char* q = Bb + b_lane + b_xo[ni] + 16 * s * (2 * BN);
                bfr[s & 1][p][ni] = lds_read_tr_pair(q, q + 4 * (2 * BN));
              } else {
                bfr[s & 1][p][ni] = __builtin_bit_cast(
                    bf16x8, As[(BM + p * BN + wn * WTN + ni * 32 + fr) * 8 + pc]);
              }
            }
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
        if (s < 4) __builtin_amdgcn_sched_group_barrier(0x100, DS_PER_STEP, 0);
        if (s > 0) __builtin_amdgcn_sched_group_barrier(0x008, NP * MI * NI, 0);
      }
    };
    stage(lds + nxt * STAGE, lds + cur * STAGE);
    // Every MFMA of this stage is issued before the next wait and barrier.
    __builtin_amdgcn_sched_barrier(0);
    cur = cur + 1 == NS ? 0 : cur + 1;
    nxt = nxt + 1 == NS ? 0 : nxt + 1;
  }
  __syncthreads();

  // Epilogue through LDS (free after the last barrier).  Per 32-row block mi,
  // each wave writes its accumulators (register r of lane l holds row
  // 8*(r/4) + 4*(l/32) + r%4, column l%32 of a 32x32 block) into its own
  // [NP][32][WTN + 4] fp32 region, then reads rows back four columns per lane
  // and stores 16 bytes (fp32) or 8 bytes (bf16) per lane, row-contiguous.
  constexpr bool NT_OUT = (GB_NT & (MODE == GM_KGROUP ? GB_NT_WGRAD
                                   : MODE == GM_NN     ? GB_NT_DGRAD
                                   : EPI == EPI_STORE_F32 ? GB_NT_FWD_F32
                                                          : GB_NT_FWD_ACT)) != 0;
  constexpr bool NT_H = (GB_NT & GB_NT_HSAVE) != 0;
  constexpr int CST = WTN + 4;
  constexpr int LPR = WTN / 4;        // lanes per row
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
    const int n = tc.n0 + wn * WTN + c4;
#pragma unroll 4
    for (int it = 0; it < 32 / RPI; ++it) {
      const int rl = it * RPI + l / LPR;
      const int mr = tc.m0 + wm * (BM / 2) + mi * 32 + rl;
      if (mr < tc.M) {
        const int64_t row = tc.row0 + mr;
        const float4 v0 = *reinterpret_cast<const float4*>(cw + rl * CST + c4);
        if constexpr (EPI == EPI_STORE_F32) {
          if (seg >= 0) {
            // partial sum of a K segment: slot (split tile, segment), [BM][BN]
            float* pp = g.sk_part + (int64_t(tile - whole) * nseg + seg) * (BM * BN);
            *reinterpret_cast<float4*>(pp + (mr - tc.m0) * BN + (n - tc.n0)) = v0;
          } else {
            float* outp = static_cast<float*>(g.out) +
                          (MODE == GM_KGROUP ? int64_t(tc.grp) * g.M_fixed * g.N : 0);
            st_f4<NT_OUT>(outp + row * g.N + n, v0);
          }
        } else if constexpr (EPI == EPI_SWIGLU_BWD) {
          // v0 = dA[row, n..n+3]; h_in row = [gate | up]; out row = [dgate | dup]
          const uint16_t* hr = static_cast<const uint16_t*>(g.h_in) + row * g.n_b;
          const float4 hg = unpack_bf4(*reinterpret_cast<const uint2*>(hr + n));
          const float4 hu = unpack_bf4(*reinterpret_cast<const uint2*>(hr + g.up_off + n));
          uint16_t* orow = static_cast<uint16_t*>(g.out) + row * g.n_b;
          st_u2<NT_OUT>(orow + n,
              make_uint2(pack_bf2(v0.x * hu.x * dsilu_fast(hg.x), v0.y * hu.y * dsilu_fast(hg.y)),
                         pack_bf2(v0.z * hu.z * dsilu_fast(hg.z), v0.w * hu.w * dsilu_fast(hg.w))));
          st_u2<NT_OUT>(orow + g.up_off + n,
              make_uint2(pack_bf2(v0.x * silu_fast(hg.x), v0.y * silu_fast(hg.y)),
                         pack_bf2(v0.z * silu_fast(hg.z), v0.w * silu_fast(hg.w))));
        } else if constexpr (EPI == EPI_GELU_BWD) {
          const float4 h = unpack_bf4(
              *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(g.h_in) + row * g.n_b + n));
          st_u2<NT_OUT>(static_cast<uint16_t*>(g.out) + row * g.n_b + n,
              make_uint2(pack_bf2(v0.x * dgelu_fast(h.x), v0.y * dgelu_fast(h.y)),
                         pack_bf2(v0.z * dgelu_fast(h.z), v0.w * dgelu_fast(h.w))));
        } else if constexpr (EPI == EPI_GELU) {
          if (g.h_save)
            st_u2<NT_H>(static_cast<uint16_t*>(g.h_save) + row * g.n_b + n,
                        make_uint2(pack_bf2(v0.x, v0.y), pack_bf2(v0.z, v0.w)));
          store_act<NT_OUT>(g, row, n, make_float4(gelu_fast(v0.x), gelu_fast(v0.y),
                                                   gelu_fast(v0.z), gelu_fast(v0.w)));
        } else {
          const float4 v1 = *reinterpret_cast<const float4*>(cw + (32 + rl) * CST + c4);
          if (g.h_save) {
            uint16_t* hs = static_cast<uint16_t*>(g.h_save) + row * g.n_b;
            st_u2<NT_H>(hs + n, make_uint2(pack_bf2(v0.x, v0.y), pack_bf2(v0.z, v0.w)));
            st_u2<NT_H>(hs + g.up_off + n, make_uint2(pack_bf2(v1.x, v1.y), pack_bf2(v1.z, v1.w)));
          }
          store_act<NT_OUT>(g, row, n, make_float4(silu_fast(v0.x) * v1.x, silu_fast(v0.y) * v1.y,
                                                   silu_fast(v0.z) * v1.z, silu_fast(v0.w) * v1.w));
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Output rows of the split tiles: the sum of their S segments' partial sums,
// added in segment order (the result depends only on the shape and the
// operands).  Work item i is 16 rows (chunk i % (BM / 16)) of split tile
// i / (BM / 16); the blocks stride over the items, and with no split tile
// they return at once.  The table written by the GEMM gives each split
// tile's first output row, first column and number of rows.
template <int BM, int BN>
__global__ __launch_bounds__(256) void gg_split_sum_kernel(const float* __restrict__ part,
                                                           const int32_t* __restrict__ tab,
                                                           float* __restrict__ out, int N) {
  constexpr int RB = 16, LPR = BN / 4, RPP = 256 / LPR;
  const int items = tab[0] * (BM / RB), S = tab[1];
  const int c4 = (threadIdx.x % LPR) * 4;
  for (int i = blockIdx.x; i < items; i += gridDim.x) {
    const int ti = i / (BM / RB), rb = i % (BM / RB);
    const int* e = tab + 2 + 3 * ti;
    const int64_t row0 = e[0];
    const int n0 = e[1], rows = e[2];
    const float* p0 = part + int64_t(ti) * S * (BM * BN);
#pragma unroll
    for (int it = 0; it < RB / RPP; ++it) {
      const int r = rb * RB + it * RPP + threadIdx.x / LPR;
      if (r < rows) {
        const float* p = p0 + r * BN + c4;
        float4 v = *reinterpret_cast<const float4*>(p);
        for (int s = 1; s < S; ++s) {
          const float4 u = *reinterpret_cast<const float4*>(p + s * (BM * BN));
          v.x += u.x;
          v.y += u.y;
          v.z += u.z;
          v.w += u.w;
        }
        st_f4<(GB_NT & (GB_NT_FWD_F32 | GB_NT_DGRAD)) != 0>(out + (row0 + r) * N + n0 + c4, v);
      }
    }
  }
}

template <int BM, int BN, int NP, int EPI, int MODE, int WV = GB_WAVES>
void launch_cfg(const GemmArgs& g0, hipStream_t st) {
  GemmArgs g = g0;
  const int64_t bound = MODE == GM_KGROUP ? int64_t(g.G) * (g.M_fixed / BM) * (g.N / BN)
                                          : (cdiv(g.max_rows, BM) + g.G) * (g.N / BN);
  unsigned grid = unsigned(cdiv(bound, 8) * 8);
  // Only long reductions are split: the split costs a second launch and the
  // partial sums' traffic (about 10 us), a last round of tiles with K >= 10240
  // several hundred.
  const bool split = MODE != GM_KGROUP && EPI == EPI_STORE_F32 && g.sk_part && g.sk_cus >= 2 &&
                     g.K >= GB_SK_MIN_K;
  if (split) {
    g.sk_grid0 = int(grid);
    grid += unsigned(g.sk_cus);
  } else {
    g.sk_part = nullptr;
  }
  constexpr size_t lds_bytes = size_t(gb_stages(BM, BN, NP)) * (BM + NP * BN) * 128;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gg_bf16_kernel<BM, BN, NP, EPI, MODE, WV>),
      hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_bytes));
  (void)attr;
  gg_bf16_kernel<BM, BN, NP, EPI, MODE, WV><<<dim3(grid), dim3(64 * WV), lds_bytes, st>>>(g);
  if (split)
    gg_split_sum_kernel<BM, BN><<<dim3(unsigned(g.sk_cus)), dim3(256), 0, st>>>(
        g.sk_part, g.sk_tab, static_cast<float*>(g.out), g.N);
}

template <int EPI, int MODE>
static void launch_rows_np1(const GemmArgs& g, bool bm256, bool bn256, hipStream_t st) {
  if (bm256) {
    if (bn256) launch_cfg<256, 256, 1, EPI, MODE>(g, st); else launch_cfg<256, 128, 1, EPI, MODE>(g, st);
  } else {
    if (bn256) launch_cfg<128, 256, 1, EPI, MODE>(g, st); else launch_cfg<128, 128, 1, EPI, MODE>(g, st);
  }
}

// Tile shape (row modes): 256-row tiles when groups average at least 192 rows
// (fewer re-reads of each weight panel), else 128; 256-column tiles when that
// still gives three tiles per four CUs.  Where 256 x 256 would not (and there
// are several groups), the tile keeps its 256 columns and drops to 128 rows:
// the two row halves of an expert share each weight panel through L2, and
// each CU streams twice the weight bytes per stage (32 experts x 245 rows,
// K = 4096, N = 1024: 85 vs 90 us against 256 x 128; the data gradient 116 vs
// 119 us).  K-grouped mode: 256 x 256 when the output dimensions allow it.
int gemm_concurrent_tiles() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    n = n < GB_SK_SLOTS ? n : GB_SK_SLOTS;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_grouped_gemm_bf16(const GemmArgs& g, hipStream_t st) {
  if (g.G == 0) return hipSuccess;
  if (g.mode == GM_KGROUP) {
    if (g.epi != EPI_STORE_F32 || g.M_fixed % 128 || g.N % 128 || (g.ldb && g.ldb < g.N))
      return hipErrorInvalidValue;
    const bool m256 = g.M_fixed % 256 == 0, n256 = g.N % 256 == 0;
    if (m256 && n256) launch_cfg<256, 256, 1, EPI_STORE_F32, GM_KGROUP>(g, st);
    else if (m256) launch_cfg<256, 128, 1, EPI_STORE_F32, GM_KGROUP>(g, st);
    else if (n256) launch_cfg<128, 256, 1, EPI_STORE_F32, GM_KGROUP>(g, st);
    else launch_cfg<128, 128, 1, EPI_STORE_F32, GM_KGROUP>(g, st);
    return hipGetLastError();
  }
  if (g.max_rows == 0) return hipSuccess;
  if (g.N % 128 || g.K % GB_BK) return hipErrorInvalidValue;
  if (g.b_kwrap && (g.mode != GM_NT || g.K != 2 * g.b_kwrap || g.b_kwrap % GB_BK))
    return hipErrorInvalidValue;
  const int64_t avg = g.max_rows / g.G;
  const bool bm256 = avg >= 192;
  const int64_t mt = cdiv(g.max_rows, bm256 ? 256 : 128);
  const bool bn256 = (g.N % 256 == 0) && mt * (g.N / 256) >= 192;
  // grouped single-panel tiles: 128 x 256 rather than 256 x 128
  const bool flip = bm256 && !bn256 && g.N % 256 == 0 && g.G > 1;
  const bool r256 = bm256 && !flip, c256 = bn256 || flip;
  if (g.mode == GM_NN) {
    switch (g.epi) {
      case EPI_STORE_F32: launch_rows_np1<EPI_STORE_F32, GM_NN>(g, r256, c256, st); break;
      case EPI_SWIGLU_BWD: launch_rows_np1<EPI_SWIGLU_BWD, GM_NN>(g, r256, c256, st); break;
      case EPI_GELU_BWD: launch_rows_np1<EPI_GELU_BWD, GM_NN>(g, r256, c256, st); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (g.epi) {
    case EPI_STORE_F32: launch_rows_np1<EPI_STORE_F32, GM_NT>(g, r256, c256, st); break;
    case EPI_GELU: launch_rows_np1<EPI_GELU, GM_NT>(g, r256, c256, st); break;
    case EPI_SWIGLU:
      if (bm256) launch_cfg<256, 128, 2, EPI_SWIGLU, GM_NT>(g, st);
      else launch_cfg<128, 128, 2, EPI_SWIGLU, GM_NT>(g, st);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
