// Router of the sparse MoE layer for gfx950.
//
// z = x . Wg (+ offset) in FP32, scores, selection-only bias, top-k with
// lowest-index tie-breaking, gates, and per-block partial sums for the load
// balance and z losses ("Mixture of Experts Explained", "What is sparsity?"
// gating equations and "Switch Transformers" full-precision router; handbook
// news digest, "confirmed" bullets on sigmoid / sqrt(softplus) scoring).
//
// The logits are an [T, d] x [d, E] contraction.  With bf16 tokens it runs on
// bf16 MFMA: Wg is split on chip, per MFMA step, into three bf16 planes whose
// sum is exactly Wg, so every product x*w is formed exactly and accumulated in
// FP32.  fp32 tokens use a plain FMA loop.
#include <type_traits>

#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace moe {

int route_pad_experts(int E) { return E <= 32 ? 32 : E <= 64 ? 64 : E <= 128 ? 128 : 256; }

// ---------------------------------------------------------------------------
// Fragment layout for the wide kernel (fp32, split into planes on chip): the
// 16-byte pieces out[((eb * (d / 64) + c) * 8 + i) * 64 + l] hold Wg of expert
// e = 32 eb + l % 32 at k = 64 c + 32 (l / 32) + 8 (i / 2) + 4 (i % 2) .. + 3,
// so pieces 2q and 2q + 1 are the eight k that lane l supplies to MFMA step q
// of 64-k chunk c, and a wave's load of one piece index is 1 KB of contiguous
// memory.  A block transposes a 64 (k) x 32 (expert) tile of Wg through LDS.
__global__ __launch_bounds__(256) void wg_frag_kernel(const float* __restrict__ Wg, int d, int E,
                                                      uint4* __restrict__ out) {
  __shared__ float tile[64][33];
  const int c = blockIdx.x, eb = blockIdx.y, tid = threadIdx.x;
  const float* src = Wg + int64_t(c) * 64 * E;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 5) + 8 * i, col = tid & 31, e = 32 * eb + col;
    tile[r][col] = e < E ? src[int64_t(r) * E + e] : 0.0f;
  }
  __syncthreads();
  uint4* o = out + (int64_t(eb) * (d / 64) + c) * 8 * 64;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = tid + 256 * h, l = idx & 63, i = idx >> 6;
    const int col = l & 31, k = 32 * (l >> 5) + 8 * (i >> 1) + 4 * (i & 1);
    o[idx] = make_uint4(__float_as_uint(tile[k][col]), __float_as_uint(tile[k + 1][col]),
                        __float_as_uint(tile[k + 2][col]), __float_as_uint(tile[k + 3][col]));
  }
}

// ---------------------------------------------------------------------------
// Score functions on the hardware exponential.  exp(x) = 2^(x log2 e)
// (v_exp_f32; relative error about 1 ulp plus |x| * 2^-24 from rounding the
// argument).  log(1 + u) for 0 <= u <= 1 from the series
// log(1 + u) = 2 artanh(s) = 2 (s + s^3/3 + s^5/5 + ...), s = u / (2 + u) <= 1/3:
// eight terms leave a truncation error below 3e-9 relative, so the result is
// within a few ulps.  softplus(z) = max(z, 0) + log(1 + exp(-|z|)).
__device__ __forceinline__ float log1p_unit(float u) {
  const float sv = u * __builtin_amdgcn_rcpf(2.0f + u);
  const float s2 = sv * sv;
  float p = 1.0f / 15.0f;
  p = fmaf(p, s2, 1.0f / 13.0f);
  p = fmaf(p, s2, 1.0f / 11.0f);
  p = fmaf(p, s2, 1.0f / 9.0f);
  p = fmaf(p, s2, 1.0f / 7.0f);
  p = fmaf(p, s2, 1.0f / 5.0f);
  p = fmaf(p, s2, 1.0f / 3.0f);
  p = fmaf(p, s2, 1.0f);
  return 2.0f * sv * p;
}
__device__ __forceinline__ float softplus_fast(float z) {
  return fmaxf(z, 0.0f) + log1p_unit(exp_fast(-fabsf(z)));
}

// ---------------------------------------------------------------------------
// Per-token epilogue shared by the logit kernels (NW waves per block).  zs
// holds KS partial logit sums for the block's BT tokens.  Each token is
// handled by a group of LG = 16 lanes (one DPP row, four tokens per wave at
// a time), each owning VPL experts e = lane_in_group + LG * v; all per-token
// reductions stay inside the row.  LDS scratch: red_p [NW * EP], red_c [EP]
// (the block's routed-slot counts, integer LDS atomics: exact in any order),
// red_s [2 * NW], ob [2 * EP] (the experts' logit offsets and selection
// biases, read once per block).
template <int EP, int KS, int NW, int BT = ROUTE_BT>
__device__ __forceinline__ void route_epilogue(const RouteArgs& a, float (*zs)[BT][EP + 1],
                                               int t0, float* red_p, int32_t* red_c,
                                               float* red_s, float* ob) {
  constexpr int LG = EP < 16 ? EP : 16;
  constexpr int TPI = 64 / LG;
  constexpr int VPL = EP / LG;
  constexpr int KMAX = 16;
  constexpr int TOK_PER_WAVE = BT / NW;
  static_assert(TOK_PER_WAVE % TPI == 0, "tokens per wave");
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int gi = l / LG, lg = l % LG;
  const int E = a.E, k = a.k;

  float pacc[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) pacc[v] = 0.0f;
  // ob: the per-expert logit offsets [0, EP) and selection biases [EP, 2 EP)
  for (int e = tid; e < EP; e += NW * 64) {
    red_c[e] = 0;
    ob[e] = (a.offset && e < E) ? a.offset[e] : 0.0f;
    ob[EP + e] = (a.bias && e < E) ? a.bias[e] : 0.0f;
  }
  __syncthreads();
  float lse2 = 0.0f;
  int32_t nf = 0;

  for (int it = 0; it < TOK_PER_WAVE / TPI; ++it) {
    const int tl = w * TOK_PER_WAVE + it * TPI + gi;
    const int t = t0 + tl;
    const bool valid = t < a.T;
    float z[VPL], s[VPL];
    bool finite = true;
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lg + LG * v;
      float zz = 0.0f;
#pragma unroll
      for (int q = 0; q < KS; ++q) zz += zs[q][tl][e];
      zz += ob[e];
      if (a.noise && valid && e < E) {
        // H = z + noise * softplus(x . W_noise)
        const float zn = a.noise_logit[int64_t(t) * E + e];
        zz += a.noise[int64_t(t) * E + e] * softplus_fast(zn);
      }
      z[v] = zz;
      if (e < E) {
        m = fmaxf(m, zz);
        finite = finite && isfinite(zz);
      }
    }
    if (a.logits_only) {
      if (valid)
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          if (lg + LG * v < E) a.logits[int64_t(t) * E + lg + LG * v] = z[v];
      continue;
    }
    if (a.logits && valid)
#pragma unroll
      for (int v = 0; v < VPL; ++v)
        if (lg + LG * v < E) a.logits[int64_t(t) * E + lg + LG * v] = z[v];
    m = row_max<LG>(m);
    float sexp = 0.0f;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      if (lg + LG * v < E) sexp += exp_fast(z[v] - m);
    sexp = row_sum<LG>(sexp);
    // divisions as one reciprocal per token (within an ulp of the quotients)
    const float rsexp = 1.0f / sexp;
    float ssum = 0.0f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lg + LG * v;
      float sv;
      if (a.score == 0) {
        sv = exp_fast(z[v] - m) * rsexp;
      } else if (a.score == 1) {
        sv = __builtin_amdgcn_rcpf(1.0f + exp_fast(-z[v]));
      } else {
        sv = __builtin_amdgcn_sqrtf(softplus_fast(z[v]));
      }
      s[v] = e < E ? sv : 0.0f;
      ssum += s[v];
    }
    ssum = row_sum<LG>(ssum);
    const float rssum = 1.0f / ssum;
    const float lse = m + logf(sexp);

    // Selection keys: order_key(s + bias) + 1 (at least 1 for every real
    // expert, NaN included), 0 for padding and for experts already taken.
    // The expert index, the tie-breaker, is implied by the register slot.
    uint32_t key[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lg + LG * v;
      key[v] = e < E ? order_key(s[v] + ob[EP + e]) + 1u : 0u;
    }
    // k selection rounds, kept rolled (the per-expert work inside is
    // unrolled): lane j of the token's group keeps round j's expert and gate,
    // which it writes below; the first two gates are kept for the random
    // second-expert rule.
    int my_e = 0;
    float my_g = 0.0f, g0 = 0.0f, g1 = 0.0f, gs = 0.0f;
#pragma unroll 1
    for (int j = 0; j < k; ++j) {
      int e;
      if (a.routing == 1) {
        e = int((int64_t(t) * k + j) % E);
      } else if (a.routing == 4) {
        e = valid ? int((int64_t(fmix32(uint32_t(a.token_ids[t]))) + j) % E) : 0;
      } else {
        // this lane's best (ascending v with a strict test: the lowest expert
        // wins a tie), then the group's: larger key, then lower expert
        uint32_t bk = 0;
        int bv = 0;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          if (key[v] > bk) {
            bk = key[v];
            bv = v;
          }
        uint64_t best = bk ? (uint64_t(bk) << 32) | uint32_t(~uint32_t(lg + LG * bv)) : 0ull;
        best = row_max_u64<LG>(best);
        e = int(~uint32_t(best));
      }
      float sv = 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v)
        if (lg + LG * v == e) {
          sv = s[v];
          key[v] = 0;
        }
      // the owner's score (the other lanes add zeros: exact)
      const float ge = row_sum<LG>(sv);
      if (lg == j) {
        my_e = e;
        my_g = ge;
      }
      if (j == 0) g0 = ge;
      if (j == 1) g1 = ge;
      gs += ge;
    }
    // Random second expert (k = 2): keep it iff u < 2 s2 / (s1 + s2); a skipped
    // slot is reported as E + expert and not counted.
    bool skip2 = false;
    if (a.routing == 3 && valid) skip2 = !(a.uniform[t] < 2.0f * g1 / (g0 + g1));
    if (valid) {
      if (lg < k) {
        if (!(lg == 1 && skip2)) atomicAdd(&red_c[my_e], 1);
        const float g = a.renorm ? (my_g / gs) * a.gate_scale : my_g * a.gate_scale;
        a.idx[int64_t(t) * k + lg] = my_e + ((lg == 1 && skip2) ? E : 0);
        a.gate[int64_t(t) * k + lg] = g;
      }
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int e = lg + LG * v;
        if (e < E) {
          if (a.scores) a.scores[int64_t(t) * E + e] = s[v];
          pacc[v] += s[v] * rssum;
        }
      }
      lse2 += lse * lse;
      nf += finite ? 0 : 1;
    }
  }
  // Combine the groups of a wave, then the waves, in a fixed order.
#pragma unroll
  for (int msk = LG; msk < 64; msk <<= 1) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) pacc[v] += shfl_xor(pacc[v], msk);
    lse2 += shfl_xor(lse2, msk);
    nf += shfl_xor(nf, msk);
  }
  if (gi == 0) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) red_p[w * EP + lg + LG * v] = pacc[v];
  }
  if (l == 0) {
    red_s[w] = lse2;
    red_s[NW + w] = __int_as_float(nf);
  }
  __syncthreads();
  const int blk = blockIdx.x;
  for (int e = tid; e < EP; e += blockDim.x) {
    float ps = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) ps += red_p[ww * EP + e];
    a.part_p[int64_t(blk) * EP + e] = ps;
    a.part_cnt[int64_t(blk) * EP + e] = red_c[e];
  }
  if (tid == 0) {
    float ls = 0.0f;
    int32_t ns = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      ls += red_s[ww];
      ns += __float_as_int(red_s[NW + ww]);
    }
    a.part_lse2[blk] = ls;
    a.part_nf[blk] = ns;
  }
}

// ---------------------------------------------------------------------------
// bf16 tokens: a block of 8 waves covers 64 tokens (two 32-token halves,
// H = 2; 32 tokens, H = 1, for small batches) and all EP experts, and the
// logits never leave the chip.  The waves split the work into NB = EP / 32 expert blocks times
// KS = 8 / NB d-ranges: wave w computes expert block eb = w % NB over d-range
// kp = w / NB for both 32-token halves, so each plane piece of Wg is loaded
// once per block, by one wave, straight into registers from the fragment
// layout (1 KB contiguous per wave load).  The block's token rows are shared
// through LDS: rows of 128 B (one 64-k chunk) whose 16-byte pieces are
// XOR-swizzled by (row >> 1) & 7, so the fragment reads are conflict-free.
// Wg is read as fp32 (two thirds of the bytes of three bf16 planes) and split
// on chip, per MFMA step, into hi = rne(w), mid = rne(w - hi),
// lo = rne(w - hi - mid) with the bf16 conversion instruction; each residual
// is exact, so hi + mid + lo == w.  The three planes accumulate into the same
// registers: z = sum over k and planes of the exact products x * plane, one
// fp32 sum.
// At chunk j a wave stores chunk j+1's token rows (loaded one chunk earlier)
// to LDS, loads chunk j+2's plane pieces (three register sets in rotation)
// and chunk j+1's token rows into registers, and multiplies chunk j.  Every
// wait is for a register, so the compiler's waits are exact.  Block b walks
// its chunks starting at chunk b mod (chunks): concurrent blocks read
// different parts of Wg, spreading their requests over the L2 channels (the
// sum order depends only on the block).  The LDS slots hold the logits after
// the loop.
template <int EP, int H>
__global__ __launch_bounds__(512) void route_wide_kernel(RouteArgs a) {
  constexpr int NW = 8;
  constexpr int NB = EP / 32;
  constexpr int KS = NW / NB;
  constexpr int BT = 32 * H;                       // tokens per block (H 32-token halves)
  constexpr int XL = KS * H / 2;                   // token-row loads per wave and chunk
  static_assert(KS * H % 2 == 0, "whole 1 KB row groups per wave");
  constexpr int XSLOT = KS * BT * 64;              // bf16 elements of one chunk's token rows
  // register sets of plane pieces in rotation (and LDS slots of token rows):
  // three (loads two chunks ahead), two with four or eight d-ranges (register
  // and LDS budget)
  constexpr int P = KS >= 4 ? 2 : 3;
  constexpr int D = P - 1;                         // chunks ahead
  constexpr int RING = P * XSLOT * 2;
  constexpr int ZSB = KS * BT * (EP + 1) * 4;
  __shared__ __attribute__((aligned(16))) char smem[RING > ZSB ? RING : ZSB];
  __shared__ float red_p[NW * EP];
  __shared__ int32_t red_c[EP];
  __shared__ float red_s[2 * NW];
  __shared__ float ob[2 * EP];
  uint4* const xs = reinterpret_cast<uint4*>(smem);

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int t0 = blockIdx.x * BT;
  const int eb = w % NB, kp = w / NB;
  const int dpart = a.d / KS;
  const int C = a.d / 64, CK = C / KS;   // 64-k chunks in all, per d-range
  const int rot = blockIdx.x % CK;
  const int fr = l & 31, fg = l >> 5;

  // Token rows: load i of wave w is 1 KB row group n = w + 8i, i.e. rows
  // 8 (n % 4H) + l/8 of d-range n / 4H; lane l holds physical piece l%8 of
  // its row, i.e. logical piece (l%8) ^ ((row >> 1) & 7).  Rows past T repeat
  // row T-1 (their tokens are never stored).
  const uint16_t* xsrc[XL];
  int xdst[XL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int n = w + 8 * i, q = n / (4 * H), row = 8 * (n % (4 * H)) + (l >> 3);
    xsrc[i] = static_cast<const uint16_t*>(a.x) + int64_t(min(t0 + row, a.T - 1)) * a.d +
              q * dpart + 8 * ((l & 7) ^ ((row >> 1) & 7));
    xdst[i] = (q * BT + row) * 8 + (l & 7);
  }
  const uint4* wf = reinterpret_cast<const uint4*>(a.wfrag) +
                    (int64_t(eb) * C + int64_t(kp) * CK) * 8 * 64 + l;
  // fragment pieces of this lane (uint4 units): rows fr (and 32 + fr),
  // logical piece 4 fg + s
  const int xo0 = (kp * BT + fr) * 8;
  const int xo1 = xo0 + 32 * 8;
  const int xsw = (fr >> 1) & 7;   // same for rows fr and 32 + fr

  floatx16 acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    acc0[r] = 0.0f;
    acc1[r] = 0.0f;
  }
  // the chunk of d-range column j of this block (j clamped to the last one,
  // so the first issues can be unconditional: every path into the loop has
  // then loaded the sets in the same order)
  auto chunk = [&](int j) {
    const int c = min(j, CK - 1) + rot;
    return c < CK ? c : c - CK;
  };
  uint4 xn[XL];
  auto load_x = [&](int j) {
    const int c = chunk(j);
#pragma unroll
    for (int i = 0; i < XL; ++i) xn[i] = ld16(xsrc[i] + 64 * c);
  };
  auto store_x = [&](uint4* slot) {
#pragma unroll
    for (int i = 0; i < XL; ++i) slot[xdst[i]] = xn[i];
  };
  // lanes of padding experts (zero weights) load nothing
  const bool wlive = 32 * eb + (l & 31) < a.E;
  // With 17 to 32 experts (no fragment layout given) Wg is small and is read
  // as stored, [d, E]: lane l takes the 32 k of its expert column that the
  // fragment layout would hold (the lanes of one k row read adjacent experts,
  // at least 68 contiguous bytes), so no layout pass runs.  Fewer experts
  // leave too few live lanes per load instruction for this to pay.
  const bool wdirect = EP == 32 && a.wfrag == nullptr;
  const float* wcol = a.Wg + (int64_t(kp) * dpart + 32 * fg) * a.E + 32 * eb + (l & 31);
  auto load_w = [&](int j, uint4 (&wr)[8]) {
    if (wdirect) {
      const float* src = wcol + int64_t(64 * chunk(j)) * a.E;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = wlive ? __float_as_uint(src[(4 * i + u) * a.E]) : 0u;
        wr[i] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    } else {
      const uint4* src = wf + int64_t(chunk(j)) * 8 * 64;
#pragma unroll
      for (int i = 0; i < 8; ++i) wr[i] = wlive ? src[64 * i] : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  // the three bf16 planes of eight fp32 weights (pieces u0, u1)
  auto split8 = [](const uint4& u0, const uint4& u1, bf16x8& ph, bf16x8& pm, bf16x8& pl) {
    const uint32_t f[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    uint32_t h[4], m[4], o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float w0 = __uint_as_float(f[2 * i]), w1 = __uint_as_float(f[2 * i + 1]);
      h[i] = pack_bf2(w0, w1);
      const float r0 = w0 - __uint_as_float(h[i] << 16);
      const float r1 = w1 - __uint_as_float(h[i] & 0xffff0000u);
      m[i] = pack_bf2(r0, r1);
      o[i] = pack_bf2(r0 - __uint_as_float(m[i] << 16), r1 - __uint_as_float(m[i] & 0xffff0000u));
    }
    ph = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
    pm = __builtin_bit_cast(bf16x8, make_uint4(m[0], m[1], m[2], m[3]));
    pl = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
  };
  // One chunk.  FULL: the chunks loaded here exist (inside the loop), so the
  // loads and the store are unconditional.
  auto step = [&](auto full, int j, const uint4* rslot, const uint4 (&cur)[8], uint4* xslot,
                  uint4 (&nxt)[8]) {
    constexpr bool FULL = decltype(full)::value;
    // every wave's stores of chunk j's token rows are visible, and every wave
    // has read the chunk whose slot is stored next
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS stores are done
    lds_barrier();
    uint4 xa[4], xb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      xa[s] = rslot[xo0 + ((4 * fg + s) ^ xsw)];
      if constexpr (H == 2) xb[s] = rslot[xo1 + ((4 * fg + s) ^ xsw)];
    }
    if (FULL || j + 1 < CK) {
      store_x(xslot);
      if (FULL || j + 2 < CK) load_x(j + 2);
    }
    if (FULL || j + D < CK) load_w(j + D, nxt);
    __builtin_amdgcn_sched_barrier(0);   // the loads go out before the MFMAs
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 b[3];
      split8(cur[2 * s], cur[2 * s + 1], b[0], b[1], b[2]);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa[s]), b[p],
                                                       acc0, 0, 0, 0);
        if constexpr (H == 2)
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xb[s]), b[p],
                                                         acc1, 0, 0, 0);
      }
    }
  };
  uint4 r[P][8];
  load_x(0);
#pragma unroll
  for (int u = 0; u < D; ++u) load_w(u, r[u]);
  store_x(xs);
  load_x(1);
  // whole rotations whose loads and stores all exist in the loop, the last
  // chunks after it
  const std::true_type full{};
  const std::false_type tail{};
  int j = 0;
  for (; j + P + 2 <= CK; j += P) {
#pragma unroll
    for (int u = 0; u < P; ++u)
      step(full, j + u, xs + u * (XSLOT / 8), r[u], xs + ((u + 1) % P) * (XSLOT / 8),
           r[(u + D) % P]);
  }
#pragma unroll
  for (int u = 0; u < P + 1; ++u)
    if (j + u < CK)
      step(tail, j + u, xs + (u % P) * (XSLOT / 8), r[u % P], xs + ((u + 1) % P) * (XSLOT / 8),
           r[(u + D) % P]);
  __syncthreads();   // every wave has read its last token rows; the slots become zs
  auto zs = reinterpret_cast<float (*)[BT][EP + 1]>(smem);
  // D[i][j] of a 32x32 block: lane l holds column j = l%32 and rows
  // i = 8*(r/4) + 4*(l/32) + r%4 in accumulator register r.
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 8 * (r >> 2) + 4 * fg + (r & 3);
    zs[kp][i][eb * 32 + fr] = acc0[r];
    if constexpr (H == 2) zs[kp][32 + i][eb * 32 + fr] = acc1[r];
  }
  __syncthreads();
  route_epilogue<EP, KS, NW, BT>(a, zs, t0, red_p, red_c, red_s, ob);
}

// ---------------------------------------------------------------------------
// Plain FMA logits (fp32 tokens, or d not a multiple of the wide kernel's d-ranges).
template <int EP>
__global__ __launch_bounds__(256) void route_simt_kernel(RouteArgs a) {
  constexpr int NW = 4;
  __shared__ float zs[1][ROUTE_BT][EP + 1];
  __shared__ float red_p[NW * EP];
  __shared__ int32_t red_c[EP];
  __shared__ float red_s[2 * NW];
  __shared__ float ob[2 * EP];
  const int t0 = blockIdx.x * ROUTE_BT;
  for (int o = threadIdx.x; o < ROUTE_BT * EP; o += blockDim.x) {
    const int tl = o / EP, e = o % EP;
    const int t = min(t0 + tl, a.T - 1);
    float acc = 0.0f;
    if (e < a.E) {
      if (a.x_bf16) {
        const uint16_t* xr = static_cast<const uint16_t*>(a.x) + int64_t(t) * a.d;
        for (int kk = 0; kk < a.d; ++kk) acc = fmaf(bf2f(xr[kk]), a.Wg[int64_t(kk) * a.E + e], acc);
      } else {
        const float* xr = static_cast<const float*>(a.x) + int64_t(t) * a.d;
        for (int kk = 0; kk < a.d; ++kk) acc = fmaf(xr[kk], a.Wg[int64_t(kk) * a.E + e], acc);
      }
    }
    zs[0][tl][e] = acc;
  }
  __syncthreads();
  route_epilogue<EP, 1, NW>(a, zs, t0, red_p, red_c, red_s, ob);
}

// ---------------------------------------------------------------------------
// One block of 1024 threads: per-expert totals over the route blocks and the
// two losses.  L_aux = aux_coef * E * sum_e (count_e / (T k)) * (P_e / T);
// L_z = z_coef * sum_t lse_t^2 / T.  Lane (c, q) owns experts 4c..4c+3 and
// sums blocks b = q, q + L, ... in order (16-byte loads, eight blocks' loads
// in flight); the L lanes of a column, then the experts, are combined by
// fixed-shape trees, in double.  The result depends only on the shape.
__global__ __launch_bounds__(1024) void route_reduce_kernel(RouteArgs a, int nblk, float aux_coef,
                                                            float z_coef, int32_t* counts,
                                                            float* losses, int32_t* n_nonfinite) {
  __shared__ double sp[4096];
  __shared__ int64_t sc[4096];
  __shared__ double sl[1024];
  __shared__ int64_t sn[1024];
  const int tid = threadIdx.x;
  const int EP = a.EP, EP4 = EP / 4, L = 1024 / EP4;
  const int c = tid % EP4, q = tid / EP4;
  double P[4] = {0.0, 0.0, 0.0, 0.0};
  int64_t C[4] = {0, 0, 0, 0};
  {
    const float4* pp = reinterpret_cast<const float4*>(a.part_p) + c;
    const int4* pc = reinterpret_cast<const int4*>(a.part_cnt) + c;
    int b = q;
    for (; b + 7 * L < nblk; b += 8 * L) {
      float4 vp[8];
      int4 vc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        vp[u] = pp[int64_t(b + u * L) * EP4];
        vc[u] = pc[int64_t(b + u * L) * EP4];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        P[0] += double(vp[u].x); P[1] += double(vp[u].y);
        P[2] += double(vp[u].z); P[3] += double(vp[u].w);
        C[0] += vc[u].x; C[1] += vc[u].y; C[2] += vc[u].z; C[3] += vc[u].w;
      }
    }
    for (; b < nblk; b += L) {
      const float4 vp = pp[int64_t(b) * EP4];
      const int4 vc = pc[int64_t(b) * EP4];
      P[0] += double(vp.x); P[1] += double(vp.y); P[2] += double(vp.z); P[3] += double(vp.w);
      C[0] += vc.x; C[1] += vc.y; C[2] += vc.z; C[3] += vc.w;
    }
  }
  double l2 = 0.0;
  int64_t nf = 0;
#pragma unroll 4
  for (int b = tid; b < nblk; b += 1024) {
    l2 += double(a.part_lse2[b]);
    nf += a.part_nf[b];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sp[q * EP + 4 * c + j] = P[j];
    sc[q * EP + 4 * c + j] = C[j];
  }
  sl[tid] = l2;
  sn[tid] = nf;
  __syncthreads();
  // lanes of each expert (rows q of sp / sc) and the lse / nonfinite sums:
  // pairwise trees of a fixed shape
  for (int h = L / 2; h > 0; h >>= 1) {
    for (int i = tid; i < h * EP; i += 1024) {
      sp[i] += sp[i + h * EP];
      sc[i] += sc[i + h * EP];
    }
    __syncthreads();
  }
  for (int h = 512; h > 0; h >>= 1) {
    if (tid < h) {
      sl[tid] += sl[tid + h];
      sn[tid] += sn[tid + h];
    }
    __syncthreads();
  }
  // per-expert terms, then a fixed-order tree over experts (sl's upper half
  // is free again and holds the terms)
  double* term = sl + 512;
  if (tid < 256) {
    double t = 0.0;
    if (tid < a.E) {
      if (counts) counts[tid] = int32_t(sc[tid]);
      t = (double(sc[tid]) / (double(a.T) * a.k)) * (sp[tid] / a.T);
    }
    term[tid] = t;
  }
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (tid < h) term[tid] += term[tid + h];
    __syncthreads();
  }
  if (tid == 0) {
    if (losses) {
      losses[0] = aux_coef != 0.0f ? float(double(aux_coef) * a.E * term[0]) : 0.0f;
      losses[1] = z_coef != 0.0f ? float(double(z_coef) * sl[0] / a.T) : 0.0f;
    }
    if (n_nonfinite) n_nonfinite[0] = int32_t(sn[0]);
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_wg_frag(const float* Wg, int d, int E, int EP, float* out, hipStream_t st) {
  if (d % 64 || EP % 32) return hipErrorInvalidValue;
  wg_frag_kernel<<<dim3(unsigned(d / 64), unsigned(EP / 32)), dim3(256), 0, st>>>(
      Wg, d, E, reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

// Tokens per wide-kernel block: 64, or 32 when 64-token blocks would leave
// compute units idle (fewer than 256 of them) and the experts' d-ranges allow
// it (not with 256 padded experts: one d-range needs whole 64-row groups).
int route_wide_bt(int64_t T, int EP) { return EP < 256 && cdiv(T, 64) < 256 ? 32 : 64; }

hipError_t launch_route_wide(const RouteArgs& a, hipStream_t st) {
  const bool small = route_wide_bt(a.T, a.EP) == 32;
  const unsigned nblk = unsigned(cdiv(a.T, small ? 32 : 64));
  switch (a.EP) {
    case 32:
      if (small) route_wide_kernel<32, 1><<<nblk, 512, 0, st>>>(a);
      else route_wide_kernel<32, 2><<<nblk, 512, 0, st>>>(a);
      break;
    case 64:
      if (small) route_wide_kernel<64, 1><<<nblk, 512, 0, st>>>(a);
      else route_wide_kernel<64, 2><<<nblk, 512, 0, st>>>(a);
      break;
    case 128:
      if (small) route_wide_kernel<128, 1><<<nblk, 512, 0, st>>>(a);
      else route_wide_kernel<128, 2><<<nblk, 512, 0, st>>>(a);
      break;
    case 256: route_wide_kernel<256, 2><<<nblk, 512, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  const unsigned nblk = unsigned(cdiv(a.T, ROUTE_BT));
  switch (a.EP) {
    case 32: route_simt_kernel<32><<<dim3(nblk), dim3(256), 0, st>>>(a); break;
    case 64: route_simt_kernel<64><<<dim3(nblk), dim3(256), 0, st>>>(a); break;
    case 128: route_simt_kernel<128><<<dim3(nblk), dim3(256), 0, st>>>(a); break;
    case 256: route_simt_kernel<256><<<dim3(nblk), dim3(256), 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_route_reduce(const RouteArgs& a, int nblk, float aux_coef, float z_coef,
                               int32_t* counts, float* losses, int32_t* n_nonfinite,
                               hipStream_t st) {
  route_reduce_kernel<<<dim3(1), dim3(1024), 0, st>>>(a, nblk, aux_coef, z_coef, counts, losses,
                                                      n_nonfinite);
  return hipGetLastError();
}

}  // namespace moe
