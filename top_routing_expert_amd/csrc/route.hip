// Router of the sparse MoE layer for gfx950.
//
// z = x . Wg (+ offset) in FP32, scores, selection-only bias, top-k with
// lowest-index tie-breaking, gates, and per-block partial sums for the load
// balance and z losses ("Mixture of Experts Explained", "What is sparsity?"
// gating equations and "Switch Transformers" full-precision router; handbook
// news digest, "confirmed" bullets on sigmoid / sqrt(softplus) scoring).
//
// The logits are an [T, d] x [d, E] contraction.  With bf16 tokens it runs on
// bf16 MFMA: Wg is split once per call into three bf16 planes whose sum is
// exactly Wg, so every product x*w is formed exactly and accumulated in FP32.
// fp32 tokens use a plain FMA loop.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

int route_pad_experts(int E) { return E <= 32 ? 32 : E <= 64 ? 64 : E <= 128 ? 128 : 256; }

// ---------------------------------------------------------------------------
// Wg [d, E] fp32 -> three bf16 planes [3][EP][d], expert-major (K-contiguous),
// followed by pad_rows zero rows (the planes are also the B operand [rows, d] of
// the logits GEMM, whose row count must be a multiple of 128); off1, when
// given, receives the row offsets {0, T} of that GEMM's single group.
// hi = rne(w), mid = rne(w - hi), lo = rne(w - hi - mid); each residual is
// exact in fp32 and the last has at most 8 significant bits, so
// hi + mid + lo == w for every normal w.  Experts e >= E are zero.
__global__ void wg_split_kernel(const float* __restrict__ Wg, int d, int E, int EP, int pad_rows,
                                uint16_t* __restrict__ out, int32_t* __restrict__ off1, int T) {
  const int64_t n = int64_t(EP) * d;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i == 0 && off1) {
    off1[0] = 0;
    off1[1] = T;
  }
  if (i >= n) return;
  if (i < int64_t(pad_rows) * d) out[3 * n + i] = 0;
  const int e = int(i / d), kk = int(i % d);
  const float w = e < E ? Wg[int64_t(kk) * E + e] : 0.0f;
  const uint16_t hi = f2bf(w);
  const float r1 = w - bf2f(hi);
  const uint16_t mid = f2bf(r1);
  const float r2 = r1 - bf2f(mid);
  out[i] = hi;
  out[n + i] = mid;
  out[2 * n + i] = f2bf(r2);
}

// ---------------------------------------------------------------------------
// Per-token epilogue shared by both logit kernels (NW waves per block).  zs
// holds KS partial logit sums for the block's 32 tokens.  Each token is
// handled by a group of LG = 16 lanes (one DPP row, four tokens per wave at
// a time), each owning VPL experts e = lane_in_group + LG * v; all per-token
// reductions stay inside the row.  LDS scratch: red_p [NW * EP], red_c [EP]
// (the block's routed-slot counts, integer LDS atomics: exact in any order),
// red_s [2 * NW].
template <int EP, int KS, int NW>
__device__ __forceinline__ void route_epilogue(const RouteArgs& a, float (*zs)[ROUTE_BT][EP + 1],
                                               int t0, float* red_p, int32_t* red_c,
                                               float* red_s) {
  constexpr int LG = EP < 16 ? EP : 16;
  constexpr int TPI = 64 / LG;
  constexpr int VPL = EP / LG;
  constexpr int KMAX = 16;
  constexpr int TOK_PER_WAVE = ROUTE_BT / NW;
  static_assert(TOK_PER_WAVE % TPI == 0, "tokens per wave");
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int gi = l / LG, lg = l % LG;
  const int E = a.E, k = a.k;

  float pacc[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) pacc[v] = 0.0f;
  for (int e = tid; e < EP; e += NW * 64) red_c[e] = 0;
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
      zz += (a.offset && e < E) ? a.offset[e] : 0.0f;
      if (a.noise && valid && e < E) {
        // H = z + noise * softplus(x . W_noise)
        const float zn = a.noise_logit[int64_t(t) * E + e];
        zz += a.noise[int64_t(t) * E + e] * (fmaxf(zn, 0.0f) + log1pf(expf(-fabsf(zn))));
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
      if (lg + LG * v < E) sexp += expf(z[v] - m);
    sexp = row_sum<LG>(sexp);
    // divisions as one reciprocal per token (within an ulp of the quotients)
    const float rsexp = 1.0f / sexp;
    float ssum = 0.0f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lg + LG * v;
      float sv;
      if (a.score == 0) {
        sv = expf(z[v] - m) * rsexp;
      } else if (a.score == 1) {
        sv = __builtin_amdgcn_rcpf(1.0f + expf(-z[v]));
      } else {
        sv = sqrtf(fmaxf(z[v], 0.0f) + log1pf(expf(-fabsf(z[v]))));
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
      key[v] = e < E ? order_key(s[v] + ((a.bias) ? a.bias[e] : 0.0f)) + 1u : 0u;
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
// bf16 tokens: logits on MFMA 32x32x16.  A block of 8 waves covers 32 tokens
// and all EP experts: wave w computes output block (w % NB) (32 experts) over
// the d-range (w / NB) of KS = 8 / NB parts, summed in order afterwards.
// Within a 64-wide K chunk a lane loads 32 contiguous k of its token row and
// of its expert row in each Wg plane; MFMA step s uses elements 8s..8s+7 of
// them, the same permutation of k for both operands.  All loads of a chunk
// are issued together and the next chunk is prefetched during the MFMAs.
template <int EP>
__global__ __launch_bounds__(512) void route_mfma_kernel(RouteArgs a) {
  constexpr int NW = 8;
  constexpr int NB = EP / 32;
  constexpr int KS = NW / NB;
  __shared__ float zs[KS][ROUTE_BT][EP + 1];
  __shared__ float red_p[NW * EP];
  __shared__ int32_t red_c[EP];
  __shared__ float red_s[2 * NW];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int t0 = blockIdx.x * ROUTE_BT;
  const int eb = w % NB, kp = w / NB;
  const int dpart = a.d / KS;
  const int row = l & 31, g = l >> 5;
  const int trow = min(t0 + row, a.T - 1);
  const uint16_t* xr = static_cast<const uint16_t*>(a.x) + int64_t(trow) * a.d + kp * dpart + 32 * g;
  const int64_t plane = int64_t(EP) * a.d;
  const uint16_t* wr = a.wsplit + int64_t(eb * 32 + row) * a.d + kp * dpart + 32 * g;

  floatx16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

  // Rows of padding experts (eb*32 + row >= E) are zero in every plane: their
  // lanes load nothing and multiply zeros.
  const bool wlive = eb * 32 + row < a.E;
  uint4 xa[4], wv[3][4], xb[4], wb[3][4];
  auto load = [&](int kc, uint4 (&xo)[4], uint4 (&wo)[3][4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) xo[q] = ld16(xr + kc + 8 * q);
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        wo[p][q] = wlive ? ld16(wr + p * plane + kc + 8 * q) : make_uint4(0, 0, 0, 0);
  };
  // Two chunks in flight: chunk c+2 is loaded while chunk c multiplies.
  load(0, xa, wv);
  if (64 < dpart) load(64, xb, wb);
  for (int kc = 0; kc < dpart; kc += 64) {
    uint4 xc[4], wc[3][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xc[q] = xa[q];
      xa[q] = xb[q];
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        wc[p][q] = wv[p][q];
        wv[p][q] = wb[p][q];
      }
    }
    if (kc + 128 < dpart) load(kc + 128, xb, wb);
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xc[s]),
                                                      __builtin_bit_cast(bf16x8, wc[p][s]), acc,
                                                      0, 0, 0);
  }
  // D[i][j] of a 32x32 block: lane l holds column j = l%32 and rows
  // i = 8*(r/4) + 4*(l/32) + r%4 in accumulator register r.
#pragma unroll
  for (int r = 0; r < 16; ++r) zs[kp][8 * (r >> 2) + 4 * g + (r & 3)][eb * 32 + row] = acc[r];
  __syncthreads();
  route_epilogue<EP, KS, NW>(a, zs, t0, red_p, red_c, red_s);
}

// ---------------------------------------------------------------------------
// Plain FMA logits (fp32 tokens, or shapes the MFMA tiling does not cover).
template <int EP>
__global__ __launch_bounds__(256) void route_simt_kernel(RouteArgs a) {
  constexpr int NW = 4;
  __shared__ float zs[1][ROUTE_BT][EP + 1];
  __shared__ float red_p[NW * EP];
  __shared__ int32_t red_c[EP];
  __shared__ float red_s[2 * NW];
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
  route_epilogue<EP, 1, NW>(a, zs, t0, red_p, red_c, red_s);
}

// ---------------------------------------------------------------------------
// One block of 1024 threads: per-expert totals over the route blocks and the
// two losses.  L_aux = aux_coef * E * sum_e (count_e / (T k)) * (P_e / T);
// L_z = z_coef * sum_t lse_t^2 / T.  Lane q of expert e sums blocks
// b = q, q + L, ... in order; lanes, then experts, are combined in a fixed
// order, in double.
__global__ __launch_bounds__(1024) void route_reduce_kernel(RouteArgs a, int nblk, float aux_coef,
                                                            float z_coef, int32_t* counts,
                                                            float* losses, int32_t* n_nonfinite) {
  __shared__ double sp[1024];
  __shared__ int64_t sc[1024];
  __shared__ double sl[1024];
  __shared__ int64_t sn[1024];
  const int tid = threadIdx.x;
  const int EP = a.EP, L = 1024 / EP;
  const int e = tid % EP, q = tid / EP;
  double P = 0.0;
  int64_t c = 0;
  if (e < a.E) {
#pragma unroll 8
    for (int b = q; b < nblk; b += L) {
      P += double(a.part_p[int64_t(b) * EP + e]);
      c += a.part_cnt[int64_t(b) * EP + e];
    }
  }
  double l2 = 0.0;
  int64_t nf = 0;
#pragma unroll 4
  for (int b = tid; b < nblk; b += 1024) {
    l2 += double(a.part_lse2[b]);
    nf += a.part_nf[b];
  }
  sp[tid] = P;
  sc[tid] = c;
  sl[tid] = l2;
  sn[tid] = nf;
  __syncthreads();
  // lanes of each expert -> lane 0 (fixed order); lse / nonfinite tree
  if (q == 0) {
    for (int qq = 1; qq < L; ++qq) {
      sp[e] += sp[qq * EP + e];
      sc[e] += sc[qq * EP + e];
    }
  }
  for (int s = 512; s > 0; s >>= 1) {
    if (tid < s) {
      sl[tid] += sl[tid + s];
      sn[tid] += sn[tid + s];
    }
    __syncthreads();
  }
  // per-expert terms, then a fixed-order tree over experts (reusing sp as the term buffer)
  double term = 0.0;
  if (tid < a.E) {
    if (counts) counts[tid] = int32_t(sc[tid]);
    term = (double(sc[tid]) / (double(a.T) * a.k)) * (sp[tid] / a.T);
  }
  __syncthreads();
  sp[tid] = tid < EP ? term : 0.0;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (tid < s) sp[tid] += sp[tid + s];
    __syncthreads();
  }
  if (tid == 0) {
    if (losses) {
      losses[0] = aux_coef != 0.0f ? float(double(aux_coef) * a.E * sp[0]) : 0.0f;
      losses[1] = z_coef != 0.0f ? float(double(z_coef) * sl[0] / a.T) : 0.0f;
    }
    if (n_nonfinite) n_nonfinite[0] = int32_t(sn[0]);
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_wg_split(const float* Wg, int d, int E, int EP, int pad_rows, uint16_t* out,
                           int32_t* off1, int T, hipStream_t st) {
  if (pad_rows > EP) return hipErrorInvalidValue;
  const int64_t n = int64_t(EP) * d;
  wg_split_kernel<<<dim3(unsigned(cdiv(n, 256))), dim3(256), 0, st>>>(Wg, d, E, EP, pad_rows, out,
                                                                      off1, T);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Route from the logits GEMM's output: z3 [T, ldz] fp32 holds, per token, the
// three plane products x . q_p at columns p*EP + e (p = 0, 1, 2), added here
// in plane order.
template <int EP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4)))
void route_from_partials_kernel(RouteArgs a, const float* z3, int ldz) {
  constexpr int NW = 8;
  __shared__ float zs[1][ROUTE_BT][EP + 1];
  __shared__ float red_p[NW * EP];
  __shared__ int32_t red_c[EP];
  __shared__ float red_s[2 * NW];
  const int t0 = blockIdx.x * ROUTE_BT;
  // every load of the block's slab is issued before the first use
  constexpr int PER = ROUTE_BT * EP / (64 * NW);
  float v[PER][3];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int o = threadIdx.x + 64 * NW * i;
    const int tl = o / EP, e = o % EP;
    const float* zr = z3 + int64_t(min(t0 + tl, a.T - 1)) * ldz + e;
    v[i][0] = zr[0];
    v[i][1] = zr[EP];
    v[i][2] = zr[2 * EP];
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int o = threadIdx.x + 64 * NW * i;
    zs[0][o / EP][o % EP] = (v[i][0] + v[i][1]) + v[i][2];
  }
  __syncthreads();
  route_epilogue<EP, 1, NW>(a, zs, t0, red_p, red_c, red_s);
}

hipError_t launch_route_from_partials(const RouteArgs& a, const float* z3, int ldz,
                                      hipStream_t st) {
  const unsigned nblk = unsigned(cdiv(a.T, ROUTE_BT));
  switch (a.EP) {
    case 32: route_from_partials_kernel<32><<<nblk, 512, 0, st>>>(a, z3, ldz); break;
    case 64: route_from_partials_kernel<64><<<nblk, 512, 0, st>>>(a, z3, ldz); break;
    case 128: route_from_partials_kernel<128><<<nblk, 512, 0, st>>>(a, z3, ldz); break;
    case 256: route_from_partials_kernel<256><<<nblk, 512, 0, st>>>(a, z3, ldz); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int EP>
static void launch_route_ep(const RouteArgs& a, bool mfma, hipStream_t st) {
  const unsigned nblk = unsigned(cdiv(a.T, ROUTE_BT));
  if (mfma)
    route_mfma_kernel<EP><<<dim3(nblk), dim3(512), 0, st>>>(a);
  else
    route_simt_kernel<EP><<<dim3(nblk), dim3(256), 0, st>>>(a);
}

hipError_t launch_route(const RouteArgs& a, bool mfma, hipStream_t st) {
  switch (a.EP) {
    case 32: launch_route_ep<32>(a, mfma, st); break;
    case 64: launch_route_ep<64>(a, mfma, st); break;
    case 128: launch_route_ep<128>(a, mfma, st); break;
    case 256: launch_route_ep<256>(a, mfma, st); break;
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
