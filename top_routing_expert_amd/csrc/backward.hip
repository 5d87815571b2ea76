// Backward pass pieces of the MoE layer for gfx950 (everything except the
// grouped expert GEMMs).
//
// The gradient is that of J = <dy, y> + L_aux + L_z.  Routing decisions (the
// kept experts, the drops) and the load fractions f_e are constants; the
// gradient reaches the router only through the kept gates ("Mixture of Experts
// Explained", "What is sparsity?": y = sum_i G(x)_i E_i(x) with G zero outside
// the top-k), plus the two router losses.
#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace moe {

constexpr int BWD_KMAX = 16;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

// ---------------------------------------------------------------------------
// Combine backward, one wave per token.  For kept slot j of token t:
//   dO[row] = gate[t,j] * dy[t]   (x element type, feeds the expert dgrad/wgrad)
//   dg[t,j] = <dy[t], o[row]>     (fp32; 0 for a dropped slot)
// and dy_x[t] = dy[t] in the x element type (the shared expert's gradient).
// As in the forward combine, each slot row of o is read through its own
// buffer descriptor (empty for a dropped slot), so the KM slot loads of a
// slab are in flight together; each lane visits its slabs in order.
template <bool BF16, int KM>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const float* __restrict__ dy, const float* __restrict__ o, const int32_t* __restrict__ ros,
    const float* __restrict__ gate, int T, int k, int d, void* __restrict__ dO,
    float* __restrict__ dg, void* __restrict__ dy_x) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (t >= T) return;
  const int my_row = l < k ? ros[int64_t(t) * k + l] : -1;
  const float my_g = l < k ? gate[int64_t(t) * k + l] : 0.0f;
  int rows[KM];
  float gs[KM], dot[KM];
  rsrc_t rs[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    rows[j] = __builtin_amdgcn_readlane(my_row, j);
    gs[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_g), j));
    rs[j] = make_rsrc(rows[j] >= 0 ? o + int64_t(rows[j]) * d : o, rows[j] >= 0 ? uint32_t(d) * 4 : 0u);
    dot[j] = 0.0f;
  }
  const float4* dyr = reinterpret_cast<const float4*>(dy + int64_t(t) * d);
  const int n4 = d >> 2;
  for (int c = l; c < n4; c += 64) {
    const float4 v = dyr[c];
    floatx4 ov[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      ov[j] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs[j], uint32_t(c) * 16, 0, 0));
    if (dy_x) {
      if constexpr (BF16)
        reinterpret_cast<uint2*>(static_cast<uint16_t*>(dy_x) + int64_t(t) * d)[c] =
            make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
      else
        reinterpret_cast<float4*>(static_cast<float*>(dy_x) + int64_t(t) * d)[c] = v;
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (rows[j] < 0) continue;
      dot[j] += v.x * ov[j][0] + v.y * ov[j][1] + v.z * ov[j][2] + v.w * ov[j][3];
      const float g = gs[j];
      if constexpr (BF16)
        reinterpret_cast<uint2*>(static_cast<uint16_t*>(dO) + int64_t(rows[j]) * d)[c] =
            make_uint2(pack_bf2(g * v.x, g * v.y), pack_bf2(g * v.z, g * v.w));
      else
        reinterpret_cast<float4*>(static_cast<float*>(dO) + int64_t(rows[j]) * d)[c] =
            make_float4(g * v.x, g * v.y, g * v.z, g * v.w);
    }
  }
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < k) {  // k is uniform over the wave
      const float s = wave_sum(dot[j]);
      if (l == 0) dg[int64_t(t) * k + j] = rows[j] >= 0 ? s : 0.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// Router backward, one wave per token; lane l owns experts l, l+64, l+128, l+192.
// From the saved logits z it recomputes the scores s, then
//   gates -> scores: renormalised gates g_j = scale * s_j / S (S = sum of kept s):
//     ds_j = scale / S * (dg_j - sum_i dg_i * s_i / S); otherwise ds_j = scale * dg_j;
//   aux loss L_aux = a * E * sum_e f_e * mean_t p_te, p = s / sum_e s:
//     ds_e += (c_e - sum_e' p_e' c_e') / sum_e s,  c_e = a * E * f_e / T;
//   scores -> logits: softmax Jacobian, s(1-s) for sigmoid, sigma(z) / (2 s) for
//     sqrt(softplus) (e^{z/2}/2 where s underflows);
//   z-loss L_z = b * mean_t lse_t^2:  dz_e += 2 b / T * lse * softmax(z)_e.
__global__ __launch_bounds__(256) void router_bwd_kernel(
    const float* __restrict__ z, const int32_t* __restrict__ idx, const float* __restrict__ dg,
    const int32_t* __restrict__ counts, int T, int E, int k, int score, int renorm, float scale,
    float aux_coef, float z_coef, float* __restrict__ dz) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (t >= T) return;
  constexpr int VPL = 4;
  float zv[VPL], s[VPL], ds[VPL];
  float m = -INFINITY;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = l + 64 * v;
    zv[v] = e < E ? z[int64_t(t) * E + e] : -INFINITY;
    if (e < E) m = fmaxf(m, zv[v]);
    ds[v] = 0.0f;
  }
  m = wave_max(m);
  float se = 0.0f;
#pragma unroll
  for (int v = 0; v < VPL; ++v)
    if (l + 64 * v < E) se += expf(zv[v] - m);
  se = wave_sum(se);
  float ssum = 0.0f;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = l + 64 * v;
    float sv = 0.0f;
    if (e < E) {
      if (score == 0) sv = expf(zv[v] - m) / se;
      else if (score == 1) sv = 1.0f / (1.0f + expf(-zv[v]));
      else sv = sqrtf(fmaxf(zv[v], 0.0f) + log1pf(expf(-fabsf(zv[v]))));
    }
    s[v] = sv;
    ssum += sv;
  }
  ssum = wave_sum(ssum);
  // kept gates
  int ix[BWD_KMAX];
  float dgv[BWD_KMAX], ssel[BWD_KMAX];
  float S = 0.0f;
#pragma unroll
  for (int j = 0; j < BWD_KMAX; ++j) {
    // a slot skipped by the random second-expert rule reads E + expert: it has
    // no gradient of its own (dg = 0) but stays in the gate normalisation
    ix[j] = j < k ? idx[int64_t(t) * k + j] : -1;
    if (ix[j] >= E && ix[j] < 2 * E) ix[j] -= E;
    dgv[j] = j < k ? dg[int64_t(t) * k + j] : 0.0f;
    ssel[j] = 0.0f;
    if (j < k && unsigned(ix[j]) < unsigned(E)) {
      const int slot = ix[j] >> 6;
      float mine = 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v)
        if (v == slot) mine = s[v];
      ssel[j] = __shfl(mine, ix[j] & 63, 64);
      S += ssel[j];
    }
  }
  float sum_dg_ghat = 0.0f;
  if (renorm) {
#pragma unroll
    for (int j = 0; j < BWD_KMAX; ++j)
      if (j < k) sum_dg_ghat += dgv[j] * (ssel[j] / S);
  }
#pragma unroll
  for (int j = 0; j < BWD_KMAX; ++j) {
    if (j >= k || unsigned(ix[j]) >= unsigned(E)) continue;
    const float dsel = renorm ? scale / S * (dgv[j] - sum_dg_ghat) : scale * dgv[j];
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      if (l + 64 * v == ix[j]) ds[v] += dsel;
  }
  if (aux_coef != 0.0f) {
    float c[VPL], pc = 0.0f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = l + 64 * v;
      c[v] = e < E ? aux_coef * float(E) * (float(counts[e]) / (float(T) * k)) / float(T) : 0.0f;
      pc += (s[v] / ssum) * c[v];
    }
    pc = wave_sum(pc);
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      if (l + 64 * v < E) ds[v] += (c[v] - pc) / ssum;
  }
  float dsum = 0.0f;
  if (score == 0) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) dsum += ds[v] * s[v];
    dsum = wave_sum(dsum);
  }
  const float lse = m + logf(se);
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = l + 64 * v;
    if (e >= E) continue;
    float d;
    if (score == 0) {
      d = s[v] * (ds[v] - dsum);
    } else if (score == 1) {
      d = ds[v] * s[v] * (1.0f - s[v]);
    } else {
      const float sig = 1.0f / (1.0f + expf(-zv[v]));
      d = ds[v] * (s[v] > 0.0f ? sig / (2.0f * s[v]) : 0.5f * expf(0.5f * zv[v]));
    }
    if (z_coef != 0.0f) d += 2.0f * z_coef / float(T) * lse * (expf(zv[v] - m) / se);
    dz[int64_t(t) * E + e] = d;
  }
}

// ---------------------------------------------------------------------------
// fp32 FMA GEMM with arbitrary strides for the router gradients:
//   P[kz][m][n] = sum over k in chunk kz of A(m,k) * B(k,n),
//   A(m,k) = A[m*sam + k*sak] (bf16 or fp32), B(k,n) = B[k*sbk + n*sbn] (fp32).
// 64x64 tiles, 256 threads with 4x4 micro-tiles; the k-chunks (grid.z) are
// summed afterwards in chunk order, so the result is deterministic.
template <typename TA>
__global__ __launch_bounds__(256) void strided_gemm_kernel(
    const TA* __restrict__ A, int64_t sam, int64_t sak, const float* __restrict__ B, int64_t sbk,
    int64_t sbn, int M, int N, int K, int kchunk, float* __restrict__ P) {
  __shared__ float As[16][68];
  __shared__ float Bs[16][68];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int kb = blockIdx.z * kchunk, ke = min(K, kb + kchunk);
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int k0 = kb; k0 < ke; k0 += 16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;          // 1024 elements of each 64x16 tile
      int mm, kk;
      if (sam == 1) { mm = e & 63; kk = e >> 6; } else { kk = e & 15; mm = e >> 4; }
      const int gm = m0 + mm, gk = k0 + kk;
      float av = 0.0f;
      if (gm < M && gk < ke) {
        if constexpr (sizeof(TA) == 2) av = bf2f(A[int64_t(gm) * sam + int64_t(gk) * sak]);
        else av = A[int64_t(gm) * sam + int64_t(gk) * sak];
      }
      As[kk][mm] = av;
      int nn, kk2;
      if (sbn == 1) { nn = e & 63; kk2 = e >> 6; } else { kk2 = e & 15; nn = e >> 4; }
      const int gn = n0 + nn, gk2 = k0 + kk2;
      Bs[kk2][nn] = (gn < N && gk2 < ke) ? B[int64_t(gk2) * sbk + int64_t(gn) * sbn] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* Pz = P + int64_t(blockIdx.z) * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + ty * 4 + i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx * 4 + j;
      if (gn < N) Pz[int64_t(gm) * N + gn] = acc[i][j];
    }
  }
}

// Noisy top-k: the logits are H = z + noise * softplus(zn), zn = x . W_noise, so
// dJ/dzn = dJ/dH * noise * sigmoid(zn).
__global__ void noise_grad_kernel(const float* __restrict__ dz, const float* __restrict__ noise,
                                  const float* __restrict__ zn, int64_t n, float* __restrict__ dzn) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  dzn[i] = dz[i] * noise[i] / (1.0f + expf(-zn[i]));
}

hipError_t launch_noise_grad(const float* dz, const float* noise, const float* zn, int64_t n,
                             float* dzn, hipStream_t st) {
  noise_grad_kernel<<<unsigned(cdiv(n, 256)), 256, 0, st>>>(dz, noise, zn, n, dzn);
  return hipGetLastError();
}

// out[i] = sum over z of P[z][i], z in order.
// Four consecutive elements per thread (16-byte loads when n is a multiple of
// 4), the loads of four partials in flight; each element still adds its
// partials in z order.  out may be P itself (each element is read before it
// is written, by the same thread).
__global__ void sum_partials_kernel(const float* P, int nz, int64_t n, float* out) {
  const int64_t i4 = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i4 >= n) return;
  if ((n & 3) == 0) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    int z = 0;
    for (; z + 4 <= nz; z += 4) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float4*>(P + int64_t(z + u) * n + i4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
      }
    }
    for (; z < nz; ++z) {
      const float4 v = *reinterpret_cast<const float4*>(P + int64_t(z) * n + i4);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    *reinterpret_cast<float4*>(out + i4) = s;
  } else {
    for (int64_t i = i4; i < i4 + 4 && i < n; ++i) {
      float s = 0.0f;
      for (int z = 0; z < nz; ++z) s += P[int64_t(z) * n + i];
      out[i] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// dx[t] = sum over kept slots j (slot order) of dXp[row_tj] + extra1[t] + extra2[t].
// One wave per token: as in the forward combine, each slot row is read through
// its own buffer descriptor (empty for a dropped slot), so the loads of all KM
// slots of a 256-float slab are issued together.
template <int KM>
__global__ __launch_bounds__(256) void unpermute_sum_kernel(
    const float* __restrict__ dxp, const int32_t* __restrict__ ros, const float* __restrict__ e1,
    const float* __restrict__ e2, int T, int k, int d, float* __restrict__ dx) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (t >= T) return;
  const int my_row = l < k ? ros[int64_t(t) * k + l] : -1;
  int rows[KM];
  rsrc_t rs[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    rows[j] = __builtin_amdgcn_readlane(my_row, j);
    rs[j] = make_rsrc(rows[j] >= 0 ? dxp + int64_t(rows[j]) * d : dxp,
                      rows[j] >= 0 ? uint32_t(d) * 4 : 0u);
  }
  for (int c = l; c < (d >> 2); c += 64) {
    floatx4 v[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      v[j] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs[j], uint32_t(c) * 16, 0, 0));
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (rows[j] < 0) continue;
      acc.x += v[j][0]; acc.y += v[j][1]; acc.z += v[j][2]; acc.w += v[j][3];
    }
    if (e1) {
      const float4 u = reinterpret_cast<const float4*>(e1 + int64_t(t) * d)[c];
      acc.x += u.x; acc.y += u.y; acc.z += u.z; acc.w += u.w;
    }
    if (e2) {
      const float4 u = reinterpret_cast<const float4*>(e2 + int64_t(t) * d)[c];
      acc.x += u.x; acc.y += u.y; acc.z += u.z; acc.w += u.w;
    }
    reinterpret_cast<float4*>(dx + int64_t(t) * d)[c] = acc;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_combine_bwd(const float* dy, const float* o, const int32_t* ros, const float* gate,
                              int T, int k, int d, bool bf16, void* dO, float* dg, void* dy_x,
                              hipStream_t st) {
  const dim3 grid(unsigned(cdiv(T, 4))), block(256);
#define MOE_CBWD(KM)                                                                           \
  (bf16 ? combine_bwd_kernel<true, KM><<<grid, block, 0, st>>>(dy, o, ros, gate, T, k, d, dO, dg, \
                                                             dy_x)                           \
        : combine_bwd_kernel<false, KM><<<grid, block, 0, st>>>(dy, o, ros, gate, T, k, d, dO, dg, \
                                                              dy_x))
  if (k <= 1) MOE_CBWD(1);
  else if (k <= 2) MOE_CBWD(2);
  else if (k <= 4) MOE_CBWD(4);
  else if (k <= 8) MOE_CBWD(8);
  else MOE_CBWD(16);
#undef MOE_CBWD
  return hipGetLastError();
}

hipError_t launch_router_bwd(const float* z, const int32_t* idx, const float* dg,
                             const int32_t* counts, int T, int E, int k, int score, int renorm,
                             float scale, float aux_coef, float z_coef, float* dz, hipStream_t st) {
  router_bwd_kernel<<<unsigned(cdiv(T, 4)), 256, 0, st>>>(z, idx, dg, counts, T, E, k, score,
                                                          renorm, scale, aux_coef, z_coef, dz);
  return hipGetLastError();
}

hipError_t launch_strided_gemm(const void* A, bool a_bf16, int64_t sam, int64_t sak, const float* B,
                               int64_t sbk, int64_t sbn, int M, int N, int K, int nsplit, float* P,
                               float* out, hipStream_t st) {
  const int kchunk = int(cdiv(cdiv(K, nsplit), 16) * 16);
  const dim3 grid(unsigned(cdiv(N, 64)), unsigned(cdiv(M, 64)), unsigned(nsplit));
  if (a_bf16)
    strided_gemm_kernel<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(A), sam, sak,
                                                        B, sbk, sbn, M, N, K, kchunk, P);
  else
    strided_gemm_kernel<float><<<grid, 256, 0, st>>>(static_cast<const float*>(A), sam, sak, B,
                                                     sbk, sbn, M, N, K, kchunk, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || out == nullptr) return e;
  const int64_t n = int64_t(M) * N;
  sum_partials_kernel<<<unsigned(cdiv(cdiv(n, 4), 256)), 256, 0, st>>>(P, nsplit, n, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router gradients on the bf16 matrix cores.  An fp32 value v splits exactly
// into three bf16 planes (hi = rne(v), mid = rne(v - hi), lo = rne(v - hi -
// mid); each residual is exact in fp32, so hi + mid + lo == v for normal v).
// With dz and Wg both split, dz . Wg^T is the sum of the six plane products
// p_i q_j with i + j <= 2 (the dropped ones are below 2^-24 relative), laid
// out as K' = 6E slots: dz slots [hi mid lo hi hi mid], Wg slots [hi hi hi mid
// lo mid].  The first three dz slots are also the B operand of dWg = x^T dz.
// One thread per (row, e) (grid.y = row): the split is computed once and
// written to the six slots; columns 6E .. KP-1 are zeroed.
__global__ void router_planes_kernel(const float* __restrict__ src, int E, int KP,
                                     uint32_t pattern, uint16_t* __restrict__ out) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = blockIdx.y;
  if (e >= E) return;
  const float x = src[r * E + e];
  const uint16_t hi = f2bf(x);
  const float r1 = x - bf2f(hi);
  const uint16_t mid = f2bf(r1);
  const uint16_t lo = f2bf(r1 - bf2f(mid));
  uint16_t* o = out + r * KP;
#pragma unroll
  for (int slot = 0; slot < 6; ++slot) {
    const int pl = int(pattern >> (4 * slot)) & 15;
    o[slot * E + e] = pl == 0 ? hi : (pl == 1 ? mid : lo);
  }
  for (int c = 6 * E + e; c < KP; c += E) o[c] = 0;
}

__global__ void dwg_reduce_kernel(const float* __restrict__ P, int nchunks, int D, int N3, int E,
                                  float* __restrict__ dWg) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(D) * E) return;
  const int dd = int(i / E), e = int(i % E);
  float acc = 0.0f;
  int c = 0;
  // four chunks' loads in flight; chunks still added in order
  for (; c + 4 <= nchunks; c += 4) {
    float v[4][3];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* p = P + (int64_t(c + u) * D + dd) * N3;
      v[u][0] = p[e];
      v[u][1] = p[E + e];
      v[u][2] = p[2 * E + e];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += (v[u][0] + v[u][1]) + v[u][2];
  }
  for (; c < nchunks; ++c) {
    const float* p = P + (int64_t(c) * D + dd) * N3;
    acc += (p[e] + p[E + e]) + p[2 * E + e];
  }
  dWg[i] = acc;
}

hipError_t launch_router_planes(const float* src, int64_t rows, int E, int KP, uint32_t pattern,
                                uint16_t* out, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  // rows beyond the grid's y limit are taken in slices
  for (int64_t r0 = 0; r0 < rows; r0 += 65535) {
    const unsigned ny = unsigned(std::min<int64_t>(65535, rows - r0));
    router_planes_kernel<<<dim3(unsigned(cdiv(E, 256)), ny), 256, 0, st>>>(
        src + r0 * E, E, KP, pattern, out + r0 * KP);
  }
  return hipGetLastError();
}

hipError_t launch_dwg_reduce(const float* P, int nchunks, int D, int N3, int E, float* dWg,
                             hipStream_t st) {
  const int64_t n = int64_t(D) * E;
  dwg_reduce_kernel<<<unsigned(cdiv(n, 256)), 256, 0, st>>>(P, nchunks, D, N3, E, dWg);
  return hipGetLastError();
}

hipError_t launch_sum_partials(const float* P, int nz, int64_t n, float* out, hipStream_t st) {
  sum_partials_kernel<<<unsigned(cdiv(cdiv(n, 4), 256)), 256, 0, st>>>(P, nz, n, out);
  return hipGetLastError();
}

hipError_t launch_unpermute_sum(const float* dxp, const int32_t* ros, const float* e1,
                                const float* e2, int T, int k, int d, float* dx, hipStream_t st) {
  const dim3 grid(unsigned(cdiv(T, 4))), block(256);
  if (k <= 1) unpermute_sum_kernel<1><<<grid, block, 0, st>>>(dxp, ros, e1, e2, T, k, d, dx);
  else if (k <= 2) unpermute_sum_kernel<2><<<grid, block, 0, st>>>(dxp, ros, e1, e2, T, k, d, dx);
  else if (k <= 4) unpermute_sum_kernel<4><<<grid, block, 0, st>>>(dxp, ros, e1, e2, T, k, d, dx);
  else if (k <= 8) unpermute_sum_kernel<8><<<grid, block, 0, st>>>(dxp, ros, e1, e2, T, k, d, dx);
  else unpermute_sum_kernel<16><<<grid, block, 0, st>>>(dxp, ros, e1, e2, T, k, d, dx);
  return hipGetLastError();
}

}  // namespace moe
