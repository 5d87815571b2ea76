// Load balancing from score histograms and router monitoring, for gfx950.
//
//  * Quantile balancing (Ultimate MoE Training Handbook news, Kimi K3: the
//    selection bias solved from per-expert score histograms summed over GPUs,
//    instead of fixed steps).  score_hist_kernel builds the fixed-size summary
//    (integer counts, so the result does not depend on the order of the
//    atomic adds); bias_solve_kernel reads, for each expert, the score above
//    which the target number of its tokens lie and centres the biases.
//  * Monitoring (handbook explainer, "router and load balancing": max expert
//    load, drop rate, spread of utilisation; handbook digest: the largest
//    expert output norm against the median).  expert_norm_kernel sums the
//    row L2 norms of each expert's outputs in a fixed order; report_kernel
//    reduces the per-expert figures in one block.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// hist[e][bin(s[t,e])] += 1, bin = floor((s - lo) * scale) clamped to
// [0, nbins-1]; NaN scores are skipped.  One thread per (token, expert) entry.
__global__ __launch_bounds__(256) void score_hist_kernel(const float* __restrict__ s, int64_t n,
                                                         int E, float lo, float scale, int nbins,
                                                         int32_t* __restrict__ hist) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float b = floorf((s[i] - lo) * scale);
  if (b != b) return;
  const int bin = b < 0.0f ? 0 : (b >= float(nbins - 1) ? nbins - 1 : int(b));
  const int e = int(i % E);
  atomicAdd(&hist[int64_t(e) * nbins + bin], 1);
}

// One block, thread e < E: walk expert e's bins from the top until the count
// reaches target; q_e = lo + (i + 1 - (target - c) / h) * w within that bin,
// lo if the expert has fewer tokens.  bias_e = mean(q) - q_e (mean summed in
// expert order).
__global__ __launch_bounds__(256) void bias_solve_kernel(const int32_t* __restrict__ hist, int E,
                                                         int nbins, float lo, float w,
                                                         float target, float* __restrict__ bias) {
  __shared__ float qs[256];
  __shared__ float mean_s;
  const int e = threadIdx.x;
  float q = lo;
  if (e < E) {
    int64_t c = 0;
    for (int i = nbins - 1; i >= 0; --i) {
      const int32_t h = hist[int64_t(e) * nbins + i];
      if (h > 0 && float(c + h) >= target) {
        q = lo + (float(i + 1) - (target - float(c)) / float(h)) * w;
        break;
      }
      c += h;
    }
  }
  qs[e] = q;
  __syncthreads();
  if (e == 0) {
    double m = 0.0;
    for (int j = 0; j < E; ++j) m += double(qs[j]);
    mean_s = float(m / E);
  }
  __syncthreads();
  if (e < E) bias[e] = mean_s - q;
}

// One block per expert: norm[e] = mean over its rows of ||o_row||_2 (0 when it
// has none).  Wave w takes rows w, w+4, ...; each lane accumulates its share
// of the row sums in row order; the four waves' sums are combined in order.
__global__ __launch_bounds__(256) void expert_norm_kernel(const float* __restrict__ o, int d,
                                                          const int32_t* __restrict__ offsets,
                                                          float* __restrict__ norm) {
  __shared__ double ws_sum[4];
  const int e = blockIdx.x;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  double acc = 0.0;
  for (int r = r0 + w; r < r1; r += 4) {
    const float* row = o + int64_t(r) * d;
    float ss = 0.0f;
    for (int c = l; c < d; c += 64) ss = fmaf(row[c], row[c], ss);
    ss = group_sum<64>(ss);
    acc += double(sqrtf(ss));
  }
  if (l == 0) ws_sum[w] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double tot = ws_sum[0] + ws_sum[1] + ws_sum[2] + ws_sum[3];
    norm[e] = r1 > r0 ? float(tot / double(r1 - r0)) : 0.0f;
  }
}

// One block: report = {max/mean load, CV of the loads, dropped/routed,
// max/median expert output norm over non-empty experts, empty experts}.
__global__ __launch_bounds__(256) void report_kernel(const int32_t* __restrict__ counts, int E,
                                                     const int32_t* __restrict__ n_dropped,
                                                     const float* __restrict__ norm,
                                                     float* __restrict__ report) {
  __shared__ double c[256];
  __shared__ float nv[256];
  __shared__ int ne[256];
  const int e = threadIdx.x;
  c[e] = e < E ? double(counts[e]) : 0.0;
  ne[e] = (e < E && counts[e] > 0) ? 1 : 0;
  nv[e] = (norm && e < E) ? norm[e] : 0.0f;
  __syncthreads();
  // median of the non-empty experts' norms: the element(s) of rank (m-1)/2 and
  // m/2 in (value, index) order
  float lo_v = 0.0f, hi_v = 0.0f;
  __shared__ float med[2];
  __shared__ int m_s;
  if (e == 0) {
    int m = 0;
    for (int j = 0; j < E; ++j) m += ne[j];
    m_s = m;
  }
  __syncthreads();
  const int m = m_s;
  if (norm && e < E && ne[e]) {
    int rank = 0;
    for (int j = 0; j < E; ++j)
      if (ne[j] && (nv[j] < nv[e] || (nv[j] == nv[e] && j < e))) ++rank;
    if (rank == (m - 1) / 2) med[0] = nv[e];
    if (rank == m / 2) med[1] = nv[e];
  }
  __syncthreads();
  if (e == 0) {
    double sum = 0.0, mx = 0.0;
    int empty = 0;
    float nmax = 0.0f;
    for (int j = 0; j < E; ++j) {
      sum += c[j];
      mx = c[j] > mx ? c[j] : mx;
      empty += c[j] == 0.0 ? 1 : 0;
      if (ne[j] && nv[j] > nmax) nmax = nv[j];
    }
    const double mean = sum / E;
    double var = 0.0;
    for (int j = 0; j < E; ++j) var += (c[j] - mean) * (c[j] - mean);
    var /= E;
    lo_v = med[0];
    hi_v = med[1];
    const double median = m > 0 ? 0.5 * (double(lo_v) + double(hi_v)) : 0.0;
    report[0] = mean > 0.0 ? float(mx / mean) : 0.0f;
    report[1] = mean > 0.0 ? float(sqrt(var) / mean) : 0.0f;
    report[2] = (n_dropped && sum > 0.0) ? float(double(n_dropped[0]) / sum) : 0.0f;
    report[3] = (norm && m > 0 && median > 0.0) ? float(double(nmax) / median) : 0.0f;
    report[4] = float(empty);
  }
}

hipError_t launch_score_hist(const float* s, int64_t T, int E, float lo, float hi, int nbins,
                             int32_t* hist, hipStream_t st) {
  hipError_t e = launch_zero_i32(hist, int64_t(E) * nbins, st);
  if (e != hipSuccess) return e;
  const int64_t n = T * E;
  if (n == 0) return hipSuccess;
  const float scale = float(nbins) / (hi - lo);
  score_hist_kernel<<<unsigned(cdiv(n, 256)), 256, 0, st>>>(s, n, E, lo, scale, nbins, hist);
  return hipGetLastError();
}

hipError_t launch_bias_solve(const int32_t* hist, int E, int nbins, float lo, float hi, float target,
                             float* bias, hipStream_t st) {
  bias_solve_kernel<<<1, 256, 0, st>>>(hist, E, nbins, lo, (hi - lo) / float(nbins), target, bias);
  return hipGetLastError();
}

hipError_t launch_router_report(int E, int d, const int32_t* counts, const int32_t* n_dropped,
                                const float* o, const int32_t* offsets, float* norm, float* report,
                                hipStream_t st) {
  if (o) {
    expert_norm_kernel<<<unsigned(E), 256, 0, st>>>(o, d, offsets, norm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  report_kernel<<<1, 256, 0, st>>>(counts, E, n_dropped, o ? norm : nullptr, report);
  return hipGetLastError();
}

}  // namespace moe
