// Dispatch of the sparse MoE layer for gfx950: per-expert histogram, capacity
// clip and exclusive scan, and a stable (token-order) permutation of the kept
// slots into expert-contiguous rows with a coalesced copy of the token rows
// ("Mixture of Experts Explained", "MoEs and Transformers": expert capacity,
// overflow through the residual; "Switch Transformers": capacity factor).
//
// Determinism: the position of a slot inside its expert is its rank by token
// index, built from per-block counts (scanned in block order), per-wave counts
// (scanned in wave order) and a ballot/popcount rank inside the wave.  No
// global atomics decide any order.
//
// Slot priority (every token's first choice before any second choice, GShard's
// overflow order): the same kernels run over the T*k slots in slot-major order,
// as virtual tokens v = j*T + t with one slot each.  With k >= 4 token priority
// runs one slot per lane as well, in flat order v = t*k + j: a token's k
// experts are distinct, so within an expert this is token order and the ranks
// are the same, with k times more waves and at most 64 distinct experts per
// wave to peel.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int DISP_KMAX = 16;

// Per-block histogram of the slots' experts.  LDS atomics only count, so the
// result is order independent.  Entries outside [0, E) are skipped.
__global__ __launch_bounds__(1024) void dispatch_hist_kernel(const int32_t* __restrict__ idx, int T,
                                                            int k, int E, int order,
                                                            int32_t* __restrict__ blockcnt) {
  __shared__ int32_t hist[256];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * blockDim.x + threadIdx.x;    // blockDim.x = the order's block size
  if (order == DISP_FLAT) {
    if (int64_t(t) < int64_t(T) * k) {
      const int e = idx[t];
      if (unsigned(e) < unsigned(E)) atomicAdd(&hist[e], 1);
    }
  } else if (order == DISP_SLOT) {
    if (int64_t(t) < int64_t(T) * k) {
      const int e = idx[int64_t(t % T) * k + t / T];
      if (unsigned(e) < unsigned(E)) atomicAdd(&hist[e], 1);
    }
  } else if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[int64_t(t) * k + j];
      if (unsigned(e) < unsigned(E)) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) blockcnt[int64_t(blockIdx.x) * E + e] = hist[e];
}

// One block of 1024 threads: expert e's per-block counts are split into four
// quarters of the blocks (thread e + 256 q takes quarter q, 16 loads in flight
// per step), the quarters' sums give each quarter's base, and a second pass
// writes the exclusive scan over the blocks.  Then the totals, the kept counts
// min(total, C) and an exclusive scan over experts -> offsets.  C < 0: no
// capacity.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int32_t* __restrict__ blockcnt,
                                                             int nblk, int E, int64_t C,
                                                             int32_t* __restrict__ blockbase,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ n_dropped) {
  __shared__ int32_t qsum[4][256];
  __shared__ int32_t sk[256];
  __shared__ int32_t sd[256];
  const int tid = threadIdx.x, e = tid & 255, q = tid >> 8;
  const int nq = (nblk + 3) / 4;
  const int b0 = q * nq, b1 = min(nblk, b0 + nq);
  int32_t part = 0;
  if (e < E) {
    for (int b = b0; b < b1; b += 16) {
      int32_t c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = b + i < b1 ? blockcnt[int64_t(b + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) part += c[i];
    }
  }
  qsum[q][e] = part;
  __syncthreads();
  int32_t run = 0, total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    run += i < q ? qsum[i][e] : 0;
    total += qsum[i][e];
  }
  if (e < E) {
    for (int b = b0; b < b1; b += 16) {
      int32_t c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = b + i < b1 ? blockcnt[int64_t(b + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (b + i < b1) blockbase[int64_t(b + i) * E + e] = run;
        run += c[i];
      }
    }
    if (q == 0 && counts) counts[e] = total;
  }
  const int32_t kept = (e < E) ? ((C >= 0 && int64_t(total) > C) ? int32_t(C) : total) : 0;
  if (q == 0) {
    sk[e] = kept;
    sd[e] = (e < E) ? total - kept : 0;
  }
  __syncthreads();
  // Hillis-Steele inclusive scan of kept counts and drop counts (threads 0..255).
  for (int st = 1; st < 256; st <<= 1) {
    const int32_t vk = (q == 0 && e >= st) ? sk[e - st] : 0;
    const int32_t vd = (q == 0 && e >= st) ? sd[e - st] : 0;
    __syncthreads();
    if (q == 0) {
      sk[e] += vk;
      sd[e] += vd;
    }
    __syncthreads();
  }
  if (q == 0 && e < E) offsets[e] = sk[e] - kept;
  if (tid == 0) {
    offsets[E] = sk[255];
    if (n_dropped) n_dropped[0] = sd[255];
  }
}

// Stable ranks and the row copy.  Block b covers the NT tokens (or slots)
// from b*NT, wave w the 64 from b*NT + 64w, one per lane.
//   1. peel: repeatedly take the expert of the first lane with a pending slot,
//      ballot the lanes holding that expert, rank = popcount of lower lanes;
//      the leader records the wave's count for the expert;
//   2. rank in expert = blockbase[b][e] + counts of lower waves + rank in wave;
//      kept iff rank < C; row = offsets[e] + rank;
// The row copy is a separate, token-parallel kernel (permute_copy_kernel).
// ORDER DISP_SLOT: the block's "tokens" are the slot-major virtual tokens
// v = j*T + t (KM = 1), slot (v % T, v / T); DISP_FLAT: flat slots v = t*k + j
// (KM = 1), token v / k.
template <int KM, int ORDER, int NT = 256>
__global__ __launch_bounds__(NT) void dispatch_rank_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int64_t C,
    const int32_t* __restrict__ blockbase, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_of_slot, int32_t* __restrict__ token_of_row) {
  __shared__ int32_t wavecnt[NT / 64][256];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  for (int i = tid; i < (NT / 64) * 256; i += NT) (&wavecnt[0][0])[i] = 0;
  const int v = blockIdx.x * NT + tid;
  constexpr bool ONE = ORDER != DISP_TOKEN;                     // one slot per lane
  const bool valid = ONE ? int64_t(v) < int64_t(T) * k : v < T;
  const int t = ORDER == DISP_SLOT ? (valid ? v % T : 0)       // token of this lane's slots
              : ORDER == DISP_FLAT ? (valid ? v / k : 0) : v;
  const int64_t slot0 = ORDER == DISP_SLOT ? int64_t(t) * k + (valid ? v / T : 0)
                      : ORDER == DISP_FLAT ? (valid ? int64_t(v) : 0) : int64_t(t) * k;
  const int kk = ONE ? 1 : k;                                   // slots per lane
  int ex[KM];
  int rk[KM];
  uint32_t pending = 0;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    ex[j] = -1;
    rk[j] = 0;
    if (valid && j < kk) {
      const int e = idx[slot0 + j];
      if (unsigned(e) < unsigned(E)) {
        ex[j] = e;
        pending |= 1u << j;
      }
    }
  }
  __syncthreads();
  const uint64_t lt_mask = (l == 0) ? 0ull : (~0ull >> (64 - l));
  while (true) {
    const uint64_t act = __ballot(pending != 0);
    if (act == 0) break;
    const int leader = __ffsll(static_cast<unsigned long long>(act)) - 1;
    int mine = -1;
    if (pending) {
      const int j0 = __ffs(pending) - 1;
#pragma unroll
      for (int j = 0; j < KM; ++j)
        if (j == j0) mine = ex[j];
    }
    const int e = __shfl(mine, leader, 64);
    int jm = -1;
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if ((pending >> j & 1u) && ex[j] == e) jm = j;
    const uint64_t m = __ballot(jm >= 0);
    if (jm >= 0) {
      const int r = __popcll(m & lt_mask);
#pragma unroll
      for (int j = 0; j < KM; ++j)
        if (j == jm) rk[j] = r;
      pending &= ~(1u << jm);
    }
    if (l == leader) wavecnt[w][e] = __popcll(m);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < kk) {
      int row = -1;
      const int e = ex[j];
      if (e >= 0) {
        int32_t rank = blockbase[int64_t(blockIdx.x) * E + e] + rk[j];
        for (int ww = 0; ww < w; ++ww) rank += wavecnt[ww][e];
        if (C < 0 || rank < C) {
          row = offsets[e] + rank;
          token_of_row[row] = t;
        }
      }
      if (valid) row_of_slot[slot0 + j] = row;
    }
  }
}

// Row copy, token-major, one wave per token: the token's x row is read once
// (16-byte lanes) and written to each of its kept rows.
template <int KM>
__global__ __launch_bounds__(256) void permute_copy_kernel(const int32_t* __restrict__ row_of_slot,
                                                           int T, int k,
                                                           const uint8_t* __restrict__ x,
                                                           int row_bytes,
                                                           uint8_t* __restrict__ x_perm) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (t >= T) return;
  int rows[KM];
  bool any = false;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    rows[j] = j < k ? row_of_slot[int64_t(t) * k + j] : -1;
    any = any || rows[j] >= 0;
  }
  if (!any) return;
  const uint8_t* src = x + int64_t(t) * row_bytes;
  const int chunks = row_bytes >> 4;
  for (int c = l; c < chunks; c += 64) {
    const uint4 v = ld16(src + 16 * c);
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (rows[j] >= 0) st16(x_perm + int64_t(rows[j]) * row_bytes + 16 * c, v);
  }
}

int dispatch_order(int k, bool slot_major) {
  return slot_major ? DISP_SLOT : (k >= 4 ? DISP_FLAT : DISP_TOKEN);
}

// Slots (or tokens) per dispatch block: 1024 in flat order (16 waves; fewer
// blocks keep the single-workgroup scan over the blocks short), else 256.
int dispatch_block_size(int order) { return order == DISP_FLAT ? 1024 : DISP_TB; }

int dispatch_blocks(int T, int k, bool slot_major) {
  const int order = dispatch_order(k, slot_major);
  return int(cdiv(order != DISP_TOKEN ? int64_t(T) * k : int64_t(T), dispatch_block_size(order)));
}

hipError_t launch_dispatch_hist(const int32_t* idx, int T, int k, int E, bool slot_major,
                                int32_t* blockcnt, hipStream_t st) {
  const unsigned nblk = unsigned(dispatch_blocks(T, k, slot_major));
  const int order = dispatch_order(k, slot_major);
  dispatch_hist_kernel<<<dim3(nblk), dim3(dispatch_block_size(order)), 0, st>>>(idx, T, k, E, order,
                                                                               blockcnt);
  return hipGetLastError();
}

hipError_t launch_dispatch_scan(const int32_t* blockcnt, int nblk, int E, int64_t C,
                                int32_t* blockbase, int32_t* counts, int32_t* offsets,
                                int32_t* n_dropped, hipStream_t st) {
  dispatch_scan_kernel<<<dim3(1), dim3(1024), 0, st>>>(blockcnt, nblk, E, C, blockbase, counts,
                                                       offsets, n_dropped);
  return hipGetLastError();
}

hipError_t launch_dispatch_permute(const int32_t* idx, int T, int k, int E, int64_t C,
                                   bool slot_major, const int32_t* blockbase,
                                   const int32_t* offsets, const void* x, int d, int elem_bytes,
                                   int32_t* row_of_slot, int32_t* token_of_row, void* x_perm,
                                   hipStream_t st) {
  const unsigned nblk = unsigned(dispatch_blocks(T, k, slot_major));
  const unsigned ncopy = unsigned(cdiv(T, 4));
  const int row_bytes = d * elem_bytes;
  const auto* xs = static_cast<const uint8_t*>(x);
  auto* xp = static_cast<uint8_t*>(x_perm);
#define MOE_PERMUTE(KM)                                                                        \
  dispatch_rank_kernel<KM, DISP_TOKEN><<<dim3(nblk), dim3(256), 0, st>>>(                      \
      idx, T, k, E, C, blockbase, offsets, row_of_slot, token_of_row);                         \
  permute_copy_kernel<KM><<<dim3(ncopy), dim3(256), 0, st>>>(row_of_slot, T, k, xs, row_bytes, xp)
  const int order = dispatch_order(k, slot_major);
  if (order != DISP_TOKEN) {
    if (order == DISP_SLOT)
      dispatch_rank_kernel<1, DISP_SLOT><<<dim3(nblk), dim3(256), 0, st>>>(
          idx, T, k, E, C, blockbase, offsets, row_of_slot, token_of_row);
    else
      dispatch_rank_kernel<1, DISP_FLAT, 1024><<<dim3(nblk), dim3(1024), 0, st>>>(
          idx, T, k, E, C, blockbase, offsets, row_of_slot, token_of_row);
    if (k <= 2) permute_copy_kernel<2><<<dim3(ncopy), dim3(256), 0, st>>>(row_of_slot, T, k, xs, row_bytes, xp);
    else if (k <= 4) permute_copy_kernel<4><<<dim3(ncopy), dim3(256), 0, st>>>(row_of_slot, T, k, xs, row_bytes, xp);
    else if (k <= 8) permute_copy_kernel<8><<<dim3(ncopy), dim3(256), 0, st>>>(row_of_slot, T, k, xs, row_bytes, xp);
    else permute_copy_kernel<16><<<dim3(ncopy), dim3(256), 0, st>>>(row_of_slot, T, k, xs, row_bytes, xp);
  } else if (k <= 1) { MOE_PERMUTE(1); }
  else if (k <= 2) { MOE_PERMUTE(2); }
  else if (k <= 4) { MOE_PERMUTE(4); }
  else if (k <= 8) { MOE_PERMUTE(8); }
  else { MOE_PERMUTE(16); }
#undef MOE_PERMUTE
  return hipGetLastError();
}

}  // namespace moe
