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
// Every kernel walks the T*k slots one per lane.  Token priority takes them in
// flat order v = t*k + j, which inside an expert is ascending token order (and
// slot order within a token, so a token that lists one expert twice keeps both
// slots, in slot order).  Slot priority (every token's first choice before any
// second choice, GShard's overflow order) takes them slot-major, v = j*T + t.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Per-block histogram of the slots' experts.  LDS atomics only count, so the
// result is order independent.  Entries outside [0, E) are skipped.
__global__ __launch_bounds__(1024) void dispatch_hist_kernel(const int32_t* __restrict__ idx, int T,
                                                            int k, int E, int order,
                                                            int32_t* __restrict__ blockcnt) {
  __shared__ int32_t hist[256];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (int64_t(v) < int64_t(T) * k) {
    const int e = order == DISP_SLOT ? idx[int64_t(v % T) * k + v / T] : idx[v];
    if (unsigned(e) < unsigned(E)) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) blockcnt[int64_t(blockIdx.x) * E + e] = hist[e];
}

// Stable ranks.  Block b covers the NT slots from b*NT in the order's sequence,
// wave w the 64 from b*NT + 64w, one per lane.
//   0. bases: from the per-block counts every block computes, for each expert,
//      the count in the blocks before it (its base) and in all blocks (the
//      total), then kept = min(total, C) and an exclusive scan over experts
//      (the rows' offsets).  Expert e's blocks are split into four quarters
//      (thread e + 256 q takes quarter q, 16 loads in flight per step) summed
//      in a fixed order.  Block 0 also writes the counts, offsets and drops.
//   1. peel: repeatedly take the expert of the first lane still pending,
//      ballot the lanes holding that expert, rank = popcount of lower lanes;
//      the leader records the wave's count for the expert;
//   2. rank in expert = base[e] + counts of lower waves + rank in wave;
//      kept iff rank < C; row = offsets[e] + rank.
// The row copy is a separate, token-parallel kernel (permute_copy_kernel).
template <int ORDER, int NT>
__global__ __launch_bounds__(NT) void dispatch_rank_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int64_t C, int nblk,
    const int32_t* __restrict__ blockcnt, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ n_dropped,
    int32_t* __restrict__ row_of_slot, int32_t* __restrict__ token_of_row) {
  static_assert(NT == 1024, "four quarters of 256 expert lanes");
  __shared__ int32_t wavecnt[NT / 64][256];
  __shared__ int32_t qsum[2][4][256];
  __shared__ int32_t sbase[256], soff[256], sk[256], sd[256];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  for (int i = tid; i < (NT / 64) * 256; i += NT) (&wavecnt[0][0])[i] = 0;
  {
    const int e = tid & 255, q = tid >> 8;
    const int nq = (nblk + 3) / 4;
    const int b0 = q * nq, b1 = min(nblk, b0 + nq), bl = min(b1, int(blockIdx.x));
    int32_t before = 0, part = 0;
    if (e < E) {
      for (int b = b0; b < b1; b += 16) {
        int32_t c[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) c[i] = b + i < b1 ? blockcnt[int64_t(b + i) * E + e] : 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          part += c[i];
          before += b + i < bl ? c[i] : 0;
        }
      }
    }
    qsum[0][q][e] = before;
    qsum[1][q][e] = part;
    __syncthreads();
    if (q == 0) {
      int32_t base = 0, total = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        base += qsum[0][i][e];
        total += qsum[1][i][e];
      }
      const int32_t kept = (e < E) ? ((C >= 0 && int64_t(total) > C) ? int32_t(C) : total) : 0;
      sbase[e] = base;
      sk[e] = kept;
      sd[e] = (e < E) ? total - kept : 0;
      if (blockIdx.x == 0 && e < E && counts) counts[e] = total;
      soff[e] = kept;
    }
    __syncthreads();
    // Hillis-Steele inclusive scan of kept counts and drop counts
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
    if (q == 0) {
      soff[e] = sk[e] - soff[e];   // exclusive: the rows of the experts before e
      if (blockIdx.x == 0 && e < E) offsets[e] = soff[e];
    }
    if (blockIdx.x == 0) {
      if (tid == 0) {
        offsets[E] = sk[255];
        if (n_dropped) n_dropped[0] = sd[255];
      }
    }
  }
  const int v = blockIdx.x * NT + tid;
  const bool valid = int64_t(v) < int64_t(T) * k;
  const int t = !valid ? 0 : (ORDER == DISP_SLOT ? v % T : v / k);      // token of this slot
  const int64_t slot = !valid ? 0 : (ORDER == DISP_SLOT ? int64_t(t) * k + v / T : int64_t(v));
  int ex = -1;
  if (valid) {
    const int e = idx[slot];
    if (unsigned(e) < unsigned(E)) ex = e;
  }
  __syncthreads();
  const uint64_t lt_mask = (l == 0) ? 0ull : (~0ull >> (64 - l));
  bool pending = ex >= 0;
  int rk = 0;
  while (true) {
    const uint64_t act = __ballot(pending);
    if (act == 0) break;
    const int leader = __ffsll(static_cast<unsigned long long>(act)) - 1;
    const int e = __shfl(ex, leader, 64);
    const bool mine = pending && ex == e;
    const uint64_t m = __ballot(mine);
    if (mine) {
      rk = __popcll(m & lt_mask);
      pending = false;
    }
    if (l == leader) wavecnt[w][e] = __popcll(m);
  }
  __syncthreads();
  int row = -1;
  if (ex >= 0) {
    int32_t rank = sbase[ex] + rk;
    for (int ww = 0; ww < w; ++ww) rank += wavecnt[ww][ex];
    if (C < 0 || rank < C) {
      row = soff[ex] + rank;
      token_of_row[row] = t;
    }
  }
  if (valid) row_of_slot[slot] = row;
}

// Row copy, token-major, one wave per token: the token's x row is read once
// (16-byte lanes, four per lane in flight) and written to each of its kept
// rows with non-temporal stores.  The copy is almost all writes (k rows per
// row read); streaming them past the caches' normal retention, with four
// loads issued before any store, took the copy of 16384 tokens x 8 slots of
// 4 KB rows from 0.45 to 0.6 of the HBM roofline.
typedef unsigned uintx4 __attribute__((ext_vector_type(4)));
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
  for (int c0 = l; c0 < chunks; c0 += 256) {
    uintx4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (c0 + 64 * u < chunks) v[u] = __builtin_bit_cast(uintx4, ld16(src + 16 * (c0 + 64 * u)));
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (rows[j] >= 0)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (c0 + 64 * u < chunks)
            __builtin_nontemporal_store(
                v[u], reinterpret_cast<uintx4*>(x_perm + int64_t(rows[j]) * row_bytes + 16 * (c0 + 64 * u)));
  }
}

int dispatch_order(bool slot_major) { return slot_major ? DISP_SLOT : DISP_FLAT; }

// Slots per dispatch block (16 waves; fewer blocks keep each block's scan over
// the per-block counts short).
constexpr int DISP_NT = 1024;

int dispatch_blocks(int T, int k, bool) { return int(cdiv(int64_t(T) * k, DISP_NT)); }

hipError_t launch_dispatch_hist(const int32_t* idx, int T, int k, int E, bool slot_major,
                                int32_t* blockcnt, hipStream_t st) {
  const unsigned nblk = unsigned(dispatch_blocks(T, k, slot_major));
  dispatch_hist_kernel<<<dim3(nblk), dim3(DISP_NT), 0, st>>>(idx, T, k, E, dispatch_order(slot_major),
                                                             blockcnt);
  return hipGetLastError();
}

hipError_t launch_dispatch_permute(const int32_t* idx, int T, int k, int E, int64_t C,
                                   bool slot_major, const int32_t* blockcnt, int32_t* counts,
                                   int32_t* offsets, int32_t* n_dropped, const void* x, int d,
                                   int elem_bytes, int32_t* row_of_slot, int32_t* token_of_row,
                                   void* x_perm, hipStream_t st) {
  const unsigned nblk = unsigned(dispatch_blocks(T, k, slot_major));
  const unsigned ncopy = unsigned(cdiv(T, 4));
  const int row_bytes = d * elem_bytes;
  const auto* xs = static_cast<const uint8_t*>(x);
  auto* xp = static_cast<uint8_t*>(x_perm);
  if (slot_major)
    dispatch_rank_kernel<DISP_SLOT, DISP_NT><<<dim3(nblk), dim3(DISP_NT), 0, st>>>(
        idx, T, k, E, C, int(nblk), blockcnt, counts, offsets, n_dropped, row_of_slot,
        token_of_row);
  else
    dispatch_rank_kernel<DISP_FLAT, DISP_NT><<<dim3(nblk), dim3(DISP_NT), 0, st>>>(
        idx, T, k, E, C, int(nblk), blockcnt, counts, offsets, n_dropped, row_of_slot,
        token_of_row);
  if (k <= 1) permute_copy_kernel<1><<<dim3(ncopy), dim3(256), 0, st>>>(row_of_slot, T, k, xs, row_bytes, xp);
  else if (k <= 2) permute_copy_kernel<2><<<dim3(ncopy), dim3(256), 0, st>>>(row_of_slot, T, k, xs, row_bytes, xp);
  else if (k <= 4) permute_copy_kernel<4><<<dim3(ncopy), dim3(256), 0, st>>>(row_of_slot, T, k, xs, row_bytes, xp);
  else if (k <= 8) permute_copy_kernel<8><<<dim3(ncopy), dim3(256), 0, st>>>(row_of_slot, T, k, xs, row_bytes, xp);
  else permute_copy_kernel<16><<<dim3(ncopy), dim3(256), 0, st>>>(row_of_slot, T, k, xs, row_bytes, xp);
  return hipGetLastError();
}

}  // namespace moe
