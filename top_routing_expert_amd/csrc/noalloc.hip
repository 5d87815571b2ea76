// moe_permute_noalloc: the dispatch step (moe_permute) for callers that cannot
// allocate device memory or pass a workspace (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The dispatch kernels' only scratch is one per-block table, the expert
// histogram of each block of 1024 slots (ceil(T*k/1024) * E int32).  Here it
// lives in one file-scope device array of NOALLOC_SCRATCH_BYTES bytes.  Every
// GPU holds its own copy at its own address; the address is fetched once per
// device with hipGetSymbolAddress and only that address is handed to kernels.
// The table is written in full before it is read, so nothing needs clearing
// between calls.  Calls that overlap on one GPU (on different streams) share
// the array and race.
#include <mutex>

#include "../../include/moe.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace moe;

constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(1) << 20;   // 1 MiB per device
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

// Device address of this GPU's copy of `scratch` (looked up on the first call
// on each device, with that device current).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int moe_permute_noalloc(const moe_dims* d, const moe_opts* o, const void* x,
                                   const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                                   int32_t* row_of_slot, int32_t* token_of_row, void* x_perm,
                                   void* stream) {
  size_t unused = 0;
  int s = moe_workspace_size(d, o, 0, &unused);   // validates dims and opts
  if (s) return s;
  if (!x || !topk_idx || !offsets || !row_of_slot || !token_of_row || !x_perm)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
  const bool slot_major = o->priority == MOE_PRIORITY_SLOT;
  const int T = int(d->T), k = int(d->k), E = int(d->E);
  const int nblk = dispatch_blocks(T, k, slot_major);
  const size_t table = round256(size_t(nblk) * size_t(E) * 4);
  if (table > NOALLOC_SCRATCH_BYTES) return MOE_ERR_UNSUPPORTED;
  int64_t C = -1;
  if ((s = moe_capacity(d, o, &C))) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (d->T == 0) return launch_zero_i32(offsets, d->E + 1, st) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  void* base = nullptr;
  if (scratch_address(&base) != hipSuccess) return MOE_ERR_HIP;
  int32_t* blockcnt = static_cast<int32_t*>(base);
  if (launch_dispatch_hist(topk_idx, T, k, E, slot_major, blockcnt, st) != hipSuccess ||
      launch_dispatch_permute(topk_idx, T, k, E, C, slot_major, blockcnt, counts, offsets,
                              nullptr, x, int(d->d), o->dtype == MOE_DTYPE_BF16 ? 2 : 4,
                              row_of_slot, token_of_row, x_perm, st) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}
