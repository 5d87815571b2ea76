// C ABI of the sparse MoE layer: argument validation, workspace carving and
// the launch sequence of each entry point on the caller's stream.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/moe.h"
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>
#include <mutex>
#include <vector>

using namespace moe;

namespace {

constexpr size_t ALIGN = 256;

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += (bytes + ALIGN - 1) / ALIGN * ALIGN;
    return o;
  }
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(const moe_opts* o) { return o->dtype == MOE_DTYPE_BF16 ? 2 : 4; }
// The routed experts' activation as a bf16 (hi, lo) pair: 2F columns per row.
bool act_pair(const moe_opts* o) { return o->act_pair && o->dtype == MOE_DTYPE_BF16; }
int64_t act_cols(const moe_opts* o, int64_t F) { return act_pair(o) ? 2 * F : F; }
int64_t n_up(const moe_opts* o, int64_t F) { return o->act == MOE_ACT_SWIGLU ? 2 * F : F; }

int check_width(const moe_opts* o, int64_t v) {
  if (v < 1) return MOE_ERR_INVALID_ARG;
  if (o->dtype == MOE_DTYPE_BF16 ? (v % 128) != 0 : (v % 4) != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_dims(const moe_dims* d, const moe_opts* o) {
  if (!d || !o) return MOE_ERR_INVALID_ARG;
  if (o->dtype != MOE_DTYPE_F32 && o->dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (o->score < MOE_SCORE_SOFTMAX || o->score > MOE_SCORE_SQRT_SOFTPLUS) return MOE_ERR_INVALID_ARG;
  if (o->routing < MOE_ROUTING_TOPK || o->routing > MOE_ROUTING_HASH) return MOE_ERR_INVALID_ARG;
  if (o->priority != MOE_PRIORITY_TOKEN && o->priority != MOE_PRIORITY_SLOT) return MOE_ERR_INVALID_ARG;
  if (o->routing == MOE_ROUTING_RANDOM_SECOND && d && d->k != 2) return MOE_ERR_INVALID_ARG;
  if (o->act != MOE_ACT_SWIGLU && o->act != MOE_ACT_GELU) return MOE_ERR_INVALID_ARG;
  if (o->act_pair != 0 && o->act_pair != 1) return MOE_ERR_INVALID_ARG;
  if (d->T < 0 || d->E < 1 || d->k < 1 || d->k > d->E || d->F_shared < 0) return MOE_ERR_INVALID_ARG;
  if (!isfinite(o->gate_scale) || !isfinite(o->capacity_factor) || !isfinite(o->aux_coef) ||
      !isfinite(o->z_coef))
    return MOE_ERR_INVALID_ARG;
  if (d->E > 256 || d->k > 16) return MOE_ERR_UNSUPPORTED;
  if (d->T * d->k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  int s = check_width(o, d->d);
  if (s) return s;
  if ((s = check_width(o, d->F))) return s;
  if (d->F_shared > 0 && (s = check_width(o, d->F_shared))) return s;
  return MOE_OK;
}

int64_t capacity_of(const moe_dims* d, const moe_opts* o) {
  const double cf = double(o->capacity_factor);
  if (!(cf > 0.0)) return -1;
  return int64_t(ceil(cf * double(d->T) * double(d->k) / double(d->E)));
}

// bf16 tokens: the wide router kernel (64 tokens per block, logits on chip,
// one fp32 accumulation over the three planes of Wg).  Its 8 waves split d
// into 256 / EP ranges of whole 64-k chunks.
bool route_wide(const moe_dims* d, const moe_opts* o, int EP) {
  return o->dtype == MOE_DTYPE_BF16 && d->d % (64 * (256 / EP)) == 0;
}

// The variant routers' inputs that opts->routing needs must be present.
int check_router_inputs(const moe_opts* o, const moe_router_inputs* ri) {
  switch (o->routing) {
    case MOE_ROUTING_NOISY_TOPK:
      return ri && ri->W_noise && ri->noise ? MOE_OK : MOE_ERR_INVALID_ARG;
    case MOE_ROUTING_RANDOM_SECOND:
      return ri && ri->uniform ? MOE_OK : MOE_ERR_INVALID_ARG;
    case MOE_ROUTING_HASH:
      return ri && ri->token_ids ? MOE_OK : MOE_ERR_INVALID_ARG;
    default:
      return MOE_OK;
  }
}

// ---- workspace plans -------------------------------------------------------
// 17 to 32 experts: the wide kernel reads Wg [d, E] as stored (no layout pass).
bool route_wg_direct(int E) { return E > 16 && E <= 32; }

struct RouteWs {
  size_t wfrag, part_p, part_cnt, part_lse2, part_nf, zn;
  int nblk, EP;
  bool wide;
};
RouteWs plan_route(Carver& c, const moe_dims* d, const moe_opts* o) {
  RouteWs r;
  r.EP = route_pad_experts(int(d->E));
  r.wide = route_wide(d, o, r.EP);
  r.nblk = int(cdiv(d->T, r.wide ? route_wide_bt(d->T, r.EP) : ROUTE_BT));
  r.wfrag = c.take(r.wide && !route_wg_direct(int(d->E)) ? size_t(r.EP) * d->d * 4 : 0);
  r.part_p = c.take(size_t(r.nblk) * r.EP * 4);
  r.part_cnt = c.take(size_t(r.nblk) * r.EP * 4);
  r.part_lse2 = c.take(size_t(r.nblk) * 4);
  r.part_nf = c.take(size_t(r.nblk) * 4);
  r.zn = c.take(o->routing == MOE_ROUTING_NOISY_TOPK ? size_t(d->T) * d->E * 4 : 0);
  return r;
}

struct PermWs { size_t blockcnt; int nblk; };
PermWs plan_perm(Carver& c, const moe_dims* d, const moe_opts* o) {
  PermWs p;
  p.nblk = dispatch_blocks(int(d->T), int(d->k), o->priority == MOE_PRIORITY_SLOT);
  p.blockcnt = c.take(size_t(p.nblk) * d->E * 4);
  return p;
}

// sk_part, sk_tab: the down projection's split of a partial last round of
// tiles (bf16 layers; see GemmArgs).
struct FfnWs { size_t tile_up, tile_down, act, sk_part, sk_tab; };
// a_cols: columns of the activation buffer (F, or 2F for bf16 pairs)
FfnWs plan_ffn(Carver& c, int64_t G, int64_t max_rows, int64_t a_cols, int eb, bool need_act,
               bool split = true) {
  FfnWs f;
  f.tile_up = c.take(size_t(G + 1) * 4);
  f.tile_down = c.take(size_t(G + 1) * 4);
  f.act = need_act ? c.take(size_t(max_rows) * a_cols * eb) : 0;
  split = split && eb == 2 && max_rows > 0;
  f.sk_part = c.take(split ? GB_SK_PART_BYTES : 0);
  f.sk_tab = c.take(split ? GB_SK_TAB_BYTES : 0);
  return f;
}


struct FwdWs {
  RouteWs route;
  PermWs perm;
  FfnWs ffn, ffn_shared;
  size_t idx, gate, counts, offsets, ros, tor, xperm, a, o, hs_unused, as, os, shared_off, losses;
};
FwdWs plan_fwd(Carver& c, const moe_dims* d, const moe_opts* o) {
  FwdWs f;
  const int eb = elem_bytes(o);
  const int64_t Tk = d->T * d->k;
  f.route = plan_route(c, d, o);
  f.perm = plan_perm(c, d, o);
  f.ffn = plan_ffn(c, d->E, Tk, d->F, eb, false);
  f.ffn_shared = plan_ffn(c, 1, d->T, d->F_shared, eb, false, false);
  f.idx = c.take(size_t(Tk) * 4);
  f.gate = c.take(size_t(Tk) * 4);
  f.counts = c.take(size_t(d->E) * 4);
  f.offsets = c.take(size_t(d->E + 1) * 4);
  f.ros = c.take(size_t(Tk) * 4);
  f.tor = c.take(size_t(Tk) * 4);
  f.xperm = c.take(size_t(Tk) * d->d * eb);
  f.a = c.take(size_t(Tk) * act_cols(o, d->F) * eb);
  f.o = c.take(size_t(Tk) * d->d * 4);
  f.as = c.take(size_t(d->T) * d->F_shared * eb);
  f.os = c.take(size_t(d->T) * d->d * 4);
  f.shared_off = c.take(2 * 4);
  f.losses = c.take(2 * 4);
  f.hs_unused = 0;
  return f;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

// The split of a partial last round of tiles into K segments (bf16 GEMMs with
// an fp32 store), on the workspace regions of `fw`.
void set_split(GemmArgs& g, void* ws, const FfnWs& fw) {
  if (fw.sk_part == fw.sk_tab) return;   // no regions carved
  g.sk_part = at<float>(ws, fw.sk_part);
  g.sk_tab = at<int32_t>(ws, fw.sk_tab);
  g.sk_cus = gemm_concurrent_tiles();
  if (g.sk_cus < 2) g.sk_part = nullptr;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                   \
  do {                                  \
    const hipError_t e_ = (expr);       \
    if (e_ != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

int check_ws(const void* ws, size_t have, size_t need) {
  if (need > have) return MOE_ERR_WORKSPACE;
  if (need > 0 && (!ws || (reinterpret_cast<uintptr_t>(ws) % ALIGN) != 0)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// ---- the steps, with validated arguments --------------------------------
// zn_out: where noisy top-k keeps x . W_noise (nullable: the workspace).
int do_route(const moe_dims* d, const moe_opts* o, const void* x, const float* Wg,
             const float* offset, const float* bias, const moe_router_inputs* ri, int32_t* idx,
             float* gate, float* scores, float* logits, int32_t* counts, float* losses,
             int32_t* n_nonfinite, float* zn_out, void* ws, const RouteWs& rw, hipStream_t st) {
  RouteArgs a{};
  a.x = x;
  a.x_bf16 = o->dtype == MOE_DTYPE_BF16;
  a.Wg = Wg;
  a.wfrag = at<float>(ws, rw.wfrag);
  a.offset = offset;
  a.bias = bias;
  a.T = int(d->T);
  a.d = int(d->d);
  a.E = int(d->E);
  a.k = int(d->k);
  a.EP = rw.EP;
  a.score = o->score;
  a.routing = o->routing;
  a.renorm = o->renorm != 0;
  a.gate_scale = o->gate_scale;
  a.idx = idx;
  a.gate = gate;
  a.scores = scores;
  a.logits = logits;
  a.part_p = at<float>(ws, rw.part_p);
  a.part_cnt = at<int32_t>(ws, rw.part_cnt);
  a.part_lse2 = at<float>(ws, rw.part_lse2);
  a.part_nf = at<int32_t>(ws, rw.part_nf);
  float* wfrag = at<float>(ws, rw.wfrag);
  // Wg in the layout the logits kernel reads, then the logits
  auto logits_pass = [&](const float* W, const RouteArgs& ra) -> hipError_t {
    if (rw.wide) {
      if (route_wg_direct(ra.E)) {   // the kernel reads Wg as stored
        RouteArgs rd = ra;
        rd.wfrag = nullptr;
        return launch_route_wide(rd, st);
      }
      hipError_t e = launch_wg_frag(W, ra.d, ra.E, ra.EP, wfrag, st);
      return e != hipSuccess ? e : launch_route_wide(ra, st);
    }
    return launch_route(ra, st);
  };
  if (o->routing == MOE_ROUTING_NOISY_TOPK) {
    // first pass: zn = x . W_noise (raw logits of the noise projection)
    float* zn = zn_out ? zn_out : at<float>(ws, rw.zn);
    RouteArgs an = a;
    an.Wg = ri->W_noise;
    an.offset = nullptr;
    an.logits = zn;
    an.logits_only = 1;
    MOE_TRY(logits_pass(ri->W_noise, an));
    a.noise = ri->noise;
    a.noise_logit = zn;
  }
  if (o->routing == MOE_ROUTING_RANDOM_SECOND) a.uniform = ri->uniform;
  if (o->routing == MOE_ROUTING_HASH) a.token_ids = ri->token_ids;
  MOE_TRY(logits_pass(Wg, a));
  if (counts || losses || n_nonfinite)
    MOE_TRY(launch_route_reduce(a, rw.nblk, o->aux_coef, o->z_coef, counts, losses, n_nonfinite, st));
  return MOE_OK;
}

int do_permute(const moe_dims* d, const moe_opts* o, const void* x, const int32_t* idx,
               int32_t* counts, int32_t* offsets, int32_t* ros, int32_t* tor, void* xperm,
               int32_t* n_dropped, void* ws, const PermWs& pw, hipStream_t st) {
  const int T = int(d->T), k = int(d->k), E = int(d->E);
  const int64_t C = capacity_of(d, o);
  int32_t* bc = at<int32_t>(ws, pw.blockcnt);
  const bool slot_major = o->priority == MOE_PRIORITY_SLOT;
  MOE_TRY(launch_dispatch_hist(idx, T, k, E, slot_major, bc, st));
  MOE_TRY(launch_dispatch_permute(idx, T, k, E, C, slot_major, bc, counts, offsets, n_dropped,
                                  x, int(d->d),
                                  elem_bytes(o), ros, tor, xperm, st));
  return MOE_OK;
}

// pair: the activation as bf16 (hi, lo) pairs, a_buf [max_rows, 2F] (bf16 only)
int do_ffn(const moe_opts* o, int64_t d, int64_t G, int64_t max_rows, int64_t F, int act,
           const void* xperm, const int32_t* offsets, const void* W13, const void* W2,
           void* h_save, void* a_buf, float* out, void* ws, const FfnWs& fw, hipStream_t st,
           bool pair = false) {
  const bool bf16 = o->dtype == MOE_DTYPE_BF16;
  pair = pair && bf16;
  const int64_t nu = act == MOE_ACT_SWIGLU ? 2 * F : F;
  GemmArgs g{};
  g.A = xperm;
  g.B = W13;
  g.b_group_stride = nu * d;
  g.offsets = offsets;
  g.G = int(G);
  g.max_rows = max_rows;
  g.N = int(F);
  g.K = int(d);
  g.up_off = act == MOE_ACT_SWIGLU ? int(F) : 0;
  g.epi = act == MOE_ACT_SWIGLU ? EPI_SWIGLU : EPI_GELU;
  g.out = a_buf;
  g.h_save = h_save;
  g.n_b = int(nu);
  g.tile_start = at<int32_t>(ws, fw.tile_up);
  if (pair) {
    g.out_ld = int(2 * F);
    g.lo_off = int(F);
  }
  MOE_TRY(bf16 ? launch_grouped_gemm_bf16(g, st) : launch_grouped_gemm_f32(g, st));
  GemmArgs g2 = g;
  g2.A = a_buf;
  g2.B = W2;
  g2.b_group_stride = d * F;
  g2.N = int(d);
  g2.K = int(pair ? 2 * F : F);
  g2.b_kwrap = pair ? int(F) : 0;
  g2.out_ld = 0;
  g2.lo_off = 0;
  g2.up_off = 0;
  g2.epi = EPI_STORE_F32;
  g2.out = out;
  g2.h_save = nullptr;
  g2.n_b = 0;
  g2.tile_start = at<int32_t>(ws, fw.tile_down);
  set_split(g2, ws, fw);
  MOE_TRY(bf16 ? launch_grouped_gemm_bf16(g2, st) : launch_grouped_gemm_f32(g2, st));
  return MOE_OK;
}

hipError_t fill_offsets_1(int32_t* off, int32_t rows, hipStream_t st) {
  return launch_fill_i32(off, 2, 0, rows, 0, 0, st);
}

// A second stream for the layer's independent branches (the shared expert,
// the router gradients, the routed dW2), forked from and joined back to the
// caller's stream with events.  One is kept per (device, caller stream), created
// on the first layer call from that stream and kept until the process ends, so
// calls made on different caller streams (from one host thread or several)
// never wait on each other through it.  The table and every record-and-wait
// pair are guarded by one lock.
struct SideStream {
  int dev;
  hipStream_t caller;
  hipStream_t s;
  hipEvent_t fork, join;
};
std::mutex g_side_mu;
std::vector<SideStream*> g_side;

hipError_t side_stream(hipStream_t caller, SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_side_mu);
  for (SideStream* sd : g_side)
    if (sd->dev == dev && sd->caller == caller) {
      *out = sd;
      return hipSuccess;
    }
  SideStream sd{dev, caller, nullptr, nullptr, nullptr};
  if ((e = hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming)) != hipSuccess) return e;
  if ((e = hipEventCreateWithFlags(&sd.join, hipEventDisableTiming)) != hipSuccess) {
    (void)hipEventDestroy(sd.fork);
    return e;
  }
  if ((e = hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking)) != hipSuccess) {
    (void)hipEventDestroy(sd.fork);
    (void)hipEventDestroy(sd.join);
    return e;
  }
  g_side.push_back(new SideStream(sd));
  *out = g_side.back();
  return hipSuccess;
}

// Work enqueued on `to` from now on waits for everything enqueued on `from` so far.
hipError_t stream_wait(hipStream_t to, hipStream_t from, hipEvent_t ev) {
  std::lock_guard<std::mutex> lk(g_side_mu);
  hipError_t e = hipEventRecord(ev, from);
  return e == hipSuccess ? hipStreamWaitEvent(to, ev, 0) : e;
}

// ---- backward workspace ------------------------------------------------------
// k-chunks of the T-reduction of dWg: enough 64x64 tiles x chunks to fill the
// chip (about 2048 workgroups), at most 64 chunks and at least 128 tokens each.
int dwg_split(const moe_dims* d) {
  const int64_t tiles = cdiv(d->d, 64) * cdiv(d->E, 64);
  int64_t s = cdiv(2048, tiles);
  s = s < 1 ? 1 : (s > 64 ? 64 : s);
  const int64_t by_t = d->T / 128 > 0 ? d->T / 128 : 1;
  return int(s < by_t ? s : by_t);
}

// Token chunks of the shared expert's weight-gradient reduction over T: enough
// 256x256 output tiles x chunks for one per CU, at most 16 chunks of at least
// 256 tokens.
int shared_split(const moe_dims* d, int64_t M, int64_t N) {
  const int64_t tiles = cdiv(M, 256) * cdiv(N, 256);
  int64_t s = cdiv(256, tiles);
  s = s < 1 ? 1 : (s > 16 ? 16 : s);
  const int64_t by_t = d->T / 256 > 0 ? d->T / 256 : 1;
  return int(s < by_t ? s : by_t);
}

// Router gradients of bf16 layers run on the bf16 grouped GEMM (dz and Wg as
// exact three-way bf16 splits): dx_router = dz Wg^T over K' = 6E plane slots,
// dWg = x^T dz over token chunks.  fp32 layers and noisy top-k use the fp32
// FMA kernels.
bool router_bwd_mfma(const moe_dims* d, const moe_opts* o) {
  return o->dtype == MOE_DTYPE_BF16 && d->d % 256 == 0 && o->routing != MOE_ROUTING_NOISY_TOPK;
}
int64_t router_kp(int64_t E) { return cdiv(6 * E, 128) * 128; }   // plane slots, padded
int64_t router_n3(int64_t E) { return cdiv(3 * E, 128) * 128; }   // dWg's B columns, padded
// Token chunks of dWg's reduction: about one 256-row output tile per CU, at
// least 256 tokens per chunk, at most 64 MB of fp32 partials.
int router_split(const moe_dims* d) {
  const int64_t n3 = router_n3(d->E);
  const int64_t tiles = (d->d / 256) * (n3 / (n3 % 256 == 0 ? 256 : 128));
  int64_t s = cdiv(256, tiles);
  const int64_t by_t = d->T / 256 > 0 ? d->T / 256 : 1;
  const int64_t by_mem = std::max<int64_t>(1, (int64_t(64) << 20) / (d->d * n3 * 4));
  s = std::min(std::min(s, by_t), by_mem);
  return int(s < 1 ? 1 : s);
}

struct BwdWs {
  FfnWs ffn, ffn_s;
  size_t dO, dg, dH, dXp, dz, dwg_part, dxr;
  size_t rplanes, wplanes, rpart, roff1, roffs;   // router gradients on the matrix cores
  size_t dyx, dHs, dxs, soff, ssplit_off, spart;
  size_t dzn, dwn_part;   // noisy top-k
};
BwdWs plan_bwd(Carver& c, const moe_dims* d, const moe_opts* o) {
  BwdWs b;
  const size_t eb = elem_bytes(o);
  const int64_t R = d->T * d->k, nu = n_up(o, d->F);
  const int64_t Fs = d->F_shared;
  b.ffn = plan_ffn(c, d->E, R, d->F, int(eb), false);
  b.ffn_s = plan_ffn(c, 1, d->T, Fs, int(eb), false, false);
  b.dO = c.take(size_t(R) * d->d * eb);
  b.dg = c.take(size_t(R) * 4);
  b.dH = c.take(size_t(R) * nu * eb);
  b.dXp = c.take(size_t(R) * d->d * 4);
  b.dz = c.take(size_t(d->T) * d->E * 4);
  const bool rm = router_bwd_mfma(d, o);
  b.dwg_part = c.take(rm ? 0 : size_t(dwg_split(d)) * d->d * d->E * 4);
  b.rplanes = c.take(rm ? size_t(d->T) * router_kp(d->E) * 2 : 0);
  b.wplanes = c.take(rm ? size_t(d->d) * router_kp(d->E) * 2 : 0);
  b.rpart = c.take(rm ? size_t(router_split(d)) * d->d * router_n3(d->E) * 4 : 0);
  b.roff1 = c.take(rm ? 2 * 4 : 0);
  b.roffs = c.take(rm ? size_t(router_split(d) + 1) * 4 : 0);
  const bool noisy = o->routing == MOE_ROUTING_NOISY_TOPK;
  // noisy top-k: dx_router = dz Wg^T + dzn W_noise^T as two partials summed in order
  b.dxr = c.take(size_t(noisy ? 2 : 1) * d->T * d->d * 4);
  b.dzn = c.take(noisy ? size_t(d->T) * d->E * 4 : 0);
  b.dwn_part = c.take(noisy ? size_t(dwg_split(d)) * d->d * d->E * 4 : 0);
  b.dyx = c.take(Fs ? size_t(d->T) * d->d * eb : 0);
  b.dHs = c.take(size_t(d->T) * 2 * Fs * eb);
  b.dxs = c.take(Fs ? size_t(d->T) * d->d * 4 : 0);
  b.soff = c.take(2 * 4);
  b.ssplit_off = c.take(Fs ? size_t(2 * 17) * 4 : 0);   // two chunk tables (dWs2, dWs13)
  b.spart = c.take(Fs ? size_t(std::max(shared_split(d, 2 * Fs, d->d) * 2 * Fs * d->d,
                                         shared_split(d, d->d, Fs) * d->d * Fs)) * 4
                      : 0);
  return b;
}

// Data gradient of an expert projection: out[rows] = epi(A[rows] . W[g]) with
// the weights W [g][K, N] read as stored.
GemmArgs gemm_dgrad(const void* A, const void* W, int64_t wstride, const int32_t* offsets, int G,
                    int64_t max_rows, int N, int K, int epi, void* out, const void* h_in, int n_b,
                    int up_off) {
  GemmArgs g{};
  g.A = A; g.B = W; g.b_group_stride = wstride; g.offsets = offsets; g.G = G;
  g.max_rows = max_rows; g.N = N; g.K = K; g.epi = epi; g.out = out; g.h_in = h_in;
  g.n_b = n_b; g.up_off = up_off; g.mode = GM_NN;
  return g;
}

// Weight gradient: out[g] = U_g^T . V_g over the rows of group g, U [rows, M],
// V [rows, N] as stored.
GemmArgs gemm_wgrad(const void* U, const void* V, const int32_t* offsets, int G, int M, int N,
                    float* out) {
  GemmArgs g{};
  g.A = U; g.B = V; g.offsets = offsets; g.G = G; g.M_fixed = M; g.N = N;
  g.epi = EPI_STORE_F32; g.out = out; g.mode = GM_KGROUP;
  return g;
}

hipError_t gemm_on(const moe_opts* o, GemmArgs g, int32_t* tile_start, hipStream_t st) {
  g.tile_start = tile_start;
  return o->dtype == MOE_DTYPE_BF16 ? launch_grouped_gemm_bf16(g, st) : launch_grouped_gemm_f32(g, st);
}

}  // namespace

// ============================================================================
extern "C" {

const char* moe_strerror(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or option";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

int moe_capacity(const moe_dims* d, const moe_opts* o, int64_t* C) {
  if (!d || !o || !C) return MOE_ERR_INVALID_ARG;
  if (d->T < 0 || d->E < 1 || d->k < 1 || !isfinite(o->capacity_factor)) return MOE_ERR_INVALID_ARG;
  *C = capacity_of(d, o);
  return MOE_OK;
}

int moe_workspace_size(const moe_dims* d, const moe_opts* o, int with_bwd, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  const int s = check_dims(d, o);
  if (s) return s;
  Carver c;
  plan_fwd(c, d, o);
  size_t need = c.off;
  if (with_bwd) {
    Carver cb;
    plan_bwd(cb, d, o);
    need = need > cb.off ? need : cb.off;
  }
  *bytes = need;
  return MOE_OK;
}

int moe_route(const moe_dims* d, const moe_opts* o, const void* x, const float* Wg,
              const float* logit_offset, const float* sel_bias, int32_t* topk_idx,
              float* topk_gate, float* scores, float* logits, int32_t* counts, float* losses,
              const moe_router_inputs* ri, void* ws, size_t ws_bytes, void* stream) {
  int s = check_dims(d, o);
  if (s) return s;
  if (d->T == 0) return MOE_OK;
  if (!x || !Wg || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x)) return MOE_ERR_INVALID_ARG;
  if ((s = check_router_inputs(o, ri))) return s;
  Carver c;
  const RouteWs rw = plan_route(c, d, o);
  if ((s = check_ws(ws, ws_bytes, c.off))) return s;
  return do_route(d, o, x, Wg, logit_offset, sel_bias, ri, topk_idx, topk_gate, scores, logits,
                  counts, losses, nullptr, nullptr, ws, rw, static_cast<hipStream_t>(stream));
}

int moe_permute(const moe_dims* d, const moe_opts* o, const void* x, const int32_t* topk_idx,
                int32_t* counts, int32_t* offsets, int32_t* row_of_slot, int32_t* token_of_row,
                void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  int s = check_dims(d, o);
  if (s) return s;
  if (!x || !topk_idx || !offsets || !row_of_slot || !token_of_row || !x_perm)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
  Carver c;
  const PermWs pw = plan_perm(c, d, o);
  if ((s = check_ws(ws, ws_bytes, c.off))) return s;
  if (d->T == 0) {
    // no tokens: every expert is empty
    return hip_status(launch_zero_i32(offsets, d->E + 1, static_cast<hipStream_t>(stream)));
  }
  return do_permute(d, o, x, topk_idx, counts, offsets, row_of_slot, token_of_row, x_perm, nullptr,
                    ws, pw, static_cast<hipStream_t>(stream));
}

int moe_expert_ffn(const moe_dims* d, const moe_opts* o, int64_t n_groups, int64_t max_rows,
                   int64_t F, const void* x_perm, const int32_t* offsets, const void* W13,
                   const void* W2, void* h_save, void* a_save, float* out, void* ws,
                   size_t ws_bytes, void* stream) {
  int s = check_dims(d, o);
  if (s) return s;
  if (n_groups < 1 || n_groups > 256 || max_rows < 0 || max_rows >= (int64_t(1) << 31))
    return MOE_ERR_INVALID_ARG;
  if ((s = check_width(o, F))) return s;
  if (!x_perm || !offsets || !W13 || !W2 || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(W13) || !aligned16(W2) || !aligned16(out))
    return MOE_ERR_INVALID_ARG;
  Carver c;
  const FfnWs fw = plan_ffn(c, n_groups, max_rows, act_cols(o, F), elem_bytes(o), a_save == nullptr);
  if ((s = check_ws(ws, ws_bytes, c.off))) return s;
  if (max_rows == 0) return MOE_OK;
  void* a_buf = a_save ? a_save : at<void>(ws, fw.act);
  return do_ffn(o, d->d, n_groups, max_rows, F, o->act, x_perm, offsets, W13, W2, h_save, a_buf,
                out, ws, fw, static_cast<hipStream_t>(stream), act_pair(o));
}

int moe_combine(const moe_dims* d, const float* out_perm, const int32_t* row_of_slot,
                const float* topk_gate, const float* shared_out, float* y, void* stream) {
  if (!d || d->T < 0 || d->k < 1 || d->k > 16 || d->d < 4 || d->d % 4) return MOE_ERR_INVALID_ARG;
  if (d->T == 0) return MOE_OK;
  if (!out_perm || !row_of_slot || !topk_gate || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(out_perm) || !aligned16(y) || (shared_out && !aligned16(shared_out)))
    return MOE_ERR_INVALID_ARG;
  if (d->T == 0) return MOE_OK;
  return hip_status(launch_combine(out_perm, row_of_slot, topk_gate, shared_out, int(d->T),
                                   int(d->k), int(d->d), y, static_cast<hipStream_t>(stream)));
}

int moe_layer_fwd(const moe_dims* d, const moe_opts* o, const moe_weights* w,
                  const moe_router_inputs* ri, const void* x, float* y, moe_saved* sv,
                  moe_stats* stats, void* ws, size_t ws_bytes, void* stream) {
  int s = check_dims(d, o);
  if (s) return s;
  if (d->T == 0) return MOE_OK;
  if (!w || !x || !y || !w->Wg || !w->W13 || !w->W2) return MOE_ERR_INVALID_ARG;
  if ((s = check_router_inputs(o, ri))) return s;
  if (sv && o->routing == MOE_ROUTING_NOISY_TOPK && !sv->noise_logits) return MOE_ERR_INVALID_ARG;
  if (d->F_shared > 0 && (!w->Ws13 || !w->Ws2)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(w->W13) || !aligned16(w->W2) ||
      (d->F_shared > 0 && (!aligned16(w->Ws13) || !aligned16(w->Ws2))))
    return MOE_ERR_INVALID_ARG;
  if (sv && (!sv->topk_idx || !sv->topk_gate || !sv->logits || !sv->counts || !sv->offsets ||
             !sv->row_of_slot || !sv->token_of_row || !sv->x_perm || !sv->h || !sv->a || !sv->o ||
             !sv->losses || (d->F_shared > 0 && (!sv->h_shared || !sv->a_shared))))
    return MOE_ERR_INVALID_ARG;
  if (sv && (!aligned16(sv->x_perm) || !aligned16(sv->o) || !aligned16(sv->a) || !aligned16(sv->h)))
    return MOE_ERR_INVALID_ARG;
  Carver c;
  const FwdWs f = plan_fwd(c, d, o);
  if ((s = check_ws(ws, ws_bytes, c.off))) return s;
  if (d->T == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);

  int32_t* idx = sv ? sv->topk_idx : at<int32_t>(ws, f.idx);
  float* gate = sv ? sv->topk_gate : at<float>(ws, f.gate);
  int32_t* counts = sv ? sv->counts : at<int32_t>(ws, f.counts);
  int32_t* offsets = sv ? sv->offsets : at<int32_t>(ws, f.offsets);
  int32_t* ros = sv ? sv->row_of_slot : at<int32_t>(ws, f.ros);
  int32_t* tor = sv ? sv->token_of_row : at<int32_t>(ws, f.tor);
  void* xperm = sv ? sv->x_perm : at<void>(ws, f.xperm);
  void* abuf = sv ? sv->a : at<void>(ws, f.a);
  float* obuf = sv ? sv->o : at<float>(ws, f.o);
  // The router losses are part of the forward whenever a coefficient is set;
  // with nowhere else to put them they land in the workspace.
  const bool want_losses = o->aux_coef != 0.0f || o->z_coef != 0.0f;
  float* losses = sv ? sv->losses
                     : (stats && stats->losses) ? stats->losses
                     : want_losses ? at<float>(ws, f.losses) : nullptr;

  // the shared expert depends only on x: it runs on the side stream while the
  // router, dispatch and routed experts run on the caller's
  SideStream* side = nullptr;
  float* shared = nullptr;
  // an error after the fork still joins the side stream before returning
  auto joined = [&](int code) {
    // the join's own status cannot replace the error being reported
    if (side) (void)stream_wait(st, side->s, side->join);
    return code;
  };
  if (d->F_shared > 0) {
    MOE_TRY(side_stream(st, &side));
    MOE_TRY(stream_wait(side->s, st, side->fork));
    int32_t* soff = at<int32_t>(ws, f.shared_off);
    if (hipError_t e = fill_offsets_1(soff, int32_t(d->T), side->s); e != hipSuccess)
      return joined(hip_status(e));
    shared = at<float>(ws, f.os);
    s = do_ffn(o, d->d, 1, d->T, d->F_shared, MOE_ACT_SWIGLU, x, soff, w->Ws13, w->Ws2,
               sv ? sv->h_shared : nullptr, sv ? sv->a_shared : at<void>(ws, f.as), shared, ws,
               f.ffn_shared, side->s);
    if (s) return joined(s);
  }
  s = do_route(d, o, x, w->Wg, w->logit_offset, w->sel_bias, ri, idx, gate, nullptr,
               sv ? sv->logits : nullptr, nullptr, losses, stats ? stats->n_nonfinite : nullptr,
               sv ? sv->noise_logits : nullptr, ws, f.route, st);
  if (s) return joined(s);
  s = do_permute(d, o, x, idx, counts, offsets, ros, tor, xperm, stats ? stats->n_dropped : nullptr,
                 ws, f.perm, st);
  if (s) return joined(s);
  s = do_ffn(o, d->d, d->E, d->T * d->k, d->F, o->act, xperm, offsets, w->W13, w->W2,
             sv ? sv->h : nullptr, abuf, obuf, ws, f.ffn, st, act_pair(o));
  if (s) return joined(s);
  if (side) MOE_TRY(stream_wait(st, side->s, side->join));
  MOE_TRY(launch_combine(obuf, ros, gate, shared, int(d->T), int(d->k), int(d->d), y, st));
  if (stats) {
    if (stats->counts) MOE_TRY(hipMemcpyAsync(stats->counts, counts, size_t(d->E) * 4,
                                              hipMemcpyDeviceToDevice, st));
    if (stats->losses && stats->losses != losses)
      MOE_TRY(hipMemcpyAsync(stats->losses, losses, 8, hipMemcpyDeviceToDevice, st));
  }
  return MOE_OK;
}

int moe_layer_bwd(const moe_dims* d, const moe_opts* o, const moe_weights* w,
                  const moe_router_inputs* ri, const void* x, const moe_saved* sv,
                  const float* dy, float* dx, moe_grads* grads, void* ws, size_t ws_bytes,
                  void* stream) {
  int s = check_dims(d, o);
  if (s) return s;
  if (d->T == 0) return MOE_OK;
  const int64_t Fs = d->F_shared;
  const bool noisy = o->routing == MOE_ROUTING_NOISY_TOPK;
  if ((s = check_router_inputs(o, ri))) return s;
  if (noisy && (!sv || !sv->noise_logits || !grads || !grads->dW_noise)) return MOE_ERR_INVALID_ARG;
  if (!w || !x || !sv || !dy || !dx || !grads || !w->Wg || !w->W13 || !w->W2) return MOE_ERR_INVALID_ARG;
  if (!grads->dWg || !grads->dW13 || !grads->dW2) return MOE_ERR_INVALID_ARG;
  if ((grads->dH && !aligned16(grads->dH)) || (grads->dH_shared && !aligned16(grads->dH_shared)))
    return MOE_ERR_INVALID_ARG;
  if (Fs > 0 && (!w->Ws13 || !w->Ws2 || !grads->dWs13 || !grads->dWs2 || !sv->h_shared ||
                 !sv->a_shared))
    return MOE_ERR_INVALID_ARG;
  if (!sv->topk_idx || !sv->topk_gate || !sv->logits || !sv->counts || !sv->offsets ||
      !sv->row_of_slot || !sv->x_perm || !sv->h || !sv->a || !sv->o)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dx) || !aligned16(sv->o) ||
      !aligned16(sv->x_perm) || !aligned16(sv->h) || !aligned16(sv->a) || !aligned16(w->W13) ||
      !aligned16(w->W2))
    return MOE_ERR_INVALID_ARG;
  Carver c;
  const BwdWs b = plan_bwd(c, d, o);
  if ((s = check_ws(ws, ws_bytes, c.off))) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = o->dtype == MOE_DTYPE_BF16;
  const int T = int(d->T), k = int(d->k), E = int(d->E), D = int(d->d), F = int(d->F);
  const int nu = int(n_up(o, d->F));
  const int64_t R = d->T * d->k;
  const bool swiglu = o->act == MOE_ACT_SWIGLU;
  int32_t* ts = at<int32_t>(ws, b.ffn.tile_up);
  int32_t* ts_s = at<int32_t>(ws, b.ffn_s.tile_up);
  // gradients of the pre-activations: the caller's buffers when given
  void* dH = grads->dH ? grads->dH : at<void>(ws, b.dH);
  void* dHs = grads->dH_shared ? grads->dH_shared : at<void>(ws, b.dHs);

  // combine backward: dO, dg, and dy in the x type for the shared expert
  void* dyx = Fs ? at<void>(ws, b.dyx) : nullptr;
  MOE_TRY(launch_combine_bwd(dy, sv->o, sv->row_of_slot, sv->topk_gate, T, k, D, bf16,
                             at<void>(ws, b.dO), at<float>(ws, b.dg), dyx, st));
  // row-offset tables of the shared expert and the router gradients, in one launch
  const bool rmfma = router_bwd_mfma(d, o);
  const int s2 = Fs ? shared_split(d, D, int(Fs)) : 0, s13 = Fs ? shared_split(d, 2 * Fs, D) : 0;
  const int rs = rmfma ? router_split(d) : 0;
  {
    SeqFills f{};
    if (Fs > 0) {
      int32_t* so = at<int32_t>(ws, b.ssplit_off);
      f.add(at<int32_t>(ws, b.soff), 2, int32_t(T), int32_t(T));
      f.add(so, s2 + 1, int32_t(cdiv(T, s2)), int32_t(T));
      f.add(so + 17, s13 + 1, int32_t(cdiv(T, s13)), int32_t(T));
    }
    if (rmfma) {
      f.add(at<int32_t>(ws, b.roff1), 2, int32_t(T), int32_t(T));
      f.add(at<int32_t>(ws, b.roffs), rs + 1, int32_t(cdiv(T, rs)), int32_t(T));
    }
    MOE_TRY(launch_fill_seqs(f, st));
  }
  // The shared expert's and the router's gradients and the routed dW2 depend
  // only on combine backward's outputs: they run on the side stream while the
  // routed experts' data gradients and dW13 run on the caller's; the join
  // precedes the unpermute-sum.  dW2 is store-bound and the data gradients
  // read weights and multiply, so the two streams overlap well (4096 tokens,
  // d = 4096, 8 experts of width 14336, top-2: 11.8 -> 10.9 ms per step).
  float* dxs = nullptr;
  float* dxr = at<float>(ws, b.dxr);
  auto side_branch = [&](hipStream_t bs) -> int {
    // shared expert (gate 1 on every token)
    if (Fs > 0) {
      const int fs = int(Fs);
      int32_t* soff = at<int32_t>(ws, b.soff);
      dxs = at<float>(ws, b.dxs);
      MOE_TRY(gemm_on(o, gemm_dgrad(dyx, w->Ws2, 0, soff, 1, T, fs, D, EPI_SWIGLU_BWD,
                                    dHs, sv->h_shared, 2 * fs, fs),
                      ts_s, bs));
      MOE_TRY(gemm_on(o, gemm_dgrad(dHs, w->Ws13, 0, soff, 1, T, D, 2 * fs,
                                    EPI_STORE_F32, dxs, nullptr, 0, 0),
                      ts_s, bs));
      // weight gradients: the T-reduction split into equal token chunks (one
      // K-grouped GEMM over the chunks), then the chunk partials summed in order
      int32_t* coff = at<int32_t>(ws, b.ssplit_off);
      float* part = at<float>(ws, b.spart);
      MOE_TRY(gemm_on(o, gemm_wgrad(dyx, sv->a_shared, coff, s2, D, fs, part), ts_s, bs));
      MOE_TRY(launch_sum_partials(part, s2, int64_t(D) * fs, grads->dWs2, bs));
      MOE_TRY(gemm_on(o, gemm_wgrad(dHs, x, coff + 17, s13, 2 * fs, D, part), ts_s, bs));
      MOE_TRY(launch_sum_partials(part, s13, int64_t(2) * fs * D, grads->dWs13, bs));
    }
    // router: dz from the kept gates' gradient and the two losses; dWg = x^T dz;
    // dx_router = dz Wg^T
    float* dz = at<float>(ws, b.dz);
    MOE_TRY(launch_router_bwd(sv->logits, sv->topk_idx, at<float>(ws, b.dg), sv->counts, T, E, k,
                              o->score, o->renorm != 0, o->gate_scale, o->aux_coef, o->z_coef, dz,
                              bs));
    if (rmfma) {
      const int KP = int(router_kp(E)), N3 = int(router_n3(E)), s = rs;
      uint16_t* zp = at<uint16_t>(ws, b.rplanes);     // [T, KP]: dz slots hi mid lo hi hi mid
      uint16_t* wp = at<uint16_t>(ws, b.wplanes);     // [D, KP]: Wg slots hi hi hi mid lo mid
      MOE_TRY(launch_router_planes(dz, T, E, KP, 0x100210u, zp, bs));
      MOE_TRY(launch_router_planes(w->Wg, D, E, KP, 0x121000u, wp, bs));
      int32_t* off1 = at<int32_t>(ws, b.roff1);
      GemmArgs gx{};
      gx.A = zp; gx.B = wp; gx.offsets = off1; gx.G = 1; gx.max_rows = T; gx.N = D; gx.K = KP;
      gx.epi = EPI_STORE_F32; gx.out = dxr; gx.mode = GM_NT;
      MOE_TRY(launch_grouped_gemm_bf16(gx, bs));
      // dWg = x^T [hi | mid | lo] per token chunk; chunks and planes summed in order
      int32_t* coff = at<int32_t>(ws, b.roffs);
      float* part = at<float>(ws, b.rpart);
      GemmArgs gw = gemm_wgrad(x, zp, coff, s, D, N3, part);
      gw.ldb = KP;
      MOE_TRY(launch_grouped_gemm_bf16(gw, bs));
      MOE_TRY(launch_dwg_reduce(part, s, D, N3, E, grads->dWg, bs));
    } else if (noisy) {
      MOE_TRY(launch_strided_gemm(x, bf16, 1, D, dz, E, 1, D, E, T, dwg_split(d),
                                  at<float>(ws, b.dwg_part), grads->dWg, bs));
      // H = z + noise * softplus(zn): dzn = dz * noise * sigmoid(zn);
      // dW_noise = x^T dzn; dx_router = dz Wg^T + dzn W_noise^T
      float* dzn = at<float>(ws, b.dzn);
      float* part = dxr + int64_t(T) * D;
      MOE_TRY(launch_noise_grad(dz, ri->noise, sv->noise_logits, int64_t(T) * E, dzn, bs));
      MOE_TRY(launch_strided_gemm(x, bf16, 1, D, dzn, E, 1, D, E, T, dwg_split(d),
                                  at<float>(ws, b.dwn_part), grads->dW_noise, bs));
      MOE_TRY(launch_strided_gemm(dz, false, E, 1, w->Wg, 1, E, T, D, E, 1, dxr, nullptr, bs));
      MOE_TRY(launch_strided_gemm(dzn, false, E, 1, ri->W_noise, 1, E, T, D, E, 1, part, nullptr, bs));
      MOE_TRY(launch_sum_partials(dxr, 2, int64_t(T) * D, dxr, bs));
    } else {
      MOE_TRY(launch_strided_gemm(x, bf16, 1, D, dz, E, 1, D, E, T, dwg_split(d),
                                  at<float>(ws, b.dwg_part), grads->dWg, bs));
      MOE_TRY(launch_strided_gemm(dz, false, E, 1, w->Wg, 1, E, T, D, E, 1, dxr, nullptr, bs));
    }
    // routed experts' dW2[e] = dO_e^T a_e needs only combine backward's dO: its
    // fp32 stores run here, beside the data gradients' weight reads and
    // products (the K-grouped mode reads no tile table)
    // (with activation pairs the saved rows are [hi | lo]; dW2 uses hi)
    GemmArgs gw2 = gemm_wgrad(at<void>(ws, b.dO), sv->a, sv->offsets, E, D, F, grads->dW2);
    gw2.ldb = act_cols(o, F);
    MOE_TRY(gemm_on(o, gw2, ts_s, bs));
    return MOE_OK;
  };
  auto routed_branch = [&]() -> int {
    // routed experts, data gradients: dA = dO W2 (+ activation backward) -> dH; dXp = dH W13
    MOE_TRY(gemm_on(o, gemm_dgrad(at<void>(ws, b.dO), w->W2, int64_t(D) * F, sv->offsets, E, R, F, D,
                                  swiglu ? EPI_SWIGLU_BWD : EPI_GELU_BWD, dH, sv->h,
                                  nu, swiglu ? F : 0),
                    ts, st));
    GemmArgs gx = gemm_dgrad(dH, w->W13, int64_t(nu) * D, sv->offsets, E, R, D, nu,
                             EPI_STORE_F32, at<void>(ws, b.dXp), nullptr, 0, 0);
    set_split(gx, ws, b.ffn);
    MOE_TRY(gemm_on(o, gx, ts, st));
    // routed experts, weight gradient over each expert's rows: dW13[e] = dH_e^T x_e
    MOE_TRY(gemm_on(o, gemm_wgrad(dH, sv->x_perm, sv->offsets, E, nu, D, grads->dW13),
                    ts, st));
    return MOE_OK;
  };
  SideStream* side = nullptr;
  MOE_TRY(side_stream(st, &side));
  MOE_TRY(stream_wait(side->s, st, side->fork));
  // Launch order: with a shared expert the side branch holds its GEMMs and is
  // launched first; without one it holds only the router's gradients and dW2,
  // and the routed branch goes first so the caller's stream, which the device
  // has usually drained by then, gets its next kernel without waiting for them.
  int e_main = 0, e_side = 0;
  if (Fs > 0) {
    e_side = side_branch(side->s);
    e_main = routed_branch();
  } else {
    e_main = routed_branch();
    e_side = side_branch(side->s);
  }
  MOE_TRY(stream_wait(st, side->s, side->join));
  if (e_side) return e_side;
  if (e_main) return e_main;
  MOE_TRY(launch_unpermute_sum(at<float>(ws, b.dXp), sv->row_of_slot, dxs, dxr, T, k, D, dx, st));
  return MOE_OK;
}

int moe_mx_quantize_weights(const moe_opts* o, const void* w, int64_t G, int64_t N, int64_t K,
                            uint8_t* codes, uint8_t* scales, void* stream) {
  if (!o || !w || !codes || !scales || G < 1 || N < 1 || K < 64 || K % 64) return MOE_ERR_INVALID_ARG;
  if (o->dtype != MOE_DTYPE_F32 && o->dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (!aligned16(w) || !aligned16(codes)) return MOE_ERR_INVALID_ARG;
  if (K >= (int64_t(1) << 31) || G * N * K >= (int64_t(1) << 40)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_mx_quantize_weights(w, o->dtype == MOE_DTYPE_BF16, G * N, int(K), int(N),
                                               codes, scales, static_cast<hipStream_t>(stream)));
}

int moe_mx_quantize_act(const moe_opts* o, const void* x, int64_t rows, int64_t K, int64_t stride,
                        uint8_t* codes, uint8_t* scales, void* stream) {
  if (!o || rows < 0 || K < 64 || K % 64 || stride < rows) return MOE_ERR_INVALID_ARG;
  if (o->dtype != MOE_DTYPE_F32 && o->dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!x || !codes || !scales || !aligned16(x) || !aligned16(codes)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_mx_quantize_act(x, o->dtype == MOE_DTYPE_BF16, rows, int(K), stride,
                                           codes, scales, static_cast<hipStream_t>(stream)));
}

int moe_expert_ffn_mx(const moe_dims* d, const moe_opts* o, int64_t n_groups, int64_t max_rows,
                      int64_t F, const uint8_t* xq, const uint8_t* xs, int64_t x_stride,
                      const int32_t* offsets, const uint8_t* W13q, const uint8_t* W13s,
                      const uint8_t* W2q, const uint8_t* W2s, uint8_t* aq, uint8_t* aqs,
                      int64_t a_stride, float* out, void* stream) {
  if (!d || !o || n_groups < 1 || n_groups > 256 || max_rows < 0 || max_rows >= (int64_t(1) << 31) ||
      F < 256 || x_stride < max_rows + 4 || a_stride < max_rows + 4 || x_stride % 4 ||
      a_stride % 4)
    return MOE_ERR_INVALID_ARG;
  if (o->act != MOE_ACT_SWIGLU && o->act != MOE_ACT_GELU) return MOE_ERR_INVALID_ARG;
  if (o->act_pair != 0 && o->act_pair != 1) return MOE_ERR_INVALID_ARG;
  if (d->d % 256 || F % 256) return MOE_ERR_UNSUPPORTED;
  if (max_rows == 0) return MOE_OK;
  if (!xq || !xs || !offsets || !W13q || !W13s || !W2q || !W2s || !aq || !aqs || !out)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(W13q) || !aligned16(W2q) || !aligned16(aq) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(W13s) & 3) || (reinterpret_cast<uintptr_t>(W2s) & 3) ||
      (reinterpret_cast<uintptr_t>(xs) & 3) || (reinterpret_cast<uintptr_t>(aqs) & 3))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_mx_ffn(xq, xs, x_stride, offsets, int(n_groups), max_rows, int(d->d),
                                  int(F), o->act, W13q, W13s, W2q, W2s, aq, aqs, a_stride, out,
                                  static_cast<hipStream_t>(stream)));
}

int moe_score_histogram(const float* scores, int64_t T, int64_t E, float lo, float hi,
                        int32_t nbins, int32_t* hist, void* stream) {
  if (!hist || T < 0 || E < 1 || nbins < 1 || !isfinite(lo) || !isfinite(hi) || !(lo < hi))
    return MOE_ERR_INVALID_ARG;
  if (T > 0 && !scores) return MOE_ERR_INVALID_ARG;
  if (E > 256 || nbins > 65536 || T * E >= (int64_t(1) << 40)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_score_hist(scores, T, int(E), lo, hi, nbins, hist,
                                      static_cast<hipStream_t>(stream)));
}

int moe_bias_from_histogram(const int32_t* hist, int64_t E, int32_t nbins, float lo, float hi,
                            float target, float* bias, void* stream) {
  if (!hist || !bias || E < 1 || nbins < 1 || !isfinite(lo) || !isfinite(hi) || !(lo < hi) ||
      !isfinite(target) || target < 0.0f)
    return MOE_ERR_INVALID_ARG;
  if (E > 256 || nbins > 65536) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_bias_solve(hist, int(E), nbins, lo, hi, target, bias,
                                      static_cast<hipStream_t>(stream)));
}

int moe_router_report(int64_t E, int64_t d, const int32_t* counts, const int32_t* n_dropped,
                      const float* out_perm, const int32_t* offsets, float* expert_norm,
                      float* report, void* stream) {
  if (!counts || !report || E < 1 || (out_perm && (!offsets || !expert_norm || d < 1)))
    return MOE_ERR_INVALID_ARG;
  if (E > 256 || d >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_router_report(int(E), int(d), counts, n_dropped, out_perm, offsets,
                                         expert_norm, report, static_cast<hipStream_t>(stream)));
}

int moe_bias_update(const int32_t* counts, float* bias, int64_t E, float target, float gamma,
                    void* stream) {
  if (!counts || !bias || E < 1 || E > (int64_t(1) << 30) || !isfinite(target) || !isfinite(gamma))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_bias_update(counts, bias, int(E), target, gamma,
                                       static_cast<hipStream_t>(stream)));
}

}  // extern "C"
