// Internal launcher interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ------------------------------------------------------------------ router
struct RouteArgs {
  const void* x;            // [T, d] bf16 or fp32
  int x_bf16;
  const float* Wg;          // [d, E]
  const float* wfrag;       // Wg in the wide kernel's fp32 fragment layout
  const float* offset;      // nullable [E]
  const float* bias;        // nullable [E]
  int T, d, E, k, EP;
  int score, renorm;
  int routing;              // moe_routing: 0 top-k, 1 uniform, 2 noisy top-k, 3 random second, 4 hash
  int logits_only;          // write the raw logits x . Wg only (the noise projection pass)
  const float* noise;       // noisy top-k: [T, E] standard-normal draws
  const float* noise_logit; // noisy top-k: [T, E] x . W_noise
  const float* uniform;     // random second expert: [T] draws in [0, 1)
  const int32_t* token_ids; // hash routing: [T]
  float gate_scale;
  int32_t* idx;             // [T, k]
  float* gate;              // [T, k]
  float* scores;            // nullable [T, E]
  float* logits;            // nullable [T, E]
  float* part_p;            // [nblk][EP]  sum_t of scores normalised over E
  int32_t* part_cnt;        // [nblk][EP]  selections per expert
  float* part_lse2;         // [nblk]      sum_t logsumexp(z_t)^2
  int32_t* part_nf;         // [nblk]      tokens with a non-finite logit
};
constexpr int ROUTE_BT = 32;   // tokens per route block

int route_pad_experts(int E);  // 32, 64, 128 or 256
// Wg in the wide kernel's fp32 fragment layout (d % 64 == 0, EP % 32 == 0).
hipError_t launch_wg_frag(const float* Wg, int d, int E, int EP, float* out, hipStream_t st);
hipError_t launch_route(const RouteArgs& a, hipStream_t st);   // fp32 FMA logits
// bf16 tokens: route_wide_bt(T, EP) tokens per block (64, or 32 for small
// batches; one partial-sum row per block), logits kept on chip, Wg in the
// fragment layout; d % (64 * 256 / EP) == 0.
int route_wide_bt(int64_t T, int EP);
hipError_t launch_route_wide(const RouteArgs& a, hipStream_t st);
hipError_t launch_route_reduce(const RouteArgs& a, int nblk, float aux_coef, float z_coef,
                               int32_t* counts, float* losses, int32_t* n_nonfinite,
                               hipStream_t st);

// ------------------------------------------------------------------ dispatch
// Orders in which the dispatch kernels walk the T*k slots, one per lane: flat
// (v = t*k + j, token priority) or slot-major (v = j*T + t, slot priority).
// Blocks of the histogram / rank kernels (and rows of their per-block count
// arrays) are runs of consecutive slots in that order.
enum DispOrder { DISP_SLOT = 1, DISP_FLAT = 2 };
int dispatch_order(bool slot_major);
int dispatch_blocks(int T, int k, bool slot_major);
hipError_t launch_dispatch_hist(const int32_t* idx, int T, int k, int E, bool slot_major,
                                int32_t* blockcnt, hipStream_t st);
hipError_t launch_dispatch_permute(const int32_t* idx, int T, int k, int E, int64_t C,
                                   bool slot_major, const int32_t* blockcnt, int32_t* counts,
                                   int32_t* offsets, int32_t* n_dropped, const void* x, int d,
                                   int elem_bytes, int32_t* row_of_slot, int32_t* token_of_row,
                                   void* x_perm, hipStream_t st);

// ------------------------------------------------------------------ grouped GEMM
// Epilogues: fp32 store; forward activations (GELU, SwiGLU of two panels);
// backward through the activation using the saved pre-activation h_in.
enum Epi { EPI_STORE_F32 = 0, EPI_GELU = 1, EPI_SWIGLU = 2, EPI_SWIGLU_BWD = 3, EPI_GELU_BWD = 4 };

// Operand layouts of the grouped GEMM (group g owns rows offsets[g]..offsets[g+1]-1):
//  GM_NT     out[rows] = epi(A[rows] . B[g]^T); A [rows, K], B [g][n, K]
//  GM_NN     out[rows] = epi(A[rows] . B[g]);   A [rows, K], B [g][K, n]
//  GM_KGROUP out[g] = A_g^T . B_g over the M_g rows of group g; A [rows, M_fixed],
//            B [rows, N], out [g][M_fixed, N] fp32 (weight gradients; empty
//            groups write zeros).
enum GemmMode { GM_NT = 0, GM_KGROUP = 1, GM_NN = 2 };
struct GemmArgs {
  const void* A;
  const void* B;
  int64_t b_group_stride;   // row modes: elements between groups of B
  const int32_t* offsets;   // [G+1] row offsets of the groups
  int G;
  int64_t max_rows;         // row modes: upper bound of offsets[G] (launch size)
  int N;                    // output columns
  int K;                    // row modes: reduction length
  int up_off;               // SwiGLU: column offset of the up half (= F)
  int epi;
  void* out;                // row modes [rows, N] (bf16 activations or fp32); K mode fp32
  void* h_save;             // nullable [rows, n_b] pre-activation (forward epilogues)
  const void* h_in;         // [rows, n_b] saved pre-activation (backward epilogues)
  int n_b;                  // row length of h_save / h_in (2F SwiGLU, F GELU)
  int32_t* tile_start;      // [G+1] scratch for the fp32 planner
  int mode;                 // GemmMode
  int M_fixed;              // K mode: rows of each group's output
  int64_t ldb;              // K mode: row stride of B in elements (0: N)
  // Activation pairs (bf16 forward layout): the GELU / SwiGLU epilogue writes
  // hi = bf16(a) at column n and lo = bf16(a - hi) at column lo_off + n of
  // rows of out_ld elements (lo_off = 0: hi only, rows of N).  The down
  // projection then runs over K = 2F with b_kwrap = F: B's element (n, k) is
  // B[n * F + k mod F], so the weights multiply both halves.
  int out_ld;
  int lo_off;
  int b_kwrap;
  // Split of a partial last round (bf16 row modes with an fp32 store and
  // K >= GB_SK_MIN_K; nullable sk_part = off).  When the tiles leave a last
  // round that fills at most half of the sk_cus workgroups that run at once,
  // those tiles are cut into S <= 4 K segments (S * tiles <= sk_cus) whose
  // fp32 partial sums go to sk_part and are added in segment order by a
  // second kernel; the whole tiles run as before.  sk_part holds GB_SK_SLOTS
  // tiles of BM * BN floats, sk_tab 2 + 3 * GB_SK_SLOTS / 2 ints.  sk_grid0
  // is set by the launcher.
  float* sk_part;
  int32_t* sk_tab;
  int sk_cus;
  int sk_grid0;
};
constexpr int GB_SK_SLOTS = 256;
constexpr int GB_SK_MIN_K = 10240;   // shortest reduction that is split
constexpr size_t GB_SK_PART_BYTES = size_t(GB_SK_SLOTS) * 256 * 256 * 4;
constexpr size_t GB_SK_TAB_BYTES = size_t(2 + 3 * GB_SK_SLOTS / 2) * 4;
// Workgroups of the grouped GEMM that run at once on the current device (one
// per compute unit), at most GB_SK_SLOTS.
int gemm_concurrent_tiles();
hipError_t launch_grouped_gemm_bf16(const GemmArgs& g, hipStream_t st);
hipError_t launch_grouped_gemm_f32(const GemmArgs& g, hipStream_t st);

// ------------------------------------------------------------------ combine
hipError_t launch_combine(const float* o, const int32_t* row_of_slot, const float* gate,
                          const float* shared, int T, int k, int d, float* y, hipStream_t st);
hipError_t launch_fill_i32(int32_t* out, int n, int32_t v0, int32_t v1, int32_t v2, int32_t v3,
                           hipStream_t st);
hipError_t launch_zero_i32(int32_t* out, int64_t n, hipStream_t st);
// out[i] = min(i * step, cap) for i < n
hipError_t launch_fill_seq_i32(int32_t* out, int n, int32_t step, int32_t cap, hipStream_t st);
// Up to 8 such tables in one launch.
struct SeqFills {
  int32_t* out[8];
  int n[8];
  int32_t step[8], cap[8];
  int count;
  void add(int32_t* o, int nn, int32_t s, int32_t c) {
    out[count] = o; n[count] = nn; step[count] = s; cap[count] = c; ++count;
  }
};
hipError_t launch_fill_seqs(const SeqFills& f, hipStream_t st);
hipError_t launch_bias_update(const int32_t* counts, float* bias, int E, float target,
                              float gamma, hipStream_t st);

// ------------------------------------------------------------------ backward
hipError_t launch_combine_bwd(const float* dy, const float* o, const int32_t* ros, const float* gate,
                              int T, int k, int d, bool bf16, void* dO, float* dg, void* dy_x,
                              hipStream_t st);
hipError_t launch_router_bwd(const float* z, const int32_t* idx, const float* dg,
                             const int32_t* counts, int T, int E, int k, int score, int renorm,
                             float scale, float aux_coef, float z_coef, float* dz, hipStream_t st);
// P [nsplit][M][N] partials; out (nullable) = their sum in split order
hipError_t launch_strided_gemm(const void* A, bool a_bf16, int64_t sam, int64_t sak, const float* B,
                               int64_t sbk, int64_t sbn, int M, int N, int K, int nsplit, float* P,
                               float* out, hipStream_t st);
// dzn = dz * noise * sigmoid(zn), n elements
hipError_t launch_noise_grad(const float* dz, const float* noise, const float* zn, int64_t n,
                             float* dzn, hipStream_t st);
// out[i] = sum over z of P[z * n + i], z = 0..nz-1 in order
hipError_t launch_sum_partials(const float* P, int nz, int64_t n, float* out, hipStream_t st);
// Router gradients on the bf16 grouped GEMM: src [rows, E] fp32 written as rows
// of KP bf16 values whose slot s (columns s*E..s*E+E-1, s < 6) holds plane
// (pattern >> 4s) & 15 of the exact three-way split (0 hi, 1 mid, 2 lo);
// columns from 6E on are zero.
hipError_t launch_router_planes(const float* src, int64_t rows, int E, int KP, uint32_t pattern,
                                uint16_t* out, hipStream_t st);
// dWg[d][e] = sum over chunks g (in order) of P[g][d][e] + P[g][d][E+e] + P[g][d][2E+e].
hipError_t launch_dwg_reduce(const float* P, int nchunks, int D, int N3, int E, float* dWg,
                             hipStream_t st);
hipError_t launch_unpermute_sum(const float* dxp, const int32_t* ros, const float* e1,
                                const float* e2, int T, int k, int d, float* dx, hipStream_t st);

// ------------------------------------------------------------------ balance / monitoring
hipError_t launch_score_hist(const float* s, int64_t T, int E, float lo, float hi, int nbins,
                             int32_t* hist, hipStream_t st);
hipError_t launch_bias_solve(const int32_t* hist, int E, int nbins, float lo, float hi, float target,
                             float* bias, hipStream_t st);
hipError_t launch_router_report(int E, int d, const int32_t* counts, const int32_t* n_dropped,
                                const float* o, const int32_t* offsets, float* norm, float* report,
                                hipStream_t st);

// ------------------------------------------------------------------ MXFP4 experts
// weights w [rows = G*N, K] (bf16 or fp32) -> codes [rows, K/2], scales [G][K/32][N]
hipError_t launch_mx_quantize_weights(const void* w, bool bf16, int64_t rows, int K, int N,
                                      uint8_t* codes, uint8_t* scales, hipStream_t st);
// activations x [rows, K] -> FP8 codes [rows, K], scales [K/64][stride]
hipError_t launch_mx_quantize_act(const void* x, bool bf16, int64_t rows, int K, int64_t stride,
                                  uint8_t* codes, uint8_t* scales, hipStream_t st);
hipError_t launch_mx_ffn(const uint8_t* xq, const uint8_t* xs, int64_t x_stride,
                         const int32_t* offsets, int G, int64_t max_rows, int d, int F, int act,
                         const uint8_t* W13q, const uint8_t* W13s, const uint8_t* W2q,
                         const uint8_t* W2s, uint8_t* aq, uint8_t* aqs, int64_t a_stride,
                         float* out, hipStream_t st);

}  // namespace moe
