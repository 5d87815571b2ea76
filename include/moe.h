/*
 * moe.h — C ABI of the MI355X (gfx950) sparse mixture-of-experts layer.
 *
 * The layer: an FP32 router scores each of T tokens against E experts,
 * keeps the top-k (optionally after adding a selection-only bias), applies an
 * expert capacity with overflow left to the residual, permutes the kept
 * (token, expert) slots into expert-contiguous rows, runs each expert's FFN
 * and combines y_t = sum_j G_tj * E_idx_tj(x_t) (+ a shared expert).
 *
 * Sources (page title, section):
 *   "Mixture of Experts Explained" — "What is sparsity?" (weighted expert sum,
 *     softmax gating, KeepTopK, softmax over the kept logits); "MoEs and
 *     Transformers" (expert capacity, overflow through the residual);
 *     "Switch Transformers" (top-1 routing, capacity equation and factor,
 *     bf16 experts with a full-precision router); "Load balancing tokens for
 *     MoEs" and "Stabilizing training with router Z-loss" (router losses).
 *   "The Ultimate MoE Training Handbook" digest — "what MoE saves"
 *     (fine-grained experts), "the three hard parts" (FP32 routing,
 *     aux loss vs loss-free bias).
 *   Handbook news digest, "confirmed" bullets — sigmoid and sqrt(softplus)
 *     scoring, routing scale near sqrt(k), fixed-step bias update, shared
 *     experts.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (HBM of the current HIP device),
 *     row-major, owned by the caller.  The struct pointers (dims, opts,
 *     weights, saved, grads, stats) are HOST pointers read during the call.
 *   - Weights use the [out, in] layout: W13 [E, n_up, d] with n_up = 2F for
 *     SwiGLU (rows 0..F-1 gate, F..2F-1 up) and F for GELU; W2 [E, d, F];
 *     shared Ws13 [2*F_shared, d], Ws2 [d, F_shared].  The router weight is
 *     Wg [d, E] fp32 (z = x . Wg).
 *   - x, x_perm, W13, W2, Ws13, Ws2, h, a share one element type, opts.dtype
 *     (bf16 or fp32).  Router tensors, gates, expert outputs o, y, dx and all
 *     gradients are fp32.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call
 *     only enqueues work on it: there is no device-to-host synchronisation and
 *     the library allocates no memory (the layer calls create one internal
 *     stream and two events per caller stream, once; see moe_layer_fwd).
 *     Shape-dependent work (per-expert row counts) is read on the device.
 *   - `ws`/`ws_bytes` is caller-owned device scratch of at least
 *     moe_workspace_size() bytes, 256-byte aligned; contents need no
 *     initialisation and are clobbered.
 *   - Errors are returned synchronously as moe_status before anything is
 *     enqueued; MOE_ERR_HIP reports a failed launch.  T = 0 is a successful
 *     no-op (nothing is read, pointers may be NULL; moe_permute still
 *     zeroes offsets).  Results are bitwise deterministic for identical inputs.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status of every int-returning entry point: 0 on success, a negative code on
 * failure (moe_strerror names it). */
typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* null required pointer, bad size or option, misalignment */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but outside what the kernels implement (see limits) */
  MOE_ERR_WORKSPACE = -3,    /* ws_bytes below moe_workspace_size() */
  MOE_ERR_HIP = -4           /* a HIP launch or runtime call failed */
} moe_status;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1, MOE_SCORE_SQRT_SOFTPLUS = 2 } moe_score;
typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_GELU = 1 } moe_act;
typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype;

/* Problem statement of one layer call.
 * T tokens, hidden size d, E routed experts, k experts kept per token,
 * F routed expert width, F_shared width of the one shared SwiGLU expert (0 = none).
 * Limits: 1 <= k <= min(E, 16); 1 <= E <= 256; T*k < 2^31;
 * bf16: d, F and F_shared multiples of 128; fp32: d, F, F_shared multiples of 4. */
typedef struct { int64_t T, d, E, k, F, F_shared; } moe_dims;

/* How the k experts of a token are chosen.  Gates are always the router scores of
 * the chosen experts (renormalised and scaled as configured).
 * MOE_ROUTING_TOPK: the k largest selection scores (score + selection bias), ties to
 *   the lower expert index ("Mixture of Experts Explained", "What is sparsity?", KeepTopK).
 * MOE_ROUTING_UNIFORM: forced-uniform assignment, slot j of token t to expert
 *   (t*k + j) mod E, the balanced baseline of the Ultimate MoE Training Handbook digest
 *   ("the three hard parts", 2).
 * MOE_ROUTING_NOISY_TOPK: noisy top-k gating ("What is sparsity?", the H(x) equation):
 *   the logits become H = z + noise * softplus(x . W_noise) (moe_router_inputs.W_noise,
 *   .noise) and everything downstream (scores, selection, gates, losses) uses H.
 * MOE_ROUTING_RANDOM_SECOND: GShard's random routing ("MoEs and Transformers"): top-2
 *   (k = 2), the first expert always kept, the second kept iff uniform[t] <
 *   2 * s2 / (s1 + s2) of the two chosen scores; a skipped second slot is reported in
 *   topk_idx as E + expert (permute treats it as not routed; its gate stays in the
 *   normalisation).
 * MOE_ROUTING_HASH: experts fixed by the token id (Handbook news, DeepSeek-V4):
 *   slot j of token t to (fmix32(token_ids[t]) + j) mod E, fmix32 the 32-bit
 *   finalizer of MurmurHash3. */
typedef enum {
  MOE_ROUTING_TOPK = 0,
  MOE_ROUTING_UNIFORM = 1,
  MOE_ROUTING_NOISY_TOPK = 2,
  MOE_ROUTING_RANDOM_SECOND = 3,
  MOE_ROUTING_HASH = 4
} moe_routing;

/* Which slots an expert keeps when more than its capacity choose it.
 * MOE_PRIORITY_TOKEN: ascending token index.  MOE_PRIORITY_SLOT: every token's
 * first choice before any second choice, then by token (GShard's overflow
 * priority, "MoEs and Transformers"). */
typedef enum { MOE_PRIORITY_TOKEN = 0, MOE_PRIORITY_SLOT = 1 } moe_priority;

/* score: moe_score; act: moe_act; dtype: moe_dtype;
 * renorm != 0: kept gates are divided by their sum, then multiplied by gate_scale;
 * capacity_factor <= 0: no capacity limit, else C = ceil(cf * T * k / E) slots per expert;
 * aux_coef, z_coef: load-balance and z-loss coefficients (0 = not computed);
 * routing: moe_routing (0 = top-k); priority: moe_priority (0 = token order);
 * act_pair (bf16 only; 0 or 1): the routed experts' activation reaches the down
 *   projection as a pair of bf16 values, hi = bf16(a) and lo = bf16(a - hi)
 *   (about 16 significant bits instead of 8), at twice the down projection's
 *   work and activation bytes; the saved activation `a` is then [rows, 2F]
 *   (hi | lo per row) and the weight gradient of W2 uses hi.  Selective
 *   precision in the sense of "Switch Transformers": for layers whose gates
 *   are raw router probabilities (top-1 without renormalisation) the single
 *   bf16 rounding of a, scaled by the few largest gates, dominates the
 *   output error. */
typedef struct {
  int32_t score, act, dtype, renorm;
  float gate_scale, capacity_factor, aux_coef, z_coef;
  int32_t routing, priority;
  int32_t act_pair;
} moe_opts;

/* Per-call inputs of the variant routers (device pointers, fp32 unless noted).
 * Only the ones opts.routing uses are read; the rest may be NULL.  Random draws
 * are inputs so that a call is reproducible; moe_router_draws fills them on the
 * device from a seed and a per-call offset. */
typedef struct {
  const float* W_noise;      /* [d, E] noise projection (noisy top-k) */
  const float* noise;        /* [T, E] standard-normal draws (noisy top-k) */
  const float* uniform;      /* [T] draws in [0, 1) (random second expert) */
  const int32_t* token_ids;  /* [T] int32 token ids (hash routing) */
} moe_router_inputs;

typedef struct {
  const float* Wg;            /* [d, E] */
  const float* logit_offset;  /* nullable [E]: added to the logits (part of z) */
  const float* sel_bias;      /* nullable [E]: added to the scores for selection only */
  const void* W13;            /* [E, n_up, d] */
  const void* W2;             /* [E, d, F] */
  const void* Ws13;           /* [2*F_shared, d] when F_shared > 0 */
  const void* Ws2;            /* [d, F_shared]   when F_shared > 0 */
} moe_weights;

/* Forward state kept for the backward pass; every field is a caller-owned
 * device buffer of the given size.  moe_layer_fwd fills it when passed. */
typedef struct {
  int32_t* topk_idx;     /* [T, k] chosen experts, descending selection score */
  float* topk_gate;      /* [T, k] gates */
  float* logits;         /* [T, E] router logits z (offset included) */
  int32_t* counts;       /* [E] slots per expert before capacity */
  int32_t* offsets;      /* [E+1] first row of each expert; offsets[E] = kept rows R */
  int32_t* row_of_slot;  /* [T, k] row of each slot, -1 when dropped */
  int32_t* token_of_row; /* [T*k] token of each row (entries >= R unspecified) */
  void* x_perm;          /* [T*k, d] expert-contiguous copy of x */
  void* h;               /* [T*k, n_up] expert pre-activations */
  void* a;               /* [T*k, F] expert activations ([T*k, 2F] with opts.act_pair) */
  float* o;              /* [T*k, d] expert outputs */
  void* h_shared;        /* [T, 2*F_shared] (when F_shared > 0) */
  void* a_shared;        /* [T, F_shared]   (when F_shared > 0) */
  float* losses;         /* [2] aux loss, z-loss */
  float* noise_logits;   /* [T, E] x . W_noise (noisy top-k training only) */
} moe_saved;

typedef struct {
  float* dWg;    /* [d, E] */
  float* dW13;   /* [E, n_up, d] */
  float* dW2;    /* [E, d, F] */
  float* dWs13;  /* [2*F_shared, d] (when F_shared > 0) */
  float* dWs2;   /* [d, F_shared]   (when F_shared > 0) */
  float* dW_noise; /* [d, E] (noisy top-k) */
  /* Nullable: when set, the gradient with respect to the saved pre-activations
   * is written here (in their element type) instead of into the workspace:
   * dH [T*k, n_up] for the routed experts' h (rows past offsets[E] are not
   * written), dH_shared [T, 2*F_shared] for the shared expert's. */
  void* dH;
  void* dH_shared;
} moe_grads;

/* Router monitoring outputs, every field nullable. */
typedef struct {
  int32_t* counts;      /* [E] slots per expert before capacity */
  int32_t* n_dropped;   /* [1] slots dropped over capacity */
  float* losses;        /* [2] aux loss, z-loss */
  int32_t* n_nonfinite; /* [1] tokens with a non-finite router logit */
} moe_stats;

/* Expert capacity ("Switch Transformers", capacity equation, tokens read as
 * the T*k routed slots): *C = ceil(cf*T*k/E) computed in double from the fp32
 * factor, or -1 when capacity_factor <= 0.  Host only. */
int moe_capacity(const moe_dims* dims, const moe_opts* opts, int64_t* C);

/* Bytes of scratch any entry point below needs for these dims/opts, with the
 * backward pass (with_bwd != 0) or without.  Host only. */
int moe_workspace_size(const moe_dims* dims, const moe_opts* opts, int with_bwd, size_t* bytes);

/* Router ("What is sparsity?" gating equations; "Switch Transformers" top-1
 * and full-precision router; news digest: sigmoid / sqrt(softplus) scoring,
 * selection-only bias, routing scale).
 * z = x . Wg (+ logit_offset) with fp32 accumulation of exact products;
 * s = score(z); top-k of s + sel_bias by (value desc, index asc), NaN lowest;
 * gate_j = s[idx_j], renormalised over the kept experts if opts.renorm, times
 * gate_scale.  Outputs: topk_idx [T,k], topk_gate [T,k]; nullable: scores
 * [T,E] (s), logits [T,E] (z), counts [E] (pre-capacity histogram of the routed
 * slots), losses [2] (aux, z-loss; zero when the coefficient is 0).  ri: the
 * variant routers' inputs (nullable for top-k and uniform routing). */
int moe_route(const moe_dims* dims, const moe_opts* opts, const void* x, const float* Wg,
              const float* logit_offset, const float* sel_bias, int32_t* topk_idx,
              float* topk_gate, float* scores, float* logits, int32_t* counts, float* losses,
              const moe_router_inputs* ri, void* ws, size_t ws_bytes, void* stream);

/* Draws of the stochastic routers from a seed (the StandardNormal term of noisy
 * top-k gating, "What is sparsity?", the H(x) equation; the uniform of GShard's
 * random second expert, "MoEs and Transformers"), for moe_router_inputs.noise
 * and .uniform.  Counter-based, so any element can be recomputed alone and a
 * call is reproducible: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3", SC 2011) keyed by (seed, 0); stream s
 * (0 normals, 1 uniforms) draws block b from counter (b, offset, s, 0), and
 * element j takes word j % 4 of block j / 4.  uniform [T]: a word's top 24
 * bits times 2^-24, in [0, 1).  noise [T, E] row-major: words (0, 1) and (2, 3)
 * of a block give two normals each by the Box-Muller transform, r = sqrt(-2
 * ln(1 - u)), (r cos 2 pi v, r sin 2 pi v), u and v uniforms as above,
 * evaluated in fp32.  Use a new offset (e.g. the step number) per call.
 * Reads dims->T and dims->E only; noise and uniform are each nullable (both
 * NULL, or T = 0: nothing is launched).  MOE_ERR_INVALID_ARG for T < 0 or
 * E < 1; MOE_ERR_UNSUPPORTED for T*E > 2^40. */
int moe_router_draws(const moe_dims* dims, uint64_t seed, uint64_t offset, float* noise,
                     float* uniform, void* stream);

/* Dispatch ("MoEs and Transformers": expert capacity, overflow to the residual).
 * counts[e] = slots choosing e; expert e keeps its first C slots in ascending
 * token order (opts.priority = MOE_PRIORITY_SLOT: first choices first); rows are expert-contiguous from offsets (exclusive scan of
 * min(counts, C)); row_of_slot[t,j] = row or -1; token_of_row[row] = t;
 * x_perm[row] = x[t].  topk_idx entries outside [0,E) are ignored (dropped)
 * and never index memory. */
int moe_permute(const moe_dims* dims, const moe_opts* opts, const void* x,
                const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                int32_t* row_of_slot, int32_t* token_of_row, void* x_perm,
                void* ws, size_t ws_bytes, void* stream);

/* moe_permute without a workspace, for callers that cannot allocate device
 * memory or pass scratch (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * moe_permute minus ws/ws_bytes.  Its scratch (the dispatch's per-block
 * histogram table, ceil(T*k/1024) x E int32 rounded up to 256 bytes) lives in
 * a 1 MiB device array inside the library, one per GPU, held until the
 * process ends; larger problems (for instance E = 256 with T*k above 1048576
 * slots) return MOE_ERR_UNSUPPORTED before anything is enqueued.  The array keeps the last call's contents and needs no clearing.
 * Calls that overlap on one GPU (concurrent streams, host threads) share the
 * array and race: serialise them.  Allocates nothing and calls no allocating
 * routine. */
int moe_permute_noalloc(const moe_dims* dims, const moe_opts* opts, const void* x,
                        const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                        int32_t* row_of_slot, int32_t* token_of_row, void* x_perm,
                        void* stream);

/* Expert FFNs over expert-contiguous rows (the "Making MoEs go brrr" grouped
 * computation): for group g, rows offsets[g]..offsets[g+1]-1 of x_perm go
 * through act(x W13[g]^T) W2[g]^T with width F (act: SwiGLU with the gate/up
 * projections fused, or exact GELU).  out [max_rows, d] fp32.  max_rows is an
 * upper bound of offsets[n_groups] used to size the launch.  h_save
 * [max_rows, n_up] and a_save [max_rows, F] ([max_rows, 2F] with
 * opts.act_pair) (nullable) receive the pre-activation and the activation in
 * the x element type. */
int moe_expert_ffn(const moe_dims* dims, const moe_opts* opts, int64_t n_groups,
                   int64_t max_rows, int64_t F, const void* x_perm, const int32_t* offsets,
                   const void* W13, const void* W2, void* h_save, void* a_save, float* out,
                   void* ws, size_t ws_bytes, void* stream);

/* Combine ("What is sparsity?", y = sum_i G(x)_i E_i(x)): y[t] = sum over
 * kept slots j, in slot order, of topk_gate[t,j] * out_perm[row_of_slot[t,j]]
 * plus shared_out[t] (nullable).  A fully dropped token gets y = shared or 0. */
int moe_combine(const moe_dims* dims, const float* out_perm, const int32_t* row_of_slot,
                const float* topk_gate, const float* shared_out, float* y, void* stream);

/* Whole forward: route, dispatch, routed expert FFNs, shared expert, combine.
 * y [T,d] fp32 (the caller adds the residual x).  ri, saved and stats nullable
 * (ri as for moe_route).
 * Streams (moe_layer_fwd and moe_layer_bwd): branches that do not depend on
 * each other (the shared expert; in the backward also the router gradients and
 * the routed experts' dW2) run
 * on an internal stream, forked from `stream` and joined back to it with
 * events before the call returns, so every result is ordered on `stream` as
 * for a single-stream call.  There is one internal stream (with its two events)
 * per (device, caller stream): it is created on the first layer call made on
 * that caller stream and kept until the process ends, so calls on different
 * caller streams do not wait on each other.  This is the library's only state;
 * it holds no data. */
int moe_layer_fwd(const moe_dims* dims, const moe_opts* opts, const moe_weights* w,
                  const moe_router_inputs* ri, const void* x, float* y, moe_saved* saved,
                  moe_stats* stats, void* ws, size_t ws_bytes, void* stream);

/* Whole backward of J = <dy, y> + L_aux + L_z from the state saved by
 * moe_layer_fwd.  Routing decisions and load fractions are constants; the
 * selection bias and logit offset get no gradient.  dx [T,d] fp32; grads
 * overwritten (not accumulated), fp32.  Noisy top-k also yields
 * dW_noise = x^T (dH * noise * sigmoid(x . W_noise)) and the matching dx term,
 * from saved.noise_logits and ri (W_noise, noise). */
int moe_layer_bwd(const moe_dims* dims, const moe_opts* opts, const moe_weights* w,
                  const moe_router_inputs* ri, const void* x, const moe_saved* saved,
                  const float* dy, float* dx, moe_grads* grads, void* ws, size_t ws_bytes,
                  void* stream);

/* Fixed-step loss-free bias update (news digest: the fixed-step baseline;
 * handbook digest: loss-free bias): bias[e] += gamma * sign(target - counts[e]),
 * sign(0) = 0; target is normally T*k/E. */
int moe_bias_update(const int32_t* counts, float* bias, int64_t E, float target, float gamma,
                    void* stream);

/* Quantile balancing, step 1 (Ultimate MoE Training Handbook news, Kimi K3: the
 * selection bias solved from score histograms summed over GPUs instead of fixed
 * steps).  scores [T, E] fp32 (moe_route's scores output); hist [E, nbins] int32,
 * overwritten: hist[e][b] = tokens t with bin(scores[t,e]) = b, bin =
 * floor((s - lo) * (nbins / (hi - lo))) in fp32 clamped to [0, nbins-1]; NaN
 * scores are not counted.  Requires E <= 256, 1 <= nbins <= 65536, lo < hi. */
int moe_score_histogram(const float* scores, int64_t T, int64_t E, float lo, float hi,
                        int32_t nbins, int32_t* hist, void* stream);

/* Quantile balancing, step 2: bias[e] = mean(q) - q[e], where q[e] is the score
 * above which `target` (normally T*k/E) tokens of expert e lie, read from its
 * histogram (bins walked from the top, linear within the bin reaching the
 * count; lo when the expert has fewer tokens).  The result is a selection-only
 * bias (moe_weights.sel_bias) that puts every expert's target-th largest biased
 * score at the same level. */
int moe_bias_from_histogram(const int32_t* hist, int64_t E, int32_t nbins, float lo, float hi,
                            float target, float* bias, void* stream);

/* Router monitoring (handbook explainer, "router and load balancing": max expert
 * load, drop rate, spread of expert utilisation; handbook digest: a layer's
 * largest expert output norm against the median).  counts [E] (pre-capacity),
 * n_dropped [1] nullable; out_perm [R, d] fp32 and offsets [E+1] (nullable
 * together) give expert_norm [E] (required with them) = mean L2 norm of each
 * expert's output rows.  report [5] fp32 on the device: max/mean load,
 * population std/mean of the loads, dropped/routed slots, max/median expert
 * norm over the non-empty experts (0 without out_perm), empty experts. */
int moe_router_report(int64_t E, int64_t d, const int32_t* counts, const int32_t* n_dropped,
                      const float* out_perm, const int32_t* offsets, float* expert_norm,
                      float* report, void* stream);

/* MXFP4 routed experts for inference (Ultimate MoE Training Handbook news: Kimi K3
 * quantises its routed experts to MXFP4).  Formats of the OCP Microscaling
 * specification: FP4 E2M1 and FP8 E4M3 elements with E8M0 block scales
 * (2^(code-127)); a block's shared exponent is floor(log2(max|v|)) minus the
 * element type's largest exponent (2 for E2M1, 8 for E4M3), elements v*2^-X
 * rounded to nearest even and saturated (6, 448).
 * Layouts are k-block-major (a 64-k step of a tile is one contiguous run).
 * Weights: one scale per 32 consecutive k; codes [G][K/64][N][32] bytes (two
 * E2M1 values per byte, low nibble = even k), scales [G][K/32][N].
 * Activations: one scale per 64 consecutive k (what the FP8 x FP4 matrix
 * instruction pairs per lane); codes [K/64][stride][64] bytes, scales
 * [K/64][stride], stride >= rows shared by both (moe_expert_ffn_mx: stride a
 * multiple of 4 and >= rows + 4, the scale arrays 4-byte aligned).
 *
 * Errors (synchronous): MOE_ERR_INVALID_ARG for null or non-16-byte-aligned
 * inputs and codes, K not a multiple of 64, stride < rows, dtype other than
 * bf16/fp32.
 *
 * moe_mx_quantize_weights: w [G, N, K] in opts.dtype (bf16 or fp32), K % 64 == 0. */
int moe_mx_quantize_weights(const moe_opts* opts, const void* w, int64_t G, int64_t N, int64_t K,
                            uint8_t* codes, uint8_t* scales, void* stream);

/* moe_mx_quantize_act: x [rows, K] in opts.dtype -> FP8 codes and scales (layout above). */
int moe_mx_quantize_act(const moe_opts* opts, const void* x, int64_t rows, int64_t K,
                        int64_t stride, uint8_t* codes, uint8_t* scales, void* stream);

/* moe_expert_ffn_mx: the routed expert FFN of moe_expert_ffn with FP8 activations
 * and MXFP4 weights: h = x W13^T, a = act(h) (SwiGLU with fused gate/up, or exact
 * GELU), a quantised to FP8 in the same pass (aq [F/64][a_stride][64], aqs
 * [F/64][a_stride]: the activation layout above), out = a W2^T [max_rows, d]
 * fp32.  xq/xs: the rows' FP8 activations (row stride x_stride); W13q/W13s,
 * W2q/W2s: MXFP4 weights of [G, n_up, d] and [G, d, F].  Requires d and F
 * multiples of 256; x_stride, a_stride multiples of 4 and >= max_rows + 4.
 * Allocates nothing. */
int moe_expert_ffn_mx(const moe_dims* dims, const moe_opts* opts, int64_t n_groups,
                      int64_t max_rows, int64_t F, const uint8_t* xq, const uint8_t* xs,
                      int64_t x_stride, const int32_t* offsets, const uint8_t* W13q,
                      const uint8_t* W13s, const uint8_t* W2q, const uint8_t* W2s, uint8_t* aq,
                      uint8_t* aqs, int64_t a_stride, float* out, void* stream);

/* Static text for a moe_status value. */
const char* moe_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
