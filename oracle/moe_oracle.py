"""Plain, slow float64 CPU oracle of the sparse MoE layer.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP path (no kernels, headers, helpers or constants) and never imports
the ``top_routing_expert_amd`` package.

Every step is written out in NumPy float64 from its definition on the pages:

  [MoE-Explained]  "Mixture of Experts Explained" (Hugging Face blog; the copy
                   read is a Chinese translation).  Sections used: "What is
                   sparsity?" (the weighted expert sum, softmax gating,
                   KeepTopK, softmax over the kept logits), "Load balancing
                   tokens for MoEs" (auxiliary loss), "MoEs and Transformers"
                   (expert capacity, overflow through the residual), "Switch
                   Transformers" (top-1 routing, the expert-capacity equation,
                   capacity factor, full-precision router), "Stabilizing
                   training with router Z-loss".
  [Handbook-digest] digest of "The Ultimate MoE Training Handbook": section
                   "what MoE saves" (64 experts / top-8 / width 1024 example)
                   and "the three hard parts" (FP32 router because close
                   scores flip; aux loss vs loss-free bias).
  [Handbook-news]  news digest "Hugging Face releases a 30k-word free MoE
                   training handbook", "confirmed" bullets: sigmoid and
                   sqrt(softplus) scoring, routing scale near sqrt(k), the
                   fixed-step bias update, shared experts.

Where the pages leave a step open, the reading taken is stated at the function
and listed in the design notes:
  * expert capacity counts routed slots: C = ceil(CF * T * k / E); CF is an
    fp32 value; CF <= 0 means no limit;
  * within an expert, tokens are kept in ascending token order; a slot beyond
    capacity is dropped on its own (the token keeps its other slots) and the
    surviving gates are not renormalised; a dropped slot adds 0 to y (the
    caller's residual carries the token);
  * ties in the selection score go to the lower expert index; NaN ranks lowest;
  * top-1 without renormalisation uses the raw softmax probability as gate;
  * aux loss  L_aux = aux_coef * E * sum_e f_e * P_e with f_e = count_e/(T*k)
    (pre-drop counts) and P_e = mean_t of the scores normalised over E;
    z-loss    L_z = z_coef * mean_t (logsumexp_e z_te)^2 on the router logits
    (including any logit offset);
  * GELU is the exact erf form; expert linears have no biases;
  * the loss-free bias update is b_e += gamma * sign(T*k/E - count_e).

Array conventions (row-major): x [T,d]; Wg [d,E] (z = x Wg); W13 [E, n_up, d]
(rows 0..F-1 gate, F..2F-1 up for SwiGLU; [E,F,d] for GELU); W2 [E,d,F];
shared Ws13 [2Fs,d], Ws2 [d,Fs].
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

F64 = np.float64
SCORES = ("softmax", "sigmoid", "sqrt_softplus")
NEAR_TIE_REL = 1e-5

__all__ = [
    "capacity", "router_logits", "score", "select_topk", "near_tie_flags", "gates",
    "logsumexp_rows", "router_losses", "route", "dispatch", "permute", "silu", "gelu",
    "expert_ffn", "shared_expert", "combine", "bias_update", "layer_fwd", "layer_bwd",
    "router_bwd", "expert_bwd", "uniform_assignment", "hash_assignment", "fmix32", "softplus",
    "score_histogram", "quantile_bias", "load_report", "expert_output_norms",
    "e2m1_decode", "e4m3_decode", "e2m1_encode", "e4m3_encode", "mx_quantize", "mx_dequantize",
    "expert_ffn_mx", "philox4x64", "uniform24", "box_muller", "router_draws",
    "NEAR_TIE_REL",
]


# ---------------------------------------------------------------------------
# Capacity
# ---------------------------------------------------------------------------
def capacity(T: int, E: int, k: int, capacity_factor: float):
    """Expert capacity [MoE-Explained, "Switch Transformers", capacity equation].

    The equation divides the tokens of a batch evenly over the experts and
    scales by the capacity factor.  "Tokens" is read as the T*k routed slots
    (equal to the printed form at k=1, where the equation is stated) and
    rounded up.  The factor is an fp32 value.  Returns None for no limit.
    """
    cf = float(np.float32(capacity_factor))
    if cf <= 0.0:
        return None
    return int(math.ceil(cf * T * k / E))


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------
def router_logits(x, Wg, offset=None):
    """z = x . W_g (+ per-expert offset) [MoE-Explained, "What is sparsity?",
    softmax gating equation], in float64."""
    z = np.asarray(x, F64) @ np.asarray(Wg, F64)
    if offset is not None:
        z = z + np.asarray(offset, F64)[None, :]
    return z


def score(z, kind: str):
    """Router scoring function over the E logits of each token.

    softmax: [MoE-Explained, "What is sparsity?"]; sigmoid and sqrt(softplus):
    [Handbook-news, "confirmed" bullets on router scoring].
    """
    z = np.asarray(z, F64)
    if kind == "softmax":
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        return e / e.sum(axis=1, keepdims=True)
    if kind == "sigmoid":
        return 1.0 / (1.0 + np.exp(-z))
    if kind == "sqrt_softplus":
        softplus = np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))
        return np.sqrt(softplus)
    raise ValueError(kind)


def select_topk(sel, k: int):
    """KeepTopK [MoE-Explained, "What is sparsity?", KeepTopK equation].

    Returns idx [T,k]: the k largest selection scores per token in descending
    order, ties to the lower expert index (a stable sort), NaN last.
    """
    sel = np.asarray(sel, F64)
    order = np.argsort(-sel, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def near_tie_flags(sel, k: int, rel: float = NEAR_TIE_REL):
    """Tokens whose selection could flip under sub-1e-5 relative rounding.

    ``boundary``: the k-th and (k+1)-th largest selection scores differ by less
    than ``rel`` * max(|a|,|b|) (the kept set is ambiguous).  ``order``: two
    adjacent kept scores are that close (the slot order is ambiguous).
    """
    sel = np.asarray(sel, F64)
    T, E = sel.shape
    srt = -np.sort(-sel, axis=1)
    def close(a, b):
        return np.abs(a - b) < rel * np.maximum(np.abs(a), np.abs(b))
    boundary = close(srt[:, k - 1], srt[:, k]) if k < E else np.zeros(T, bool)
    order = np.zeros(T, bool)
    for j in range(k - 1):
        order |= close(srt[:, j], srt[:, j + 1])
    return boundary, order


def gates(s, idx, renorm: bool, gate_scale: float):
    """Gates of the kept experts.

    g_j = s[idx_j] (the selection bias is not part of the gate); renormalising
    over the kept experts reproduces Softmax(KeepTopK(z)) for softmax scoring
    [MoE-Explained, "What is sparsity?", last gating equation]; top-1 without
    renormalisation keeps the raw probability [MoE-Explained, "Switch
    Transformers"]; the result is multiplied by the routing scale
    [Handbook-news, routing scale near sqrt(k)].
    """
    g = np.take_along_axis(np.asarray(s, F64), idx, axis=1)
    if renorm:
        g = g / g.sum(axis=1, keepdims=True)
    return g * float(np.float32(gate_scale))


def logsumexp_rows(z):
    z = np.asarray(z, F64)
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def router_losses(z, s, counts, k: int, aux_coef: float, z_coef: float):
    """Auxiliary load-balance loss and router z-loss.

    [MoE-Explained, "Load balancing tokens for MoEs" and "Switch
    Transformers"] name the load-balance loss that pushes experts toward equal
    importance and equal token counts; [MoE-Explained, "Stabilizing training
    with router Z-loss"] names the penalty on large logits.  Formulas (the
    pages give none): L_aux = aux_coef * E * sum_e f_e P_e with f_e the
    fraction of routed slots sent to e (pre-drop) and P_e the mean over tokens
    of the scores normalised over E; L_z = z_coef * mean_t logsumexp(z_t)^2.
    """
    s = np.asarray(s, F64)
    T, E = s.shape
    p_hat = s / s.sum(axis=1, keepdims=True)
    P = p_hat.mean(axis=0)
    f = np.asarray(counts, F64) / (T * k)
    aux = float(np.float32(aux_coef)) * E * float(np.sum(f * P))
    lse = logsumexp_rows(z)
    zl = float(np.float32(z_coef)) * float(np.mean(lse * lse))
    return aux, zl


def uniform_assignment(T: int, E: int, k: int):
    """Forced-uniform routing [Handbook digest, "the three hard parts", 2: the
    balanced-routing baseline that runs about 1.5x faster than learned
    routing]: slot j of token t goes to expert (t*k + j) mod E, so every expert
    receives T*k/E slots (when E divides T*k) and a token's k experts are
    distinct (k <= E)."""
    t = np.arange(T, dtype=np.int64)[:, None]
    j = np.arange(k, dtype=np.int64)[None, :]
    return (t * k + j) % E


def fmix32(v):
    """The 32-bit finalizer of Appleby's MurmurHash3 (public domain): xor-shift
    16, multiply by 0x85ebca6b, xor-shift 13, multiply by 0xc2b2ae35, xor-shift
    16, all modulo 2^32.  A bijection of the 32-bit integers."""
    h = np.asarray(v).astype(np.uint64) & 0xFFFFFFFF
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & 0xFFFFFFFF
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & 0xFFFFFFFF
    h ^= h >> 16
    return h


def hash_assignment(token_ids, E: int, k: int):
    """Token-id hash routing [Handbook news, DeepSeek-V4: the first MoE layers
    pick experts by a fixed hash of the token id]: the token's experts are the
    k consecutive experts (fmix32(id) + j) mod E, j = 0..k-1 (distinct for
    k <= E; the same for every occurrence of the id)."""
    h = fmix32(np.asarray(token_ids).astype(np.int64) & 0xFFFFFFFF).astype(np.int64)
    return (h[:, None] + np.arange(k, dtype=np.int64)[None, :]) % E


def softplus(v):
    return np.logaddexp(0.0, np.asarray(v, F64))


def route(x, Wg, k, score_kind, renorm, gate_scale, offset=None, sel_bias=None,
          aux_coef=0.0, z_coef=0.0, routing="topk", W_noise=None, noise=None, uniform=None,
          token_ids=None):
    """The FP32-router step of the layer in float64 [Handbook-digest, "the three
    hard parts", 1: routing in full precision].  Returns a dict with z, s, sel,
    idx [T,k], g [T,k], active [T,k], counts [E] (pre-drop, active slots),
    losses and near-tie flags.

    routing:
      "topk"      KeepTopK of the selection scores;
      "uniform"   the forced-uniform assignment;
      "noisy_topk" noisy top-k gating [MoE-Explained, "What is sparsity?", the
                  H(x) equation]: the logits become H = z + noise * softplus(x W_noise)
                  (noise: the caller's standard-normal draws [T,E]); scores,
                  selection, gates and losses all use H (returned as z; the
                  projection x W_noise as zn);
      "gshard"    random routing [MoE-Explained, "MoEs and Transformers", GShard]:
                  top-2, the first expert always kept, the second kept iff
                  uniform[t] < 2 * g2 / (g1 + g2) (probability proportional to its
                  weight, 1 when the two weights are equal); a skipped slot is
                  inactive (no output, not counted) but stays in the gate
                  normalisation;
      "hash"      the token-id hash assignment.
    Gates are always the scores of the chosen experts (renormalised and scaled
    as configured)."""
    z = router_logits(x, Wg, offset)
    zn = None
    if routing == "noisy_topk":
        zn = np.asarray(x, F64) @ np.asarray(W_noise, F64)
        z = z + np.asarray(noise, F64) * softplus(zn)
    s = score(z, score_kind)
    sel = s + (np.asarray(sel_bias, F64)[None, :] if sel_bias is not None else 0.0)
    T, E = z.shape
    if routing == "uniform":
        idx = uniform_assignment(T, E, k)
    elif routing == "hash":
        idx = hash_assignment(token_ids, E, k)
    elif routing in ("topk", "noisy_topk", "gshard"):
        if routing == "gshard" and k != 2:
            raise ValueError("random routing is a top-2 scheme")
        idx = select_topk(sel, k)
    else:
        raise ValueError(f"unknown routing {routing!r}")
    g = gates(s, idx, renorm, gate_scale)
    active = np.ones((T, k), bool)
    if routing == "gshard":
        s1 = np.take_along_axis(s, idx[:, :1], axis=1)[:, 0]
        s2 = np.take_along_axis(s, idx[:, 1:], axis=1)[:, 0]
        active[:, 1] = np.asarray(uniform, F64) < 2.0 * s2 / (s1 + s2)
    counts = np.bincount(idx[active], minlength=E).astype(np.int64)
    aux, zl = router_losses(z, s, counts, k, aux_coef, z_coef)
    boundary, order = near_tie_flags(sel, k)
    if routing in ("uniform", "hash"):
        boundary, order = np.zeros_like(boundary), np.zeros_like(order)
    return dict(z=z, zn=zn, s=s, sel=sel, idx=idx, g=g, active=active, counts=counts, aux=aux,
                zloss=zl, near_tie=boundary, near_tie_order=order)


# ---------------------------------------------------------------------------
# Dispatch: capacity, drop set, expert-contiguous permutation
# ---------------------------------------------------------------------------
def dispatch(idx, E: int, C, active=None, priority: str = "token"):
    """Group routed slots by expert [MoE-Explained, "MoEs and Transformers",
    expert capacity and overflow].

    counts_e = active slots that chose e (pre-drop); each expert keeps its
    first C slots in ascending token order (priority "token"), or with every
    token's first choices ahead of any second choice (priority "slot": order by
    slot, then token; GShard's overflow priority in the same section); kept
    rows are laid out expert by expert: row = offsets[e] + position, offsets =
    exclusive scan of min(counts, C).  Inactive slots are skipped.
    Returns counts [E], offsets [E+1], row_of_slot [T,k] (-1 = dropped or
    inactive) and token_of_row [T*k] (-1 past the last kept row).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    act = np.ones((T, k), bool) if active is None else np.asarray(active, bool)
    counts = np.zeros(E, np.int64)
    for e in range(E):
        counts[e] = int(np.count_nonzero((idx == e) & act))
    kept = counts.copy() if C is None else np.minimum(counts, C)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(kept)
    row_of_slot = np.full((T, k), -1, np.int64)
    token_of_row = np.full(T * k, -1, np.int64)
    for e in range(E):
        if priority == "slot":
            js, ts = np.nonzero(((idx == e) & act).T)   # slot-major, then ascending token
        else:
            ts, js = np.nonzero((idx == e) & act)       # row-major: ascending token index
        n = int(kept[e])
        rows = offsets[e] + np.arange(n)
        row_of_slot[ts[:n], js[:n]] = rows
        token_of_row[rows] = ts[:n]
    return counts, offsets, row_of_slot, token_of_row


def permute(x, token_of_row, R: int):
    """x_perm[r] = x[token_of_row[r]] for the R kept rows."""
    return np.asarray(x, F64)[np.asarray(token_of_row[:R])]


# ---------------------------------------------------------------------------
# Experts
# ---------------------------------------------------------------------------
def silu(v):
    return v / (1.0 + np.exp(-v))


def gelu(v):
    """Exact (erf) GELU."""
    return 0.5 * v * (1.0 + erf(v / math.sqrt(2.0)))


def _ffn(X, W13e, W2e, act):
    X = np.asarray(X, F64)
    h = X @ np.asarray(W13e, F64).T
    if act == "swiglu":
        F = h.shape[1] // 2
        a = silu(h[:, :F]) * h[:, F:]
    elif act == "gelu":
        a = gelu(h)
    else:
        raise ValueError(act)
    return h, a, a @ np.asarray(W2e, F64).T


def expert_ffn(x_perm, offsets, W13, W2, act: str, keep_hidden: bool = False):
    """Each expert is an FFN [MoE-Explained, "What is MoE?": experts are FFNs]
    applied to its contiguous rows: SwiGLU a = silu(x Wg^T) * (x Wu^T) or GELU
    a = gelu(x W1^T); o = a W2^T.  Returns o [R,d] (and h, a if asked)."""
    x_perm = np.asarray(x_perm, F64)
    G = len(offsets) - 1
    R = int(offsets[-1])
    d = W2.shape[1]
    o = np.zeros((R, d), F64)
    hs, as_ = [], []
    for e in range(G):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            hs.append(np.zeros((0, W13.shape[1]))); as_.append(np.zeros((0, W2.shape[2])))
            continue
        h, a, oe = _ffn(x_perm[r0:r1], W13[e], W2[e], act)
        o[r0:r1] = oe
        if keep_hidden:
            hs.append(h); as_.append(a)
    if keep_hidden:
        return o, hs, as_
    return o


def shared_expert(x, Ws13, Ws2, keep_hidden: bool = False):
    """Always-on SwiGLU expert applied to every token with gate 1
    [Handbook-news, "confirmed" bullets on shared experts]."""
    h, a, o = _ffn(x, Ws13, Ws2, "swiglu")
    return (o, h, a) if keep_hidden else o


def combine(o, row_of_slot, g, shared_out=None):
    """y_t = sum over kept slots j of g_tj * E_idx(x_t) [MoE-Explained, "What is
    sparsity?", the weighted expert sum]; experts not kept (gate 0, or dropped
    over capacity) contribute nothing; plus the shared expert's output."""
    o = np.asarray(o, F64)
    T, k = row_of_slot.shape
    y = np.zeros((T, o.shape[1]), F64)
    for j in range(k):
        kept = row_of_slot[:, j] >= 0
        y[kept] += np.asarray(g, F64)[kept, j, None] * o[row_of_slot[kept, j]]
    if shared_out is not None:
        y += np.asarray(shared_out, F64)
    return y


def bias_update(counts, bias, T: int, k: int, gamma: float):
    """Fixed-step loss-free selection-bias update [Handbook-news, "confirmed":
    the fixed-step update; Handbook-digest, "the three hard parts", 2]:
    b_e += gamma * sign(T*k/E - count_e), sign(0) = 0."""
    counts = np.asarray(counts, F64)
    E = counts.shape[0]
    return np.asarray(bias, F64) + float(np.float32(gamma)) * np.sign(T * k / E - counts)


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------
def layer_fwd(p, inp, keep_hidden: bool = False):
    """Forward pass of the layer for preset ``p`` on inputs ``inp`` (the dict
    from the seeded generator).  Steps in order: route, capacity, dispatch,
    permute, expert FFN, shared expert, combine."""
    r = route(inp["x"], inp["Wg"], p.k, p.score, p.renorm, p.gate_scale,
              inp.get("offset"), inp.get("sel_bias"), p.aux_coef, p.z_coef, p.routing,
              inp.get("W_noise"), inp.get("noise"), inp.get("uniform"), inp.get("token_ids"))
    C = capacity(p.T, p.E, p.k, p.capacity_factor)
    counts, offsets, row_of_slot, token_of_row = dispatch(r["idx"], p.E, C, r["active"],
                                                          p.priority)
    R = int(offsets[-1])
    x_perm = permute(inp["x"], token_of_row, R)
    res = expert_ffn(x_perm, offsets, inp["W13"], inp["W2"], p.act, keep_hidden)
    o, hs, as_ = res if keep_hidden else (res, None, None)
    shared = None
    sh = None
    if p.F_shared > 0:
        sh = shared_expert(inp["x"], inp["Ws13"], inp["Ws2"], keep_hidden=True)
        shared = sh[0]
    y = combine(o, row_of_slot, r["g"], shared)
    out = dict(r, C=C, counts=counts, offsets=offsets, row_of_slot=row_of_slot,
               token_of_row=token_of_row, R=R, x_perm=x_perm, o=o, shared_out=shared, y=y)
    if keep_hidden:
        out.update(h=hs, a=as_, shared_h=None if sh is None else sh[1],
                   shared_a=None if sh is None else sh[2])
    return out


def expert_bwd(X, h, a, W13e, W2e, dO, act, dH_in=None, keep_dH=False):
    """Backward of o = act(X W13^T) W2^T for one expert; returns dX, dW13, dW2
    (and the pre-activation gradient dH when keep_dH).  With dH_in given, dX
    and dW13 are formed from it instead of from the dH computed here (each
    product checked on another implementation's own dH)."""
    dA = dO @ np.asarray(W2e, F64)
    dW2 = dO.T @ a
    if act == "swiglu":
        F = h.shape[1] // 2
        hg, hu = h[:, :F], h[:, F:]
        sg = 1.0 / (1.0 + np.exp(-hg))
        dsilu = sg * (1.0 + hg * (1.0 - sg))
        dH = np.concatenate([dA * hu * dsilu, dA * (hg * sg)], axis=1)
    else:
        phi = np.exp(-0.5 * h * h) / math.sqrt(2.0 * math.pi)
        Phi = 0.5 * (1.0 + erf(h / math.sqrt(2.0)))
        dH = dA * (Phi + h * phi)
    dHu = dH if dH_in is None else np.asarray(dH_in, F64)
    dX = dHu @ np.asarray(W13e, F64)
    dW13 = dHu.T @ np.asarray(X, F64)
    return (dX, dW13, dW2, dH) if keep_dH else (dX, dW13, dW2)


def router_bwd(p, s, z, idx, counts, dg):
    """Gradient of <dy, y> + L_aux + L_z with respect to the router logits z,
    given dg [T,k] = d<dy,y>/d(gate) of the kept gates.  The gradient reaches
    the router only through the kept gates and the two losses; idx, the
    pre-drop counts (hence f_e) and the selection bias are constants."""
    s = np.asarray(s, F64)
    z = np.asarray(z, F64)
    dg = np.asarray(dg, F64)
    T, E = s.shape
    k = idx.shape[1]
    # gates -> scores
    scale = float(np.float32(p.gate_scale))
    ssel = np.take_along_axis(s, idx, axis=1)
    if p.renorm:
        S = ssel.sum(axis=1, keepdims=True)
        ghat = ssel / S
        dsel = scale / S * (dg - np.sum(dg * ghat, axis=1, keepdims=True))
    else:
        dsel = scale * dg
    ds = np.zeros((T, E), F64)
    np.put_along_axis(ds, idx, dsel, axis=1)      # idx rows are distinct experts
    aux_coef = float(np.float32(p.aux_coef))
    if aux_coef != 0.0:
        f = np.asarray(counts, F64) / (T * k)
        c = aux_coef * E * f / T                   # dL_aux / dp_hat_te
        Ssum = s.sum(axis=1, keepdims=True)
        p_hat = s / Ssum
        ds += (c[None, :] - np.sum(p_hat * c[None, :], axis=1, keepdims=True)) / Ssum
    # scores -> logits
    if p.score == "softmax":
        dz = s * (ds - np.sum(ds * s, axis=1, keepdims=True))
    elif p.score == "sigmoid":
        dz = ds * s * (1.0 - s)
    else:
        sig = 1.0 / (1.0 + np.exp(-z))
        safe = np.where(s > 0, s, 1.0)
        dz = ds * np.where(s > 0, sig / (2.0 * safe), 0.5 * np.exp(0.5 * z))
    z_coef = float(np.float32(p.z_coef))
    if z_coef != 0.0:
        lse = logsumexp_rows(z)
        sm = np.exp(z - lse[:, None])
        dz += 2.0 * z_coef / T * lse[:, None] * sm
    return dz


def layer_bwd(p, inp, fwd, dy):
    """Gradients of J = <dy, y> + L_aux + L_z, by the chain rule.

    Routing decisions (idx, drops) and the load fractions f_e are piecewise
    constant and carry no gradient; the selection bias and the logit offset get
    none (the gradient reaches the router only through the kept gates
    [Handbook explainer, "router and load balancing": top-k selection is not
    differentiable]).  Returns dx [T,d], dWg [d,E], dW13, dW2, dWs13, dWs2.
    """
    dy = np.asarray(dy, F64)
    x = np.asarray(inp["x"], F64)
    T, d = x.shape
    E, k = p.E, p.k
    row_of_slot, g, o = fwd["row_of_slot"], fwd["g"], fwd["o"]
    R = fwd["R"]
    # combine backward
    dO = np.zeros((R, d), F64)
    dg = np.zeros((T, k), F64)
    for j in range(k):
        kept = row_of_slot[:, j] >= 0
        rows = row_of_slot[kept, j]
        dO[rows] = g[kept, j, None] * dy[kept]
        dg[kept, j] = np.sum(dy[kept] * o[rows], axis=1)
    # expert backward
    offsets = fwd["offsets"]
    dXp = np.zeros((R, d), F64)
    dW13 = np.zeros(inp["W13"].shape, F64)
    dW2 = np.zeros(inp["W2"].shape, F64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        dX, dW13[e], dW2[e] = expert_bwd(fwd["x_perm"][r0:r1], fwd["h"][e], fwd["a"][e],
                                       inp["W13"][e], inp["W2"][e], dO[r0:r1], p.act)
        dXp[r0:r1] = dX
    dx = np.zeros((T, d), F64)
    for j in range(k):
        kept = row_of_slot[:, j] >= 0
        dx[kept] += dXp[row_of_slot[kept, j]]
    dWs13 = dWs2 = None
    if p.F_shared > 0:
        dxs, dWs13, dWs2 = expert_bwd(x, fwd["shared_h"], fwd["shared_a"], inp["Ws13"],
                                    inp["Ws2"], dy, "swiglu")
        dx += dxs
    dz = router_bwd(p, fwd["s"], fwd["z"], fwd["idx"], fwd["counts"], dg)
    dWg = x.T @ dz
    dx += dz @ np.asarray(inp["Wg"], F64).T
    dW_noise = None
    if p.routing == "noisy_topk":
        # H = z + noise * softplus(zn): dH/dzn = noise * sigmoid(zn)
        dzn = dz * np.asarray(inp["noise"], F64) / (1.0 + np.exp(-fwd["zn"]))
        dW_noise = x.T @ dzn
        dx += dzn @ np.asarray(inp["W_noise"], F64).T
    return dict(dx=dx, dWg=dWg, dW13=dW13, dW2=dW2, dWs13=dWs13, dWs2=dWs2, dW_noise=dW_noise,
                dO=dO, dg=dg, dz=dz, dXp=dXp)


# ---------------------------------------------------------------------------
# Load balance from score histograms; router monitoring
# ---------------------------------------------------------------------------
def score_histogram(s, lo: float, hi: float, nbins: int):
    """Per-expert histogram of the scores s [T,E] over nbins equal bins of
    [lo, hi): bin = floor((s - lo) * (nbins / (hi - lo))) clamped to
    [0, nbins-1], evaluated in fp32 (the precision the scores have); NaN
    scores are not counted.  This is the fixed-size summary a multi-GPU job
    sums over GPUs before solving the bias [Handbook news, Kimi K3]."""
    s32 = np.asarray(s, np.float32)
    T, E = s32.shape
    scale = np.float32(nbins) / (np.float32(hi) - np.float32(lo))
    with np.errstate(invalid="ignore"):
        b = np.floor((s32 - np.float32(lo)) * scale)
    ok = ~np.isnan(b)
    b = np.clip(np.where(ok, b, 0), 0, nbins - 1).astype(np.int64)
    hist = np.zeros((E, nbins), np.int64)
    for e in range(E):
        hist[e] = np.bincount(b[ok[:, e], e], minlength=nbins)
    return hist


def quantile_bias(hist, lo: float, hi: float, target: float):
    """Quantile balancing [Handbook news, Kimi K3: the bias solved from score
    histograms instead of fixed steps].  For each expert e, q_e is the score
    above which `target` of its tokens lie, read off its histogram (bins walked
    from the top, linear within the bin where the count is reached; lo if the
    expert has fewer tokens in all).  The bias b_e = mean(q) - q_e puts every
    expert's target-th largest biased score at the same level, so a threshold
    on s + b would give each expert exactly `target` tokens."""
    hist = np.asarray(hist, np.int64)
    E, nb = hist.shape
    w = (float(hi) - float(lo)) / nb
    q = np.full(E, float(lo))
    for e in range(E):
        c = 0
        for i in range(nb - 1, -1, -1):
            h = int(hist[e, i])
            if h > 0 and c + h >= target:
                q[e] = float(lo) + (i + 1 - (target - c) / h) * w
                break
            c += h
    return q.mean() - q


def load_report(counts, n_dropped: int):
    """Router monitoring [Handbook explainer, "router and load balancing": max
    expert load, drop rate, spread of expert utilisation]: max/mean load, the
    coefficient of variation of the per-expert counts (population std / mean),
    the dropped fraction of the routed slots and the number of empty experts."""
    c = np.asarray(counts, F64)
    mean = c.mean()
    return dict(max_over_mean=float(c.max() / mean), cv=float(c.std() / mean),
                drop_rate=float(n_dropped) / float(c.sum()), n_empty=int(np.sum(c == 0)))


def expert_output_norms(o, offsets):
    """Mean L2 norm of each expert's output rows (0 for an empty expert) and
    max/median over the non-empty experts [Handbook digest, the failure case
    where a layer's largest expert output norm grew from ~14x to 5700x the
    median]."""
    o = np.asarray(o, F64)
    offsets = np.asarray(offsets, np.int64)
    E = offsets.size - 1
    n = np.zeros(E)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            n[e] = np.mean(np.sqrt(np.sum(o[r0:r1] ** 2, axis=1)))
    ne = n[np.diff(offsets) > 0]
    ratio = float(ne.max() / np.median(ne)) if ne.size else 0.0
    return n, ratio


# ---------------------------------------------------------------------------
# MXFP4 routed experts for inference [Handbook news: Kimi K3 quantises its
# routed experts to MXFP4].  Element and scale formats are those of the OCP
# Microscaling (MX) specification: FP4 E2M1 (1 sign, 2 exponent bits with bias
# 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), FP8 E4M3 (bias 7,
# 3 mantissa bits, largest 448, code S.1111.111 is NaN) and the E8M0 shared
# scale 2^(code - 127).  A block's shared exponent is floor(log2(max|v|)) minus
# the element type's largest exponent (2 for E2M1, 8 for E4M3); elements are
# v / 2^X rounded to nearest, ties to even, saturating at the largest
# magnitude.  Weights: FP4 with one scale per 32 consecutive k.  Activations:
# FP8 with one scale per 64 consecutive k (the pairing of the CDNA4 FP8 x FP4
# matrix instruction gives each activation lane halves of two 32-blocks).
# ---------------------------------------------------------------------------
def e2m1_decode(c):
    c = np.asarray(c, np.int64)
    e, m = (c >> 1) & 3, c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(c & 8, -mag, mag)


def e4m3_decode(c):
    c = np.asarray(c, np.int64)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def _encode(v, mbits: int, emin: int, maxmag: float, bias: int):
    """Round |v| to the nearest value of a sign-magnitude float grid with mbits
    mantissa bits, smallest normal exponent emin (subnormals below), ties to
    even, saturating at maxmag; returns codes with the sign at bit
    1 + exponent bits + mbits."""
    v = np.asarray(v, F64)
    a = np.minimum(np.abs(v), maxmag)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    q = np.rint(a / np.ldexp(1.0, (e - mbits).astype(np.int64)))      # units of the grid step
    # q in [0, 2^(mbits+1)]: q = 2^(mbits+1) moves to the next binade
    normal = a >= np.ldexp(1.0, emin)
    m = np.where(q >= 2 ** (mbits + 1), 0, q - np.where(normal, 2 ** mbits, 0))
    ebits = np.where(q >= 2 ** (mbits + 1), e + 1 + bias,
                     np.where(normal, e + bias, np.where(q >= 2 ** mbits, 1, 0)))
    m = np.where(~normal & (q >= 2 ** mbits), q - 2 ** mbits, m)
    code = (ebits.astype(np.int64) << mbits) | m.astype(np.int64)
    sign = np.signbit(v).astype(np.int64) << (mbits + (4 if mbits == 3 else 2))
    return code | sign


def e2m1_encode(v):
    return _encode(v, 1, 0, 6.0, 1)


def e4m3_encode(v):
    return _encode(v, 3, -6, 448.0, 7)


def mx_quantize(w, block: int, fmt: str):
    """Quantise the rows of w [rows, K] in blocks of `block` consecutive k.
    Returns codes [rows, K] (int, one per element) and scale codes
    [rows, K/block] (E8M0)."""
    w = np.asarray(w, F64)
    rows, K = w.shape
    emax = {"e2m1": 2, "e4m3": 8}[fmt]
    blk = w.reshape(rows, K // block, block)
    amax = np.max(np.abs(blk), axis=2)
    _, ex = np.frexp(amax)                        # amax = f * 2^ex, f in [0.5, 1)
    X = np.where(amax > 0, ex - 1 - emax, -127)
    scode = np.clip(X + 127, 0, 254).astype(np.int64)
    scaled = blk / np.ldexp(1.0, (scode - 127))[:, :, None]
    enc = e2m1_encode if fmt == "e2m1" else e4m3_encode
    return enc(scaled).reshape(rows, K), scode


def mx_dequantize(codes, scodes, block: int, fmt: str):
    dec = e2m1_decode if fmt == "e2m1" else e4m3_decode
    v = dec(codes)
    rows, K = v.shape
    return (v.reshape(rows, K // block, block) *
            np.ldexp(1.0, np.asarray(scodes, np.int64) - 127)[:, :, None]).reshape(rows, K)


def expert_ffn_mx(xq, xs, offsets, W13q, W13s, W2q, W2s, act: str, aq=None, as_=None):
    """Grouped expert FFN with FP8 activations (64-blocks) and MXFP4 weights
    (32-blocks): h = deq(x) deq(W13)^T, a = act(h), a quantised to FP8
    (64-blocks), o = deq(a) deq(W2)^T.  With aq/as_ given (the GPU's quantised
    activation), the down projection uses them (a step-wise check).  Returns
    o [R,d], a (float64, before quantisation), aq, as."""
    x = mx_dequantize(xq, xs, 64, "e4m3")
    R = x.shape[0]
    E = len(offsets) - 1
    F = W2q.shape[2] if W2q.ndim == 3 else None
    outs, acts = np.zeros((R, W2q.shape[1])), None
    a_full = None
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        W13 = mx_dequantize(W13q[e], W13s[e], 32, "e2m1")
        h = x[r0:r1] @ W13.T
        if act == "swiglu":
            Fh = W13.shape[0] // 2
            a = silu(h[:, :Fh]) * h[:, Fh:]
        else:
            a = gelu(h)
        if a_full is None:
            a_full = np.zeros((R, a.shape[1]))
        a_full[r0:r1] = a
    if aq is None:
        aq, as_ = mx_quantize(a_full, 64, "e4m3")
    ad = mx_dequantize(aq, as_, 64, "e4m3")
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        W2 = mx_dequantize(W2q[e], W2s[e], 32, "e2m1")
        outs[r0:r1] = ad[r0:r1] @ W2.T
    return outs, a_full, aq, as_


# ---------------------------------------------------------------------------
# Counter-based draws for the stochastic routers.  The noisy top-k router adds
# a standard-normal draw per (token, expert) [MoE-Explained, "What is
# sparsity?", the H(x) equation]; GShard's random routing draws one uniform
# per token to decide its second expert [MoE-Explained, "MoEs and
# Transformers"].  The pages name no generator.  The reading taken: the
# counter-based Philox4x64-10 of Salmon, Moraes, Dror and Shaw ("Parallel
# random numbers: as easy as 1, 2, 3", SC 2011), keyed by (seed, 0); the
# block for draw stream s (0 normals, 1 uniforms) of a call with offset o is
# counter (b, o, s, 0), b = element index // 4, the element taking output word
# index % 4.  A uniform is the word's top 24 bits times 2^-24 (in [0, 1),
# exact in fp32).  Normals come in pairs from the words (0, 1) and (2, 3) of a
# block by the Box-Muller transform (Box and Muller, "A note on the
# generation of random normal deviates", 1958): with uniforms u, v,
# r = sqrt(-2 ln(1 - u)), z0 = r cos(2 pi v), z1 = r sin(2 pi v).
# ---------------------------------------------------------------------------
_PHILOX_M = (0xD2E7470EE14C6C93, 0xCA5A826395121157)   # round multipliers
_PHILOX_W = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)   # key schedule increments
_U64 = np.uint64
_M32 = _U64(0xFFFFFFFF)


def _mulhilo64(a, b):
    """Full 128-bit product of uint64 arrays as (hi, lo), by 32-bit limbs."""
    a0, a1 = a & _M32, a >> _U64(32)
    b0, b1 = b & _M32, b >> _U64(32)
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> _U64(32)) + (p01 & _M32) + (p10 & _M32)
    hi = p11 + (p01 >> _U64(32)) + (p10 >> _U64(32)) + (mid >> _U64(32))
    lo = (mid << _U64(32)) | (p00 & _M32)
    return hi, lo


def philox4x64(counters, key, rounds: int = 10):
    """Philox4x64 of each row of counters [n, 4] (uint64) under key (k0, k1):
    each round multiplies counter words 0 and 2 by the two round multipliers,
    and the new counter is (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
    lo(M0 c0)); the key then advances by the two Weyl increments."""
    c = [np.asarray(counters, dtype=_U64)[:, i].copy() for i in range(4)]
    k0, k1 = int(key[0]), int(key[1])
    with np.errstate(over="ignore"):
        for r in range(rounds):
            hi0, lo0 = _mulhilo64(_U64(_PHILOX_M[0]), c[0])
            hi1, lo1 = _mulhilo64(_U64(_PHILOX_M[1]), c[2])
            c = [hi1 ^ c[1] ^ _U64(k0), lo1, hi0 ^ c[3] ^ _U64(k1), lo0]
            k0 = (k0 + _PHILOX_W[0]) % (1 << 64)
            k1 = (k1 + _PHILOX_W[1]) % (1 << 64)
    return np.stack(c, axis=1)


def _draw_words(n: int, seed: int, offset: int, stream: int):
    """The first n output words of draw stream `stream`, in element order."""
    nb = -(-n // 4)
    ctr = np.zeros((nb, 4), dtype=_U64)
    ctr[:, 0] = np.arange(nb, dtype=_U64)
    ctr[:, 1] = _U64(offset)
    ctr[:, 2] = _U64(stream)
    return philox4x64(ctr, (seed, 0)).reshape(-1)[:n]


def uniform24(words):
    """Uniforms in [0, 1): the top 24 bits of each uint64 word times 2^-24."""
    return (np.asarray(words, dtype=_U64) >> _U64(40)).astype(F64) * 2.0 ** -24


def box_muller(u, v):
    """Two independent standard normals per uniform pair (u, v)."""
    r = np.sqrt(-2.0 * np.log(1.0 - u))
    return r * np.cos(2.0 * np.pi * v), r * np.sin(2.0 * np.pi * v)


def router_draws(T: int, E: int, seed: int, offset: int):
    """The stochastic routers' draws for one call: noise [T, E] standard
    normals (noisy top-k) and uniform [T] in [0, 1) (GShard's second expert),
    element j of either taking word j % 4 of its stream's block j // 4."""
    n = T * E
    w = uniform24(_draw_words(n + (-n) % 4, seed, offset, 0)).reshape(-1, 4)
    z0, z1 = box_muller(w[:, 0], w[:, 1])
    z2, z3 = box_muller(w[:, 2], w[:, 3])
    noise = np.stack([z0, z1, z2, z3], axis=1).reshape(-1)[:n].reshape(T, E)
    uniform = uniform24(_draw_words(T, seed, offset, 1))
    return noise, uniform
