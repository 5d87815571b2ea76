"""Pins of the CPU oracle against what the pages and the mathematics fix.

No GPU.  Each test checks the oracle against something other than itself: a
value the pages print (golden files), a closed form, an invariant the method
guarantees, a library routine for a special case, or brute force on tiny
inputs.  A dropped term, a wrong sign or index, or a transposed operand in any
oracle function fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special as sps
import torch
import torch.nn.functional as TF

import oracle as orc
from top_routing_expert_amd import presets, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(**kw):
    base = dict(name="tiny", T=48, d=16, E=6, k=2, F=8, act="swiglu", score="softmax",
                renorm=True, gate_scale=1.0, capacity_factor=0.0, dtype="f32",
                wg_std=0.5, w_std=0.4)
    base.update(kw)
    return presets.Preset(**base)


# ---------------------------------------------------------------------------
# capacity (golden values from the pages' equation)
# ---------------------------------------------------------------------------
def test_capacity_golden():
    g = json.load(open(os.path.join(GOLDEN, "capacity.json")))
    for c in g["cases"]:
        assert orc.capacity(c["T"], c["E"], c["k"], c["capacity_factor"]) == c["C"], c


def test_capacity_of_presets():
    assert orc.capacity(256, 8, 2, presets.get("c1").capacity_factor) == 80
    assert orc.capacity(8192, 32, 1, presets.get("c2").capacity_factor) == 256


# ---------------------------------------------------------------------------
# scoring functions against library routines
# ---------------------------------------------------------------------------
def test_scores_match_library():
    rng = np.random.default_rng(1)
    z = rng.normal(size=(40, 9)) * 3
    np.testing.assert_allclose(orc.score(z, "softmax"), sps.softmax(z, axis=1), rtol=1e-13)
    np.testing.assert_allclose(orc.score(z, "sigmoid"), sps.expit(z), rtol=1e-13)
    np.testing.assert_allclose(orc.score(z, "sqrt_softplus"),
                               np.sqrt(np.logaddexp(0.0, z)), rtol=1e-13)
    zt = torch.from_numpy(z)
    np.testing.assert_allclose(orc.score(z, "sqrt_softplus"),
                               torch.sqrt(TF.softplus(zt)).numpy(), rtol=1e-12)


def test_logsumexp_matches_library():
    z = np.random.default_rng(2).normal(size=(30, 7)) * 5
    np.testing.assert_allclose(orc.logsumexp_rows(z), sps.logsumexp(z, axis=1), rtol=1e-14)


def test_gelu_closed_forms_and_library():
    v = np.linspace(-6, 6, 1001)
    assert orc.gelu(np.array([0.0]))[0] == 0.0
    # x*Phi(x) - (-x)*Phi(-x) = x for the exact erf GELU
    np.testing.assert_allclose(orc.gelu(v) - orc.gelu(-v), v, atol=1e-13)
    np.testing.assert_allclose(orc.gelu(v), TF.gelu(torch.from_numpy(v)).numpy(), atol=1e-14)
    np.testing.assert_allclose(orc.silu(v), TF.silu(torch.from_numpy(v)).numpy(), atol=1e-14)


# ---------------------------------------------------------------------------
# selection and gates
# ---------------------------------------------------------------------------
def _bruteforce_topk(sel, k):
    T, E = sel.shape
    out = np.zeros((T, k), np.int64)
    for t in range(T):
        rank = []
        for e in range(E):
            # number of experts that beat e: larger score, or equal and lower index
            beat = sum(1 for f in range(E)
                       if sel[t, f] > sel[t, e] or (sel[t, f] == sel[t, e] and f < e))
            rank.append(beat)
        for e in range(E):
            if rank[e] < k:
                out[t, rank[e]] = e
    return out


@pytest.mark.parametrize("k", [1, 2, 3, 6])
def test_topk_bruteforce_with_bias(k):
    rng = np.random.default_rng(3)
    s = rng.random((64, 6))
    b = rng.normal(size=6) * 0.1
    sel = s + b
    np.testing.assert_array_equal(orc.select_topk(sel, k), _bruteforce_topk(sel, k))


def test_exact_ties_go_to_lowest_index():
    sel = np.array([[0.5, 0.7, 0.7, 0.1, 0.7], [0.2, 0.2, 0.2, 0.2, 0.2], [-0.0, 0.0, -1, -0.0, 0.0]])
    idx = orc.select_topk(sel, 3)
    np.testing.assert_array_equal(idx, [[1, 2, 4], [0, 1, 2], [0, 1, 3]])


def test_nan_ranks_lowest():
    sel = np.array([[np.nan, 0.1, -np.inf, 0.3]])
    np.testing.assert_array_equal(orc.select_topk(sel, 4), [[3, 1, 2, 0]])


def test_duplicated_router_columns_tie_to_lowest_index():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(20, 8))
    Wg = rng.normal(size=(8, 5))
    Wg[:, 3] = Wg[:, 1]        # experts 1 and 3 always tie
    r = orc.route(x, Wg, k=5, score_kind="softmax", renorm=False, gate_scale=1.0)
    pos = {e: np.argmax(r["idx"] == e, axis=1) for e in (1, 3)}
    assert np.all(pos[1] < pos[3])


def test_softmax_renorm_equals_softmax_of_keeptopk():
    """G(x) = Softmax(KeepTopK(x W_g, k)), written out from the gating equations."""
    rng = np.random.default_rng(5)
    x, Wg = rng.normal(size=(50, 12)), rng.normal(size=(12, 8))
    k = 3
    r = orc.route(x, Wg, k=k, score_kind="softmax", renorm=True, gate_scale=1.0)
    z = x @ Wg
    kept = np.full_like(z, -np.inf)
    for t in range(z.shape[0]):
        for e in range(z.shape[1]):
            if np.sum(z[t] > z[t, e]) < k:       # no ties in continuous data
                kept[t, e] = z[t, e]
    G = sps.softmax(kept, axis=1)
    G_from_oracle = np.zeros_like(G)
    np.put_along_axis(G_from_oracle, r["idx"], r["g"], axis=1)
    np.testing.assert_allclose(G_from_oracle, G, rtol=1e-12, atol=1e-15)


def test_top1_gate_is_max_probability():
    rng = np.random.default_rng(6)
    x, Wg = rng.normal(size=(40, 10)), rng.normal(size=(10, 7))
    r = orc.route(x, Wg, k=1, score_kind="softmax", renorm=False, gate_scale=1.0)
    np.testing.assert_allclose(r["g"][:, 0], sps.softmax(x @ Wg, axis=1).max(axis=1), rtol=1e-13)


@pytest.mark.parametrize("kind", ["softmax", "sigmoid", "sqrt_softplus"])
def test_k_distinct_experts_and_gate_sum(kind):
    p = tiny(score=kind, k=3, gate_scale=math.sqrt(3.0), sel_bias_std=0.1, zipf_s=1.1)
    inp = synth.make_inputs(p, seed=7, experts=False)
    r = orc.route(inp["x"], inp["Wg"], p.k, kind, True, p.gate_scale, inp["offset"], inp["sel_bias"])
    for t in range(p.T):
        assert len(set(r["idx"][t].tolist())) == p.k
    np.testing.assert_allclose(r["g"].sum(axis=1), np.float32(math.sqrt(3.0)), rtol=1e-13)


def test_selection_bias_selects_but_does_not_gate():
    rng = np.random.default_rng(8)
    x, Wg = rng.normal(size=(30, 6)), rng.normal(size=(6, 5)) * 0.3
    bias = np.array([0.0, 0.0, 0.0, 100.0, 0.0])
    r = orc.route(x, Wg, k=1, score_kind="sigmoid", renorm=False, gate_scale=1.0, sel_bias=bias)
    assert np.all(r["idx"][:, 0] == 3)
    np.testing.assert_allclose(r["g"][:, 0], sps.expit((x @ Wg)[:, 3]), rtol=1e-13)


def test_near_tie_flags():
    sel = np.array([[1.0, 1.0 + 5e-6, 0.2], [1.0, 0.5, 0.5 + 1e-7], [1.0, 0.5, 0.2]])
    b, o = orc.near_tie_flags(sel, 1)
    np.testing.assert_array_equal(b, [True, False, False])
    b, o = orc.near_tie_flags(sel, 2)
    np.testing.assert_array_equal(b, [False, True, False])
    np.testing.assert_array_equal(o, [True, False, False])


# ---------------------------------------------------------------------------
# losses
# ---------------------------------------------------------------------------
def test_aux_loss_collapse_and_uniform():
    T, E, k = 64, 8, 1
    z = np.zeros((T, E)); z[:, 0] = 60.0           # every token sends ~all mass to expert 0
    s = orc.score(z, "softmax")
    counts = np.bincount(orc.select_topk(s, k).ravel(), minlength=E)
    aux, _ = orc.router_losses(z, s, counts, k, 0.5, 0.0)
    assert counts[0] == T
    np.testing.assert_allclose(aux, np.float32(0.5) * E, rtol=1e-12)
    # perfectly uniform probabilities and loads give exactly the coefficient
    s_u = np.full((T, E), 1.0 / E)
    aux_u, _ = orc.router_losses(np.zeros((T, E)), s_u, np.full(E, T * 2 // E), 2, 0.5, 0.0)
    np.testing.assert_allclose(aux_u, 0.5, rtol=1e-12)


def test_aux_loss_normalises_nonsoftmax_scores():
    # sigmoid scores are normalised over E before averaging: doubling every
    # score leaves the loss unchanged
    rng = np.random.default_rng(9)
    s = rng.random((20, 5)) + 0.1
    counts = np.array([4, 10, 6, 12, 8])
    a1, _ = orc.router_losses(np.zeros_like(s), s, counts, 2, 1.0, 0.0)
    a2, _ = orc.router_losses(np.zeros_like(s), 2 * s, counts, 2, 1.0, 0.0)
    P = (s / s.sum(1, keepdims=True)).mean(0)
    np.testing.assert_allclose(a1, a2, rtol=1e-13)
    np.testing.assert_allclose(a1, 5 * np.sum(counts / 40 * P), rtol=1e-13)


def test_zloss_closed_form():
    T, E = 10, 16
    _, zl = orc.router_losses(np.zeros((T, E)), np.full((T, E), 1 / E), np.zeros(E), 1, 0.0, 0.25)
    np.testing.assert_allclose(zl, 0.25 * math.log(E) ** 2, rtol=1e-14)
    z = np.random.default_rng(10).normal(size=(T, E)) * 4
    _, zl = orc.router_losses(z, orc.score(z, "softmax"), np.zeros(E), 1, 0.0, 0.25)
    np.testing.assert_allclose(zl, 0.25 * np.mean(sps.logsumexp(z, axis=1) ** 2), rtol=1e-13)


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------
def _check_dispatch_invariants(idx, E, C, counts, offsets, row_of_slot, token_of_row):
    T, k = idx.shape
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    kept = counts if C is None else np.minimum(counts, C)
    drops = 0 if C is None else int(np.maximum(counts - C, 0).sum())
    R = int(offsets[-1])
    assert R == T * k - drops == int(kept.sum())
    assert int(np.count_nonzero(row_of_slot >= 0)) == R
    rows = row_of_slot[row_of_slot >= 0]
    assert sorted(rows.tolist()) == list(range(R))          # each kept slot exactly once
    assert np.all(token_of_row[R:] == -1)
    for t in range(T):
        for j in range(k):
            r = row_of_slot[t, j]
            if r >= 0:
                assert token_of_row[r] == t
                e = idx[t, j]
                assert offsets[e] <= r < offsets[e + 1]
    for e in range(E):
        seg = token_of_row[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)                      # ascending token order


def test_dispatch_bruteforce_ranks():
    rng = np.random.default_rng(11)
    T, E, k, C = 40, 5, 2, 13
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    counts, offsets, ros, tor = orc.dispatch(idx, E, C)
    _check_dispatch_invariants(idx, E, C, counts, offsets, ros, tor)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            rank = sum(1 for u in range(t) if e in idx[u])
            base = sum(min(int(np.sum(idx == f)), C) for f in range(e))
            assert ros[t, j] == (base + rank if rank < C else -1)


def test_dispatch_bruteforce_with_repeated_experts():
    """A token listing one expert in several slots occupies one row per slot:
    the rank of slot (t, j) in expert e counts every earlier (token, slot) pair
    with e, in (token, slot) order."""
    rng = np.random.default_rng(13)
    T, E, k, C = 50, 4, 3, 20
    idx = rng.integers(0, E, size=(T, k))
    idx[::4, 1] = idx[::4, 0]
    idx[::9] = 2
    counts, offsets, ros, tor = orc.dispatch(idx, E, C)
    np.testing.assert_array_equal(counts, [int(np.sum(idx == e)) for e in range(E)])
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            rank = sum(1 for u in range(T) for i in range(k)
                       if idx[u, i] == e and (u, i) < (t, j))
            base = sum(min(int(np.sum(idx == f)), C) for f in range(e))
            assert ros[t, j] == (base + rank if rank < C else -1)
            if ros[t, j] >= 0:
                assert tor[ros[t, j]] == t


def test_dispatch_invariants_on_presets():
    for name in ("c1", "c2"):
        p = presets.get(name)
        inp = synth.make_inputs(p, seed=0, experts=False)
        r = orc.route(inp["x"], inp["Wg"], p.k, p.score, p.renorm, p.gate_scale,
                      inp["offset"], inp["sel_bias"])
        C = orc.capacity(p.T, p.E, p.k, p.capacity_factor)
        out = orc.dispatch(r["idx"], p.E, C)
        _check_dispatch_invariants(r["idx"], p.E, C, *out)


def test_forced_collapse_keeps_first_tokens():
    p = tiny(T=64, E=4, k=1, capacity_factor=1.0)
    inp = synth.make_inputs(p, seed=12, experts=False)
    offset = np.array([50.0, 0.0, 0.0, 0.0])
    r = orc.route(inp["x"], inp["Wg"], 1, "softmax", False, 1.0, offset)
    C = orc.capacity(p.T, p.E, 1, 1.0)
    assert C == 16
    counts, offsets, ros, tor = orc.dispatch(r["idx"], p.E, C)
    assert counts[0] == 64
    np.testing.assert_array_equal(tor[:C], np.arange(C))
    np.testing.assert_array_equal(ros[:C, 0], np.arange(C))
    assert np.all(ros[C:, 0] == -1)


# ---------------------------------------------------------------------------
# whole layer against brute force and special cases
# ---------------------------------------------------------------------------
def _torch_ffn(x, W13e, W2e, act):
    x, W13e, W2e = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, W13e, W2e))
    if act == "swiglu":
        F = W13e.shape[0] // 2
        a = TF.silu(TF.linear(x, W13e[:F])) * TF.linear(x, W13e[F:])
    else:
        a = TF.gelu(TF.linear(x, W13e))
    return TF.linear(a, W2e).numpy()


@pytest.mark.parametrize("kind,renorm,scale,act", [
    ("softmax", True, 1.0, "swiglu"), ("sigmoid", True, math.sqrt(2), "swiglu"),
    ("sqrt_softplus", True, math.sqrt(2), "gelu"), ("softmax", False, 1.0, "gelu")])
def test_layer_equals_dense_bruteforce(kind, renorm, scale, act):
    """y_t = sum over all experts of G_te E_e(x_t), G zero outside the top-k."""
    p = tiny(score=kind, renorm=renorm, gate_scale=scale, act=act, F_shared=6,
             sel_bias_std=0.05, zipf_s=1.1)
    inp = synth.make_inputs(p, seed=13)
    f = orc.layer_fwd(p, inp)
    z = inp["x"].astype(np.float64) @ inp["Wg"] + inp["offset"]
    s = {"softmax": lambda v: sps.softmax(v, axis=1), "sigmoid": sps.expit,
         "sqrt_softplus": lambda v: np.sqrt(np.logaddexp(0, v))}[kind](z)
    sel = s + inp["sel_bias"]
    mask = np.array([[np.sum(sel[t] > sel[t, e]) < p.k for e in range(p.E)] for t in range(p.T)])
    G = np.where(mask, s, 0.0)
    if renorm:
        G = G / G.sum(axis=1, keepdims=True)
    G = G * np.float32(scale)
    y = _torch_ffn(inp["x"], inp["Ws13"], inp["Ws2"], "swiglu")
    for e in range(p.E):
        y = y + G[:, e:e + 1] * _torch_ffn(inp["x"], inp["W13"][e], inp["W2"][e], act)
    np.testing.assert_allclose(f["y"], y, rtol=1e-11, atol=1e-12)


def test_single_expert_is_plain_ffn():
    p = tiny(E=1, k=1, renorm=False)
    inp = synth.make_inputs(p, seed=14)
    f = orc.layer_fwd(p, inp)
    np.testing.assert_allclose(f["g"], 1.0)
    np.testing.assert_allclose(f["y"], _torch_ffn(inp["x"], inp["W13"][0], inp["W2"][0], "swiglu"),
                               rtol=1e-12, atol=1e-13)


def test_k_equals_E_is_dense_softmax_mixture():
    p = tiny(k=6, renorm=False)
    inp = synth.make_inputs(p, seed=15)
    f = orc.layer_fwd(p, inp)
    P = sps.softmax(inp["x"].astype(np.float64) @ inp["Wg"], axis=1)
    y = sum(P[:, e:e + 1] * _torch_ffn(inp["x"], inp["W13"][e], inp["W2"][e], "swiglu")
            for e in range(p.E))
    np.testing.assert_allclose(f["y"], y, rtol=1e-11, atol=1e-12)


def test_identity_experts_with_drops():
    """With E_i = I the layer returns (sum of kept gates) * x; dropped slots add 0."""
    p = tiny(T=64, k=2, capacity_factor=0.75)
    inp = synth.make_inputs(p, seed=16, experts=False)
    r = orc.route(inp["x"], inp["Wg"], p.k, p.score, p.renorm, p.gate_scale)
    C = orc.capacity(p.T, p.E, p.k, p.capacity_factor)
    counts, offsets, ros, tor = orc.dispatch(r["idx"], p.E, C)
    R = int(offsets[-1])
    assert R < p.T * p.k                                   # some slots dropped
    y = orc.combine(orc.permute(inp["x"], tor, R), ros, r["g"])
    gk = np.where(ros >= 0, r["g"], 0.0).sum(axis=1)
    np.testing.assert_allclose(y, gk[:, None] * inp["x"], rtol=1e-14, atol=1e-15)


def test_handbook_example_accounting():
    g = json.load(open(os.path.join(GOLDEN, "handbook_example.json")))
    assert g["top_k"] * g["expert_width"] == g["dense_width"]
    assert g["experts"] * g["expert_width"] == g["param_ratio"] * g["dense_width"]
    p = presets.get("c4")
    assert (p.E, p.k, p.F) == (g["experts"], g["top_k"], g["expert_width"])


# ---------------------------------------------------------------------------
# bias update
# ---------------------------------------------------------------------------
def test_bias_update_sign_rule():
    counts = np.array([2, 4, 6, 4])        # T*k/E = 4
    b = orc.bias_update(counts, np.zeros(4), T=8, k=2, gamma=0.5)
    np.testing.assert_array_equal(b, [0.5, 0.0, -0.5, 0.0])


# ---------------------------------------------------------------------------
# backward against central finite differences (fp64, away from ties/edges)
# ---------------------------------------------------------------------------
def _objective(p, inp, dy):
    f = orc.layer_fwd(p, inp)
    return float(np.sum(dy * f["y"]) + f["aux"] + f["zloss"]), f


@pytest.mark.parametrize("kind,act,cf,shared,routing", [
    ("softmax", "swiglu", 0.0, 0, "topk"), ("sigmoid", "swiglu", 0.0, 6, "topk"),
    ("sqrt_softplus", "swiglu", 0.0, 6, "topk"), ("softmax", "gelu", 0.75, 0, "topk"),
    ("sqrt_softplus", "gelu", 0.75, 6, "topk"), ("sigmoid", "swiglu", 0.0, 6, "uniform"),
    ("softmax", "swiglu", 0.75, 6, "noisy_topk"), ("softmax", "gelu", 0.0, 0, "gshard"),
    ("sqrt_softplus", "swiglu", 0.0, 0, "hash")])
def test_backward_finite_differences(kind, act, cf, shared, routing):
    p = tiny(T=24, d=10, E=5, k=2, F=6, score=kind, act=act, capacity_factor=cf,
             F_shared=shared, gate_scale=math.sqrt(2.0), aux_coef=0.3, z_coef=0.2,
             sel_bias_std=0.05, zipf_s=1.1, renorm=kind != "softmax" or act == "swiglu",
             routing=routing)
    inp = synth.make_inputs(p, seed=17, with_dy=True)
    inp = {k_: (None if v is None else np.asarray(v, np.float64)) for k_, v in inp.items()}
    dy = inp["dy"]
    J0, f0 = _objective(p, inp, dy)
    assert not f0["near_tie"].any() and not f0["near_tie_order"].any()
    fk = orc.layer_fwd(p, inp, keep_hidden=True)
    grads = orc.layer_bwd(p, inp, fk, dy)
    names = [("x", "dx"), ("Wg", "dWg"), ("W13", "dW13"), ("W2", "dW2")]
    if routing == "noisy_topk":
        names += [("W_noise", "dW_noise")]
    if shared:
        names += [("Ws13", "dWs13"), ("Ws2", "dWs2")]
    rng = np.random.default_rng(18)
    eps = 1e-6
    for pname, gname in names:
        arr = inp[pname]
        flat = arr.reshape(-1)
        picks = rng.choice(flat.size, size=min(flat.size, 25), replace=False)
        for i in picks:
            old = flat[i]
            flat[i] = old + eps
            Jp, fp = _objective(p, inp, dy)
            flat[i] = old - eps
            Jm, fm = _objective(p, inp, dy)
            flat[i] = old
            assert np.array_equal(fp["row_of_slot"], f0["row_of_slot"])
            assert np.array_equal(fm["row_of_slot"], f0["row_of_slot"])
            fd = (Jp - Jm) / (2 * eps)
            an = grads[gname].reshape(-1)[i]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (pname, i, fd, an)


# ---------------------------------------------------------------------------
# forced-uniform routing (the handbook's balanced baseline)
# ---------------------------------------------------------------------------
def test_uniform_routing_round_robin_balanced_distinct():
    """Read slot by slot (token-major), the experts cycle 0..E-1; every expert
    gets T*k/E slots and a token's k experts are distinct."""
    p = tiny(T=48, E=6, k=4, routing="uniform")
    inp = synth.make_inputs(p, seed=21)
    r = orc.route(inp["x"], inp["Wg"], p.k, p.score, p.renorm, p.gate_scale, routing="uniform")
    flat = r["idx"].reshape(-1)
    assert np.array_equal(flat[:p.E], np.arange(p.E))
    assert np.array_equal(flat[p.E:], flat[:-p.E])
    assert (r["counts"] == p.T * p.k // p.E).all()
    assert all(len(set(row)) == p.k for row in r["idx"].tolist())
    assert not r["near_tie"].any()


def test_uniform_routing_aux_loss_is_coefficient():
    """f_e = 1/E for every expert, so L_aux = a * E * sum_e P_e / E = a."""
    p = tiny(T=60, E=5, k=2, routing="uniform", aux_coef=0.37)
    inp = synth.make_inputs(p, seed=22)
    for kind in ("softmax", "sigmoid", "sqrt_softplus"):
        r = orc.route(inp["x"], inp["Wg"], p.k, kind, True, 1.0, aux_coef=p.aux_coef,
                      routing="uniform")
        assert abs(r["aux"] - float(np.float32(p.aux_coef))) < 1e-14   # coefficients are fp32


@pytest.mark.parametrize("kind,renorm", [("softmax", True), ("sigmoid", False)])
def test_uniform_routing_layer_equals_dense_bruteforce(kind, renorm):
    """y_t = sum_e G_te E_e(x_t) with G the scores on the forced experts only."""
    p = tiny(T=30, E=5, k=2, score=kind, renorm=renorm, gate_scale=1.5, routing="uniform",
             capacity_factor=0.0)
    inp = synth.make_inputs(p, seed=23)
    f = orc.layer_fwd(p, inp)
    z = inp["x"].astype(np.float64) @ inp["Wg"]
    s = sps.softmax(z, axis=1) if kind == "softmax" else sps.expit(z)
    mask = np.zeros((p.T, p.E), bool)
    e = 0
    for t in range(p.T):          # hand the slots out one by one, cycling over experts
        for _ in range(p.k):
            mask[t, e] = True
            e = (e + 1) % p.E
    G = np.where(mask, s, 0.0)
    if renorm:
        G = G / G.sum(axis=1, keepdims=True)
    G = G * np.float32(1.5)
    y = np.zeros((p.T, p.d))
    for e in range(p.E):
        y = y + G[:, e:e + 1] * _torch_ffn(inp["x"], inp["W13"][e], inp["W2"][e], p.act)
    np.testing.assert_allclose(f["y"], y, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# variant routers: noisy top-k, random second expert, token-id hash; overflow priority
# ---------------------------------------------------------------------------
def _dense_y(p, inp, G):
    y = np.zeros((p.T, p.d))
    for e in range(p.E):
        y = y + G[:, e:e + 1] * _torch_ffn(inp["x"], inp["W13"][e], inp["W2"][e], p.act)
    return y


def test_noisy_topk_without_noise_is_topk():
    p = tiny(routing="noisy_topk", k=2)
    inp = synth.make_inputs(p, seed=31)
    a = orc.route(inp["x"], inp["Wg"], 2, "softmax", True, 1.0, routing="noisy_topk",
                  W_noise=inp["W_noise"], noise=np.zeros_like(inp["noise"]))
    b = orc.route(inp["x"], inp["Wg"], 2, "softmax", True, 1.0)
    assert np.array_equal(a["idx"], b["idx"]) and np.allclose(a["g"], b["g"], rtol=0, atol=0)


def test_noisy_topk_large_draw_wins():
    """A large positive draw on expert e makes it the first choice."""
    p = tiny(routing="noisy_topk", k=2)
    inp = synth.make_inputs(p, seed=32)
    noise = inp["noise"].copy()
    want = np.arange(p.T) % p.E
    noise[np.arange(p.T), want] = 1e4
    r = orc.route(inp["x"], inp["Wg"], 2, "softmax", True, 1.0, routing="noisy_topk",
                  W_noise=inp["W_noise"], noise=noise)
    assert np.array_equal(r["idx"][:, 0], want)


def test_noisy_topk_layer_equals_dense_bruteforce():
    """G = Softmax(KeepTopK(H, k)) with H = x Wg + eps * log(1 + exp(x Wn)),
    summed densely over all experts."""
    p = tiny(T=40, E=6, k=2, routing="noisy_topk", renorm=True, gate_scale=1.0)
    inp = synth.make_inputs(p, seed=33)
    f = orc.layer_fwd(p, inp)
    x = inp["x"].astype(np.float64)
    H = x @ inp["Wg"] + inp["noise"] * np.log1p(np.exp(x @ inp["W_noise"]))
    keep = np.array([[np.sum(H[t] > H[t, e]) < p.k for e in range(p.E)] for t in range(p.T)])
    Hk = np.where(keep, H, -np.inf)
    G = np.exp(Hk - Hk.max(axis=1, keepdims=True))
    G = G / G.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(f["y"], _dense_y(p, inp, G), rtol=1e-11, atol=1e-12)


def _top2_by_hand(s):
    out = []
    for row in s:
        order = sorted(range(len(row)), key=lambda e: (-row[e], e))
        out.append(order[:2])
    return np.array(out)


def test_random_second_expert_rule():
    """First expert always; second kept iff u < 2 g2 / (g1 + g2); u = 0 keeps all."""
    p = tiny(T=200, E=6, k=2, routing="gshard")
    inp = synth.make_inputs(p, seed=34)
    r = orc.route(inp["x"], inp["Wg"], 2, "softmax", True, 1.0, routing="gshard",
                  uniform=inp["uniform"])
    s = sps.softmax(inp["x"].astype(np.float64) @ inp["Wg"], axis=1)
    top = _top2_by_hand(s)
    assert np.array_equal(r["idx"], top)
    s1, s2 = s[np.arange(p.T), top[:, 0]], s[np.arange(p.T), top[:, 1]]
    assert r["active"][:, 0].all()
    np.testing.assert_array_equal(r["active"][:, 1], inp["uniform"] < 2 * s2 / (s1 + s2))
    assert 0 < r["active"][:, 1].sum() < p.T
    np.testing.assert_array_equal(r["counts"], np.bincount(r["idx"][r["active"]], minlength=p.E))
    r0 = orc.route(inp["x"], inp["Wg"], 2, "softmax", True, 1.0, routing="gshard",
                   uniform=np.zeros(p.T, np.float32))
    assert r0["active"].all()


def test_random_second_expert_layer_dense():
    """y = g1 E1 + [second kept] g2 E2, gates normalised over both experts."""
    p = tiny(T=50, E=5, k=2, routing="gshard", renorm=True)
    inp = synth.make_inputs(p, seed=35)
    f = orc.layer_fwd(p, inp)
    s = sps.softmax(inp["x"].astype(np.float64) @ inp["Wg"], axis=1)
    top = _top2_by_hand(s)
    s1, s2 = s[np.arange(p.T), top[:, 0]], s[np.arange(p.T), top[:, 1]]
    keep2 = inp["uniform"] < 2 * s2 / (s1 + s2)
    G = np.zeros((p.T, p.E))
    G[np.arange(p.T), top[:, 0]] = s1 / (s1 + s2)
    G[np.arange(p.T), top[:, 1]] = np.where(keep2, s2 / (s1 + s2), 0.0)
    np.testing.assert_allclose(f["y"], _dense_y(p, inp, G), rtol=1e-11, atol=1e-12)


def test_slot_priority_dispatch_bruteforce():
    """Top-1-first overflow: walk the slots in (slot, token) order, each expert
    filling its C places in that order."""
    rng = np.random.default_rng(36)
    T, k, E, C = 40, 3, 5, 9
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    active = rng.random((T, k)) < 0.85
    counts, offsets, ros, tor = orc.dispatch(idx, E, C, active, "slot")
    fill = np.zeros(E, np.int64)
    want = np.full((T, k), -1)
    kept = np.minimum(np.bincount(idx[active], minlength=E), C)
    base = np.concatenate([[0], np.cumsum(kept)])
    for j in range(k):
        for t in range(T):
            e = idx[t, j]
            if active[t, j] and fill[e] < C:
                want[t, j] = base[e] + fill[e]
                fill[e] += 1
    np.testing.assert_array_equal(ros, want)
    np.testing.assert_array_equal(offsets, base)
    np.testing.assert_array_equal(counts, np.bincount(idx[active], minlength=E))
    R = int(offsets[-1])
    assert sorted(ros[ros >= 0].tolist()) == list(range(R))
    assert all(tor[ros[t, j]] == t for t in range(T) for j in range(k) if ros[t, j] >= 0)


def test_fmix32_is_a_bijection():
    v = np.arange(1 << 18, dtype=np.int64)
    h = orc.fmix32(v)
    assert len(np.unique(h)) == v.size and int(orc.fmix32(np.array([0]))[0]) == 0
    # invert it: undo each xor-shift and multiply by the inverse constants mod 2^32
    def unshift(x, s):
        y = x.copy()
        for _ in range(32 // s + 1):
            y = x ^ (y >> s)
        return y
    y = unshift(h, 16)
    y = (y * pow(0xC2B2AE35, -1, 1 << 32)) & 0xFFFFFFFF
    y = unshift(y, 13)
    y = (y * pow(0x85EBCA6B, -1, 1 << 32)) & 0xFFFFFFFF
    y = unshift(y, 16)
    assert np.array_equal(y.astype(np.int64), v)


def test_hash_routing_fixed_per_id_distinct_balanced():
    p = tiny(T=4000, E=8, k=3, routing="hash")
    inp = synth.make_inputs(p, seed=37)
    ids = inp["token_ids"].copy()
    ids[100:200] = ids[0]                     # repeated ids route identically
    r = orc.route(inp["x"], inp["Wg"], p.k, "softmax", True, 1.0, routing="hash", token_ids=ids)
    assert (r["idx"][100:200] == r["idx"][0]).all()
    assert all(len(set(row)) == p.k for row in r["idx"].tolist())
    # experts are k consecutive ones (mod E) from a start that depends only on the id
    assert ((r["idx"][:, 1:] - r["idx"][:, :-1]) % p.E == 1).all()
    c = r["counts"] / r["counts"].sum()
    assert np.max(np.abs(c - 1 / p.E)) < 0.02


# ---------------------------------------------------------------------------
# quantile balancing from score histograms; router monitoring
# ---------------------------------------------------------------------------
def test_score_histogram_matches_numpy_away_from_edges():
    rng = np.random.default_rng(40)
    nb, lo, hi = 64, 0.0, 1.0
    centres = (rng.integers(0, nb, size=(500, 7)) + 0.5) / nb
    s = centres + rng.uniform(-0.3, 0.3, size=centres.shape) / nb
    h = orc.score_histogram(s, lo, hi, nb)
    for e in range(7):
        ref, _ = np.histogram(s[:, e], bins=nb, range=(lo, hi))
        np.testing.assert_array_equal(h[e], ref)
    s[0, 0], s[1, 0], s[2, 0] = -5.0, 7.0, np.nan          # clamped, clamped, skipped
    h2 = orc.score_histogram(s, lo, hi, nb)
    assert h2[0, 0] >= 1 and h2[0, -1] >= 1 and h2[0].sum() == 499


def test_quantile_bias_closed_form_grid():
    """One token per bin: expert e's L-th largest score is exactly lo + (nb - L) w."""
    nb, E, L = 100, 3, 17
    s = np.repeat(((np.arange(nb) + 0.5) / nb)[:, None], E, axis=1)
    s[:, 1] = s[:, 1] * 0.5          # expert 1: bins 0..49 with two tokens in each of half of them
    h = orc.score_histogram(s, 0.0, 1.0, nb)
    b = orc.quantile_bias(h, 0.0, 1.0, L)
    q0 = (nb - L) / nb
    # expert 1: scores (i + 0.5) / 200 -> bin floor((i+0.5)/2): two tokens per bin 0..49
    c, q1 = 0, None
    for i in range(nb - 1, -1, -1):
        hh = h[1, i]
        if hh and c + hh >= L:
            q1 = (i + 1 - (L - c) / hh) / nb
            break
        c += hh
    q = np.array([q0, q1, q0])
    np.testing.assert_allclose(b, q.mean() - q, rtol=0, atol=1e-12)
    assert abs(q1 - (50 - 8.5) / nb) < 1e-12          # 8 full bins (16 tokens) + half a bin


def test_quantile_bias_undoes_a_shift_and_balances():
    rng = np.random.default_rng(41)
    T, E, nb, k = 4000, 6, 400, 2
    base = rng.uniform(0.1, 0.6, size=T)
    shift = np.array([0.0, 0.05, 0.1, 0.15, 0.2, 0.25])          # multiples of the bin width 1/400
    s = base[:, None] + shift[None, :]
    L = T * k / E
    b = orc.quantile_bias(orc.score_histogram(s, 0.0, 1.0, nb), 0.0, 1.0, L)
    np.testing.assert_allclose(b - b[0], -shift, atol=1e-12)
    # balance: with the bias, a common threshold gives every expert L tokens
    # (to within one bin's tokens)
    s2 = s + b[None, :]
    tau = np.sort(s2[:, 0])[::-1][int(L) - 1]
    counts = (s2 >= tau - 1e-12).sum(axis=0)
    assert np.all(np.abs(counts - L) <= np.max(orc.score_histogram(s, 0.0, 1.0, nb)))
    # q_e = mean(q) - b_e lies within a bin width of the exact empirical
    # quantile, so mean(exact) - b_e lies within two
    exact = np.sort(s, axis=0)[::-1][int(L) - 1]
    assert np.all(np.abs(exact.mean() - b - exact) <= 2.0 / nb + 1e-12)


def test_load_report_closed_forms():
    E, T, k = 8, 64, 2
    r = orc.load_report(np.full(E, T * k // E), 0)
    assert r == dict(max_over_mean=1.0, cv=0.0, drop_rate=0.0, n_empty=0)
    c = np.zeros(E, np.int64)
    c[3] = T * k
    r = orc.load_report(c, 100)
    assert r["max_over_mean"] == E and abs(r["cv"] - math.sqrt(E - 1)) < 1e-12
    assert r["drop_rate"] == 100 / (T * k) and r["n_empty"] == E - 1


def test_expert_output_norms_bruteforce():
    rng = np.random.default_rng(42)
    offsets = np.array([0, 3, 3, 10, 11])
    o = rng.normal(size=(11, 5))
    n, ratio = orc.expert_output_norms(o, offsets)
    want = [np.mean([np.linalg.norm(o[r]) for r in range(a, b)]) if b > a else 0.0
            for a, b in zip(offsets[:-1], offsets[1:])]
    np.testing.assert_allclose(n, want, rtol=1e-14)
    import statistics
    ne = [want[0], want[2], want[3]]
    assert abs(ratio - max(ne) / statistics.median(ne)) < 1e-14


# ---------------------------------------------------------------------------
# MX formats (OCP Microscaling): FP4 E2M1, FP8 E4M3, E8M0 block scales
# ---------------------------------------------------------------------------
def test_mx_element_tables():
    np.testing.assert_array_equal(orc.e2m1_decode(np.arange(8)), [0, 0.5, 1, 1.5, 2, 3, 4, 6])
    np.testing.assert_array_equal(orc.e2m1_decode(np.arange(8, 16)), -orc.e2m1_decode(np.arange(8)))
    d = orc.e4m3_decode(np.array([0x01, 0x07, 0x08, 0x38, 0x3F, 0x7E, 0x7F, 0xFE]))
    np.testing.assert_array_equal(d[[0, 1, 2, 3, 4, 5, 7]],
                                  [2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.875, 448.0, -448.0])
    assert np.isnan(d[6])


def _nearest_even(v, table_codes, dec):
    """Brute force: the representable value nearest to v (ties to the even
    code, i.e. mantissa bit 0), saturating at the largest magnitude."""
    vals = dec(table_codes)
    out = []
    for x in np.atleast_1d(v):
        dist = np.abs(vals - x)
        best = np.nonzero(dist == dist.min())[0]
        cand = table_codes[best]
        pick = cand[(cand & 1) == 0] if np.any((cand & 1) == 0) else cand
        out.append(int(pick[0]))
    return np.array(out)


def test_e2m1_e4m3_round_to_nearest_even_bruteforce():
    rng = np.random.default_rng(50)
    pos4 = np.arange(8)                                         # non-negative E2M1 codes
    mids = (orc.e2m1_decode(pos4[:-1]) + orc.e2m1_decode(pos4[1:])) / 2
    v = np.concatenate([mids, rng.uniform(0, 7.5, 400), [0.0, 6.0, 9.0, 1e9]])
    np.testing.assert_array_equal(orc.e2m1_encode(v), _nearest_even(v, pos4, orc.e2m1_decode))
    np.testing.assert_array_equal(orc.e2m1_encode(-v) & 7, orc.e2m1_encode(v))
    assert (orc.e2m1_encode(-v[v > 0]) & 8 == 8).all()
    pos8 = np.arange(0x7F)                                      # finite non-negative E4M3 codes
    vals = orc.e4m3_decode(pos8)
    mids8 = (vals[:-1] + vals[1:]) / 2
    v8 = np.concatenate([mids8, rng.uniform(0, 500, 400), np.exp(rng.uniform(-12, 6, 300)), [448.0, 1e6]])
    np.testing.assert_array_equal(orc.e4m3_encode(v8), _nearest_even(v8, pos8, orc.e4m3_decode))


@pytest.mark.parametrize("fmt,block,emax,top", [("e2m1", 32, 2, 6.0), ("e4m3", 64, 8, 448.0)])
def test_mx_block_scale_rule(fmt, block, emax, top):
    """The shared scale puts the block's largest magnitude in [2^emax, 2^(emax+1))
    after scaling; every element is the nearest grid value (saturating)."""
    rng = np.random.default_rng(51)
    w = rng.normal(size=(6, 4 * block)) * np.exp(rng.uniform(-8, 8, size=(6, 1)))
    w[0, :block] = 0.0                                          # an all-zero block
    codes, sc = orc.mx_quantize(w, block, fmt)
    dec = orc.e2m1_decode if fmt == "e2m1" else orc.e4m3_decode
    scale = np.ldexp(1.0, sc - 127)
    amax = np.abs(w.reshape(6, -1, block)).max(axis=2)
    ratio = amax[amax > 0] / scale[amax > 0]
    assert np.all((ratio >= 2.0 ** emax) & (ratio < 2.0 ** (emax + 1)))
    assert np.all(codes[0, :block] % (8 if fmt == "e2m1" else 128) == 0)
    table = np.arange(8) if fmt == "e2m1" else np.arange(0x7F)
    scaled = (w.reshape(6, -1, block) / scale[:, :, None]).reshape(6, -1)
    want = _nearest_even(np.abs(scaled[1:4].ravel()), table, dec)
    got = codes[1:4].ravel() & (7 if fmt == "e2m1" else 0x7F)
    np.testing.assert_array_equal(got, want)
    deq = orc.mx_dequantize(codes, sc, block, fmt)
    assert np.all(np.abs(deq) <= top * scale.repeat(block, axis=1) + 0)


@pytest.mark.parametrize("fmt,block", [("e2m1", 32), ("e4m3", 64)])
def test_mx_dequantize_block_scale_mapping(fmt, block):
    """Element k of a row is scaled by the E8M0 scale of its own block k // block:
    a row whose blocks carry distinct scale codes and one repeated element code
    decodes to that element's value times 2^(scale code - 127), block by block
    (the element value from the format's table: E2M1 code 3 = 1.5, E4M3 code
    0x3A = 1.25)."""
    nb = 5
    code, val = (3, 1.5) if fmt == "e2m1" else (0x3A, 1.25)
    codes = np.full((2, nb * block), code)
    codes[1] |= 8 if fmt == "e2m1" else 0x80                    # second row negative
    sc = np.array([[127, 120, 131, 1, 250], [254, 0, 127, 64, 200]])
    deq = orc.mx_dequantize(codes, sc, block, fmt)
    for r, sign in ((0, 1.0), (1, -1.0)):
        for b in range(nb):
            want = sign * val * 2.0 ** (int(sc[r, b]) - 127)
            assert np.all(deq[r, b * block:(b + 1) * block] == want), (r, b)


@pytest.mark.parametrize("fmt,block,mbits", [("e2m1", 32, 1), ("e4m3", 64, 3)])
def test_mx_round_trip_within_half_a_grid_step(fmt, block, mbits):
    """deq(quant(w)) differs from w by at most half the grid step of the
    element's binade times its block's scale (nearest rounding), on rows whose
    blocks differ in magnitude by up to 2^40; elements beyond the largest grid
    value after scaling (the scale rule lets a block's maximum land up to
    2^(emax+1)) decode to that value with their sign."""
    rng = np.random.default_rng(53)
    rows, nb = 4, 6
    mag = np.ldexp(1.0, rng.integers(-20, 21, size=(rows, nb)))
    w = rng.uniform(-1, 1, size=(rows, nb, block)) * mag[:, :, None]
    w = w.reshape(rows, nb * block)
    codes, sc = orc.mx_quantize(w, block, fmt)
    deq = orc.mx_dequantize(codes, sc, block, fmt)
    scale = np.ldexp(1.0, sc - 127).repeat(block, axis=1)
    emin = 0 if fmt == "e2m1" else -6
    v = np.abs(w) / scale
    with np.errstate(divide="ignore"):
        e = np.maximum(np.floor(np.log2(np.where(v > 0, v, 1.0))), emin)
    step = np.ldexp(1.0, (e - mbits).astype(np.int64))          # grid spacing at v's binade
    top = 6.0 if fmt == "e2m1" else 448.0
    ok = v <= top                                               # not saturated
    assert 0.5 < ok.mean() < 1.0
    err = np.abs(deq - w)
    assert np.all(err[ok] <= 0.5 * step[ok] * scale[ok] * (1 + 1e-12))
    np.testing.assert_array_equal(deq[~ok], np.sign(w[~ok]) * top * scale[~ok])
    # blocks keep their own scale: the error of every block is tiny against the
    # largest block of the row
    for r in range(rows):
        for b in range(nb):
            blk = slice(b * block, (b + 1) * block)
            assert np.max(err[r, blk]) <= 0.5 * np.max(np.abs(w[r, blk]))


def test_expert_ffn_mx_composition():
    """h, a and o of the MX expert FFN against torch on the dequantised values."""
    rng = np.random.default_rng(52)
    d, F, E = 64, 64, 3
    offsets = np.array([0, 5, 5, 12])
    x = rng.normal(size=(12, d))
    W13 = rng.normal(size=(E, 2 * F, d)) * 0.2
    W2 = rng.normal(size=(E, d, F)) * 0.2
    xq, xs = orc.mx_quantize(x, 64, "e4m3")
    W13q = np.stack([orc.mx_quantize(W13[e], 32, "e2m1")[0] for e in range(E)])
    W13s = np.stack([orc.mx_quantize(W13[e], 32, "e2m1")[1] for e in range(E)])
    W2q = np.stack([orc.mx_quantize(W2[e], 32, "e2m1")[0] for e in range(E)])
    W2s = np.stack([orc.mx_quantize(W2[e], 32, "e2m1")[1] for e in range(E)])
    o, a, aq, as_ = orc.expert_ffn_mx(xq, xs, offsets, W13q, W13s, W2q, W2s, "swiglu")
    xd = torch.from_numpy(orc.mx_dequantize(xq, xs, 64, "e4m3"))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        W13d = torch.from_numpy(orc.mx_dequantize(W13q[e], W13s[e], 32, "e2m1"))
        W2d = torch.from_numpy(orc.mx_dequantize(W2q[e], W2s[e], 32, "e2m1"))
        h = xd[r0:r1] @ W13d.T
        ar = TF.silu(h[:, :F]) * h[:, F:]
        np.testing.assert_allclose(a[r0:r1], ar.numpy(), rtol=1e-12, atol=1e-12)
        aqe, ase = orc.mx_quantize(ar.numpy(), 64, "e4m3")
        ad = torch.from_numpy(orc.mx_dequantize(aqe, ase, 64, "e4m3"))
        np.testing.assert_allclose(o[r0:r1], (ad @ W2d.T).numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Counter-based draws (Philox4x64-10 and Box-Muller)
# ---------------------------------------------------------------------------
def test_mulhilo64_against_integers():
    """The limb-wise 128-bit product against Python integers, extremes included."""
    rng = np.random.default_rng(70)
    edge = np.array([0, 1, 2**32 - 1, 2**32, 2**63, 2**64 - 1], dtype=np.uint64)
    a = np.concatenate([edge, np.repeat(edge, len(edge)),
                        rng.integers(0, 2**64, size=3000, dtype=np.uint64)])
    b = np.concatenate([edge[::-1], np.tile(edge, len(edge)),
                        rng.integers(0, 2**64, size=3000, dtype=np.uint64)])
    with np.errstate(over="ignore"):
        hi, lo = orc.moe_oracle._mulhilo64(a, b)
    for x, y, h, l in zip(a.tolist(), b.tolist(), hi.tolist(), lo.tolist()):
        assert (h << 64) | l == x * y


def _ctr_add(ctr, i):
    """The 256-bit counter (word 0 least significant) plus i."""
    v = sum(int(w) << (64 * n) for n, w in enumerate(ctr)) + i
    return [(v >> (64 * n)) % 2**64 for n in range(4)]


@pytest.mark.parametrize("key,ctr", [
    ((0, 0), (0, 0, 0, 0)),
    ((2**64 - 1, 2**64 - 1), (2**64 - 1, 2**64 - 1, 2**64 - 1, 2**64 - 2)),
    ((0x243F6A8885A308D3, 0x13198A2E03707344), (2**64 - 3, 5, 0, 9)),
    ((12345, 0), (2**64 - 1, 6, 1, 0)),
])
def test_philox_matches_numpy(key, ctr):
    """numpy's Philox bit generator is Philox4x64-10 from the same paper; it
    advances its 256-bit counter by one (carrying word 0 into 1, 2, 3) before
    each block and returns the block's four words in order."""
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
    raw = bg.random_raw(4 * 6).reshape(6, 4)
    ctrs = np.array([_ctr_add(ctr, i + 1) for i in range(6)], dtype=np.uint64)
    np.testing.assert_array_equal(orc.philox4x64(ctrs, key), raw)


def _numpy_stream_words(seed, offset, stream, n):
    """Words of draw stream `stream` from numpy's Philox: started one below
    counter (0, offset, stream, 0), its blocks are b = 0, 1, 2, ... (offset >= 1)."""
    bg = np.random.Philox(key=np.array([seed, 0], dtype=np.uint64),
                          counter=np.array([2**64 - 1, offset - 1, stream, 0], dtype=np.uint64))
    return bg.random_raw(n + (-n) % 4)[:n]


def test_router_uniforms_are_numpy_philox_words():
    seed, offset, T = 987654321, 7, 1001
    _, u = orc.router_draws(T, 3, seed, offset)
    w = _numpy_stream_words(seed, offset, 1, T)
    np.testing.assert_array_equal(u, (w >> np.uint64(40)).astype(np.float64) / 2**24)
    assert u.min() >= 0.0 and u.max() < 1.0


def test_router_noise_pairs_against_numpy_words():
    """Each pair (z0, z1) of a block satisfies z0^2 + z1^2 = -2 ln(1 - u) and
    angle(z0, z1) = 2 pi v for the pair's first and second uniforms, taken from
    numpy's Philox words (the polar form of the Box-Muller transform)."""
    seed, offset, T, E = 2**63 + 11, 3, 37, 9           # 333 normals: a ragged last block
    z, _ = orc.router_draws(T, E, seed, offset)
    n = T * E
    w = _numpy_stream_words(seed, offset, 0, n + (-n) % 4)
    u = (w >> np.uint64(40)).astype(np.float64) / 2**24
    zf = np.concatenate([z.reshape(-1), np.full((-n) % 4, np.nan)])
    for j in range(0, n - 1, 2):
        z0, z1 = zf[j], zf[j + 1]
        assert math.isclose(z0 * z0 + z1 * z1, -2 * math.log(1 - u[j]), rel_tol=1e-12, abs_tol=1e-15)
        ang = math.atan2(z1, z0) / (2 * math.pi) % 1.0
        assert abs(ang - u[j + 1]) < 1e-12 or abs(abs(ang - u[j + 1]) - 1) < 1e-12


def test_box_muller_closed_forms():
    r1 = 1 - math.exp(-0.5)                                  # radius 1
    for u, v, want in [(0.0, 0.3, (0.0, 0.0)), (r1, 0.0, (1.0, 0.0)), (r1, 0.25, (0.0, 1.0)),
                       (r1, 0.5, (-1.0, 0.0)), (r1, 0.125, (math.sqrt(0.5), math.sqrt(0.5))),
                       (1 - math.exp(-2), 0.75, (0.0, -2.0))]:
        z0, z1 = orc.box_muller(np.array([u]), np.array([v]))
        assert abs(z0[0] - want[0]) < 1e-12 and abs(z1[0] - want[1]) < 1e-12, (u, v)


def test_router_draws_distribution():
    """Normals: Kolmogorov-Smirnov against the standard normal, moments, and no
    correlation between the two members of a pair or between neighbouring
    tokens; uniforms: Kolmogorov-Smirnov against U[0, 1)."""
    import scipy.stats as ss
    z, u = orc.router_draws(4096, 64, 31337, 1)
    zf = z.reshape(-1)
    assert ss.kstest(zf, "norm").pvalue > 1e-3
    assert abs(zf.mean()) < 5 / math.sqrt(zf.size) and abs(zf.var() - 1) < 0.01
    assert abs(np.corrcoef(zf[0::2], zf[1::2])[0, 1]) < 0.01
    assert abs(np.corrcoef(z[:-1].reshape(-1), z[1:].reshape(-1))[0, 1]) < 0.01
    assert ss.kstest(u, "uniform").pvalue > 1e-3


def test_router_draws_layout_and_streams():
    """Draws depend on the flat element index only (not on the [T, E] split),
    and seed, offset and stream each give a different sequence."""
    z1, u1 = orc.router_draws(12, 5, 8, 2)
    z2, u2 = orc.router_draws(6, 10, 8, 2)
    np.testing.assert_array_equal(z1.reshape(-1), z2.reshape(-1))
    np.testing.assert_array_equal(u1[:6], u2)
    z3, u3 = orc.router_draws(12, 5, 9, 2)
    z4, u4 = orc.router_draws(12, 5, 8, 3)
    assert not np.any(z3 == z1) and not np.any(z4 == z1)
    assert not np.any(u3 == u1) and not np.any(u4 == u1)
    w0 = orc.moe_oracle._draw_words(16, 8, 2, 0)
    w1 = orc.moe_oracle._draw_words(16, 8, 2, 1)
    assert not np.any(w0 == w1)
