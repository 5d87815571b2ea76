"""GPU parity of the layer backward (moe_layer_bwd through the C ABI) against
the CPU oracle.

fp32 layers: every gradient is compared in full with the oracle's chain rule,
max-abs error <= 1e-4 * RMS(reference) (+1e-7).

c5 training shape (bf16 experts, FP32 router), step-wise on the GPU's own
routing.  The bf16 path stores dO = g*dy, the pre-activation h, the
activation a and dH in bf16 (round-to-nearest, relative error <= 2^-8 each)
and accumulates every product in fp32.  A gradient entry sum_r u_r v_r built
from such factors is off by at most a few of these roundings per term, so the
bar is elementwise:
    |got - ref| <= 2^-6 * (|U|^T |V|)   (the sum of absolute terms),
plus an RMS-level check  rms(got - ref) <= 1e-2 * rms(ref).
(A flat max-abs <= 2e-2 * rms bar is wrong for experts with a handful of rows:
replaying the bf16 roundings in fp64 gives 6.9% for a 7-row expert.)
dWg (fp32 router: exact bf16-plane products, fp32 sums over T) keeps
max-abs <= 1e-4 * rms.
"""

import math

import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle as orc
from top_routing_expert_amd import binding as B, presets, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BF16_BOUND = 2.0 ** -6
# Step-wise bar: a product of exact bf16 factors accumulated in fp32 differs
# from float64 only by the order and rounding of its fp32 additions (2^-24 each,
# of random sign): about sqrt(n/16) * 2^-24 of its sum of absolute terms for n
# rows in chains of 16-product MFMA steps, 2^-19 at n = 16384.  2^-16 leaves an
# 8x margin, and a row dropped or counted twice moves an entry by a whole term
# (about sum|terms| / n), 4x the bar or more even for 16384 rows.
STEP_BOUND = 2.0 ** -16


def _train(p, inp):
    x = torch.from_numpy(inp["x"]).to(DEV).to(B.TORCH_DTYPE[p.dtype]).contiguous()
    w = B.weights_to_device(p, inp, DEV)
    ri = B.router_inputs_to_device(inp, DEV)
    saved = B.alloc_saved(p, DEV)
    ws = B.Workspace(DEV)
    y = B.layer_fwd(p, w, x, saved=saved, ri=ri, ws=ws)
    dy = torch.from_numpy(inp["dy"]).to(DEV)
    g = B.layer_bwd(p, w, x, saved, dy, ri=ri, ws=ws)
    torch.cuda.synchronize()
    return x, w, saved, y, g


def _close(got, ref, rel, what):
    got = np.asarray(got, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= rel * rms + 1e-7, f"{what}: max-abs {err:.3e} vs {rel} * rms {rms:.3e}"
    return err / max(rms, 1e-30)


def _bounded(got, ref, cond, what):
    """Elementwise bound BF16_BOUND * cond and an RMS-level check."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    worst = float(np.max(err / (BF16_BOUND * cond + 1e-6 * rms + 1e-30)))
    assert worst <= 1.0, f"{what}: error exceeds 2^-6 * sum|terms| by {worst:.2f}x"
    rel_rms = float(np.sqrt(np.mean(err ** 2))) / max(rms, 1e-30)
    assert rel_rms <= 1e-2, f"{what}: rms error {rel_rms:.3e} of rms(ref)"
    return rel_rms


@pytest.mark.parametrize("over", [
    dict(),
    dict(act="gelu"),
    dict(score="sigmoid", F_shared=64, aux_coef=0.1, z_coef=0.05, sel_bias_std=0.1, zipf_s=1.1,
         gate_scale=math.sqrt(2.0)),
    dict(score="sqrt_softplus", capacity_factor=0.8, aux_coef=0.1, z_coef=0.1, F_shared=128,
         gate_scale=math.sqrt(2.0)),
    dict(T=333, k=3, aux_coef=0.05),
    dict(renorm=False, k=1, z_coef=0.2),
    dict(routing="noisy_topk", aux_coef=0.1, z_coef=0.05, F_shared=64),
    dict(routing="gshard", priority="slot", capacity_factor=0.9, aux_coef=0.1),
    dict(routing="hash", score="sigmoid", aux_coef=0.1),
    # 9..16 slots per token (the 16-slot combine, combine-backward and
    # unpermute kernels), with drops
    dict(E=32, k=12, aux_coef=0.05, capacity_factor=0.7),
    dict(E=32, k=16, score="sigmoid", aux_coef=0.05),
])
def test_layer_bwd_fp32(over):
    p = presets.get("c1", train=True, **over)
    inp = synth.make_inputs(p, seed=5, with_dy=True)
    fk = orc.layer_fwd(p, inp, keep_hidden=True)
    assert not (fk["near_tie"].any() or fk["near_tie_order"].any())
    ref = orc.layer_bwd(p, inp, fk, inp["dy"])
    _, _, saved, y, g = _train(p, inp)
    np.testing.assert_array_equal(saved["topk_idx"].cpu().numpy(),
                                  np.where(fk["active"], fk["idx"], fk["idx"] + p.E))
    names = ("dx", "dWg", "dW13", "dW2") + (("dWs13", "dWs2") if p.F_shared else ())
    if p.routing == "noisy_topk":
        names += ("dW_noise",)
    for name in names:
        _close(g[name].cpu().numpy(), ref[name], 1e-4, name)


def _bwd_terms(X, W13e, W2e, dO, F, act):
    """Oracle expert backward, plus the magnitudes that carry the bf16
    roundings into dH (for the error bounds) and |a|.

    dA = dO W2 can cancel, so its rounding error scales with |dO| |W2|; the
    rounding of the saved pre-activation h moves each activation factor by its
    derivative times h: dsilu(h) by h * dsilu'(h) (dsilu has a zero near
    h = -2.4), silu(h) by h * dsilu(h), gelu'(h) by h * gelu''(h)."""
    h = X @ W13e.T
    cA = np.abs(dO) @ np.abs(W2e)
    if act == "swiglu":
        a = orc.silu(h[:, :F]) * h[:, F:]
        hg, hu = h[:, :F], h[:, F:]
        sg = 1.0 / (1.0 + np.exp(-hg))
        ds = sg * (1 + hg * (1 - sg))
        dds = sg * (1 - sg) * (2 + hg * (1 - 2 * sg))
        adH = np.concatenate([cA * np.abs(hu) * (np.abs(ds) + np.abs(hg * dds)),
                              cA * (np.abs(hg * sg) + np.abs(hg * ds))], 1)
    else:
        a = orc.gelu(h)
        phi = np.exp(-0.5 * h * h) / math.sqrt(2 * math.pi)
        dg1 = 0.5 * (1 + sps.erf(h / math.sqrt(2))) + h * phi
        dg2 = phi * (2 - h * h)
        adH = cA * (np.abs(dg1) + np.abs(h * dg2))
    dX, dW13, dW2 = orc.expert_bwd(X, h, a, W13e, W2e, dO, act)
    return dX, dW13, dW2, adH, np.abs(a)


def _bf16(v):
    """float32 values rounded to bf16 (nearest even), as float64."""
    t = torch.from_numpy(np.ascontiguousarray(v, np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def _np(t, rows=None):
    """A device tensor (bf16 or fp32) as a float64 array, optionally its first rows."""
    t = t if rows is None else t[:rows]
    return t.float().cpu().numpy().astype(np.float64)


def _step_bounded(got, ref, cond, what, tiny=1e-30):
    """Step-wise bar: |got - ref| <= 2^-16 * cond elementwise (cond = sum of
    absolute terms), the products recomputed in float64 from the GPU's own
    bf16 operands."""
    err = np.abs(np.asarray(got, np.float64) - ref)
    worst = float(np.max(err / (STEP_BOUND * cond + tiny))) if err.size else 0.0
    assert worst <= 1.0, f"{what}: step-wise error {worst:.2f}x over 2^-16 * sum|terms|"
    return worst


def _act_bwd_bound(cA, h, F, act):
    """Magnitude through which the errors of dA (bounded by cA = |dO| |W2|) and
    of the epilogue's activation derivative reach dH; the same factors as in
    _bwd_terms."""
    if act == "swiglu":
        hg, hu = h[:, :F], h[:, F:]
        sg = 1.0 / (1.0 + np.exp(-hg))
        ds = sg * (1 + hg * (1 - sg))
        return np.concatenate([cA * np.abs(hu) * (np.abs(ds) + 1.0), cA * (np.abs(hg * sg) + 1.0)], 1)
    phi = np.exp(-0.5 * h * h) / math.sqrt(2 * math.pi)
    dg1 = 0.5 * (1 + sps.erf(h / math.sqrt(2))) + h * phi
    return cA * (np.abs(dg1) + 1.0)


@pytest.mark.parametrize("name,over", [
    ("c2", {}), ("c5", {}),
    # ragged token counts through the bf16 router-gradient GEMMs (chunk tails,
    # one-tile grids) and the router's 32- and 64-token blocks
    ("c5", dict(T=300, d=256, F=256, F_shared=256)),
    ("c4", dict(T=333, d=256, F=256, F_shared=0)),
    ("c2", dict(T=257, d=256, F=512)),
    # 1024 routed rows per expert (the c3 and c4 training shapes' row counts)
    # at small widths, one with the shared expert beside them
    ("c3", dict(T=4096, d=256, F=256)),
    ("c4", dict(T=8192, d=256, F=128, F_shared=128)),
    # long reductions (K >= 10240) whose last, partial round of tiles is cut
    # into K segments (256 compute units): in the down projection and dXp,
    # 291 tiles of 128x128 (35 past one whole round, 4 segments each), and
    # 20 tiles of 128x256 (all split, 4 segments each)
    ("c3", dict(T=4096, E=64, d=384, F=10240)),
    ("c3", dict(T=1024, d=256, F=10240))])
def test_layer_bwd_full_size(name, over):
    """Every expert's dW13 and dW2, every routed row's dH, every token's dx and
    the shared expert's gradients, on the GPU's own routing:
      * step-wise: each product recomputed in float64 from the GPU's bf16
        operands (dO reproduced bit for bit as bf16(gate * dy) in fp32, the
        saved h and a, the returned dH), within 2^-16 of its sum of absolute
        terms; dH within 2^-8 (its bf16 rounding) plus 2^-16 of the magnitude
        its inputs' errors propagate through;
      * end to end: against the oracle's chain rule from x, within 2^-6 of the
        sum of absolute terms and 1e-2 in RMS (the bf16 roundings of dO, h, a
        and dH, each at most 2^-8 relative, compounded)."""
    p = presets.get(name, **over)
    print(f"[{name} {over} bwd] generating inputs", flush=True)
    inp = synth.make_inputs(p, seed=0, with_dy=True)
    x = torch.from_numpy(inp["x"]).to(DEV).to(B.TORCH_DTYPE[p.dtype]).contiguous()
    w = B.weights_to_device(p, inp, DEV)
    saved = B.alloc_saved(p, DEV)
    ws = B.Workspace(DEV)
    B.layer_fwd(p, w, x, saved=saved, ws=ws)
    g = B.layer_bwd(p, w, x, saved, torch.from_numpy(inp["dy"]).to(DEV), ws=ws, want_dH=True)
    torch.cuda.synchronize()
    print(f"[{name} {over} bwd] GPU done; oracle steps", flush=True)
    T, k, E, d, F = p.T, p.k, p.E, p.d, p.F
    idx = saved["topk_idx"].cpu().numpy().astype(np.int64)
    ros = saved["row_of_slot"].cpu().numpy().astype(np.int64)
    offsets = saved["offsets"].cpu().numpy().astype(np.int64)
    counts = saved["counts"].cpu().numpy()
    gate32 = saved["topk_gate"].cpu().numpy()
    R = int(offsets[-1])
    o = saved["o"][:R].cpu().numpy()
    tor = saved["token_of_row"].cpu().numpy()[:R].astype(np.int64)
    slot_of_row = np.zeros(R, np.int64)
    kept = ros >= 0
    slot_of_row[ros[kept]] = np.nonzero(kept)[1]
    X64 = inp["x"].astype(np.float64)
    dy32 = inp["dy"].astype(np.float32)
    dy = dy32.astype(np.float64)
    # the saved activation (its hi half when the layer carries (hi, lo) pairs:
    # the weight gradient of W2 uses hi)
    h_all, a_all, dH_all = _np(saved["h"], R), _np(saved["a"], R)[:, :F], _np(g["dH"], R)

    # router gradient on the GPU's routing and expert outputs
    r = orc.route(inp["x"], inp["Wg"], k, p.score, p.renorm, p.gate_scale, inp["offset"],
                  inp["sel_bias"])
    dg = np.zeros((T, k))
    for j in range(k):
        m = ros[:, j] >= 0
        dg[m, j] = np.sum(dy[m] * o[ros[m, j]], axis=1)
    dz = orc.router_bwd(p, r["s"], r["z"], idx, counts, dg)
    # FP32 router: dWg is formed from exact bf16-plane products with fp32 sums
    e1 = _close(g["dWg"].cpu().numpy(), X64.T @ dz, 1e-4, "dWg")
    print(f"[{name} bwd] dWg max-abs error / rms {e1:.2e}", flush=True)

    Wg = inp["Wg"].astype(np.float64)
    dx_step = dz @ Wg.T
    # the router's term within 1e-3 of its absolute terms (fp32 dz against float64)
    c_step = np.abs(dz) @ np.abs(Wg.T) * (1e-3 / STEP_BOUND)
    dx_ref = dz @ Wg.T
    c_ref = np.abs(dz) @ np.abs(Wg.T)
    dW13, dW2 = g["dW13"], g["dW2"]
    worst = dict(dW2=0.0, dW13=0.0, dH=0.0)
    sizes = np.diff(offsets)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        got13 = dW13[e].cpu().numpy()
        got2 = dW2[e].cpu().numpy()
        if r1 == r0:
            assert not got13.any() and not got2.any(), f"empty expert {e} must have zero grads"
            continue
        toks = tor[r0:r1]
        assert len(np.unique(toks)) == len(toks)
        Xe = X64[toks]
        W13e = inp["W13"][e].astype(np.float64)
        W2e = inp["W2"][e].astype(np.float64)
        g32 = gate32[toks, slot_of_row[r0:r1]]
        dO_bf = _bf16(g32[:, None] * dy32[toks])              # the GPU's dO, bit for bit
        he, ae, dHe = h_all[r0:r1], a_all[r0:r1], dH_all[r0:r1]
        # step-wise, on the GPU's operands
        dX_s, dW13_s, dW2_s, dH_s = orc.expert_bwd(Xe, he, ae, W13e, W2e, dO_bf, p.act, dH_in=dHe,
                                                   keep_dH=True)
        worst["dW2"] = max(worst["dW2"], _step_bounded(got2, dW2_s, np.abs(dO_bf).T @ np.abs(ae),
                                                       f"dW2[{e}] step"))
        worst["dW13"] = max(worst["dW13"], _step_bounded(got13, dW13_s, np.abs(dHe).T @ np.abs(Xe),
                                                         f"dW13[{e}] step"))
        cA = np.abs(dO_bf) @ np.abs(W2e)
        cH = 2.0 ** -8 / STEP_BOUND * np.abs(dH_s) + _act_bwd_bound(cA, he, F, p.act)
        worst["dH"] = max(worst["dH"], _step_bounded(dHe, dH_s, cH, f"dH rows of expert {e}"))
        dx_step[toks] += dX_s
        c_step[toks] += np.abs(dHe) @ np.abs(W13e)
        # end to end, from x
        dO = gate32[toks, slot_of_row[r0:r1], None].astype(np.float64) * dy[toks]
        dX, dW13_ref, dW2_ref, adH, aa = _bwd_terms(Xe, W13e, W2e, dO, F, p.act)
        _bounded(got13, dW13_ref, adH.T @ np.abs(Xe), f"dW13[{e}]")
        _bounded(got2, dW2_ref, np.abs(dO).T @ aa, f"dW2[{e}]")
        dx_ref[toks] += dX
        c_ref[toks] += adH @ np.abs(W13e)
    print(f"[{name} bwd] all {int(np.count_nonzero(sizes))} non-empty experts (rows "
          f"{int(sizes.min())}..{int(sizes.max())}); step-wise worst/bar {worst}", flush=True)

    if p.F_shared:
        Fs = p.F_shared
        Ws13 = inp["Ws13"].astype(np.float64)
        Ws2 = inp["Ws2"].astype(np.float64)
        hs, as_, dHs = _np(saved["h_shared"]), _np(saved["a_shared"]), _np(g["dH_shared"])
        dyb = _bf16(dy32)                                     # the GPU's bf16 copy of dy
        dxs_s, dWs13_s, dWs2_s, dHs_s = orc.expert_bwd(X64, hs, as_, Ws13, Ws2, dyb, "swiglu",
                                                       dH_in=dHs, keep_dH=True)
        _step_bounded(g["dWs2"].cpu().numpy(), dWs2_s, np.abs(dyb).T @ np.abs(as_), "dWs2 step")
        _step_bounded(g["dWs13"].cpu().numpy(), dWs13_s, np.abs(dHs).T @ np.abs(X64), "dWs13 step")
        cHs = 2.0 ** -8 / STEP_BOUND * np.abs(dHs_s) + _act_bwd_bound(
            np.abs(dyb) @ np.abs(Ws2), hs, Fs, "swiglu")
        _step_bounded(dHs, dHs_s, cHs, "dH_shared")
        dx_step += dxs_s
        c_step += np.abs(dHs) @ np.abs(Ws13)
        dxs_ref, dWs13_ref, dWs2_ref, adHs, aas = _bwd_terms(X64, Ws13, Ws2, dy, Fs, "swiglu")
        _bounded(g["dWs13"].cpu().numpy(), dWs13_ref, adHs.T @ np.abs(X64), "dWs13")
        _bounded(g["dWs2"].cpu().numpy(), dWs2_ref, np.abs(dy).T @ aas, "dWs2")
        dx_ref += dxs_ref
        c_ref += adHs @ np.abs(Ws13)

    # every token's dx: the routed rows' dH W13 summed per token, the shared
    # expert's and the router's terms
    dx = g["dx"].cpu().numpy()
    ws_ = _step_bounded(dx, dx_step, c_step, "dx step")
    e2 = _bounded(dx, dx_ref, c_ref, "dx")
    print(f"[{name} bwd] dWg err/rms {e1:.2e}; dx on all {T} tokens: step-wise worst/bar "
          f"{ws_:.2f}, end-to-end rms-err/rms {e2:.2e}")
