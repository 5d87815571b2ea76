"""GPU parity of quantile balancing (score histogram, bias solve) and of the
router monitoring report, against the CPU oracle on the GPU's own scores,
counts and expert outputs.

Histogram counts are integers decided by one fp32 formula on both sides: they
must match exactly.  The bias solve and the report are fp32 on the GPU and
float64 in the oracle: 2e-6 of the score range for biases, 1e-5 relative for
the report's ratios and norms.
"""

import numpy as np
import pytest
import torch

import oracle as orc
from top_routing_expert_amd import binding as B, presets, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
RANGE = {"softmax": (0.0, 1.0), "sigmoid": (0.0, 1.0), "sqrt_softplus": (0.0, 8.0)}


def _setup(name, **over):
    p = presets.get(name, **over)
    inp = synth.make_inputs(p, seed=0)
    x = torch.from_numpy(inp["x"]).to(DEV).to(B.TORCH_DTYPE[p.dtype]).contiguous()
    w = B.weights_to_device(p, inp, DEV)
    return p, inp, x, w


@pytest.mark.parametrize("name,nbins", [("c4", 256), ("c5", 1024), ("c2", 100)])
def test_histogram_and_quantile_bias_parity(name, nbins):
    p, inp, x, w = _setup(name)
    lo, hi = RANGE[p.score]
    r = B.route(p, x, w.Wg, w.offset, w.sel_bias, want_scores=True)
    hist = B.score_histogram(r["scores"], lo, hi, nbins)
    target = p.T * p.k / p.E
    bias = B.bias_from_histogram(hist, lo, hi, target)
    torch.cuda.synchronize()
    s_gpu = r["scores"].cpu().numpy()
    h_ref = orc.score_histogram(s_gpu, lo, hi, nbins)
    np.testing.assert_array_equal(hist.cpu().numpy(), h_ref)
    b_ref = orc.quantile_bias(h_ref, lo, hi, target)
    err = np.max(np.abs(bias.cpu().numpy() - b_ref))
    assert err <= 2e-6 * (hi - lo), err
    print(f"{name}: bias range [{b_ref.min():.4f}, {b_ref.max():.4f}], max err {err:.2e}")


def test_quantile_bias_flattens_skewed_load():
    """The c4 layer's Zipf-skewed routing, re-routed with the solved bias as its
    selection bias: the load spread collapses in one solve (the fixed-step
    update needs many steps of its gamma)."""
    p, inp, x, w = _setup("c4")
    lo, hi = RANGE[p.score]
    r0 = B.route(p, x, w.Wg, w.offset, w.sel_bias, want_scores=True)
    bias = B.bias_from_histogram(B.score_histogram(r0["scores"], lo, hi, 1024), lo, hi,
                                 p.T * p.k / p.E)
    r1 = B.route(p, x, w.Wg, w.offset, bias)
    rep0 = B.router_report(r0["counts"])["report"]
    rep1 = B.router_report(r1["counts"])["report"]
    torch.cuda.synchronize()
    m0, m1 = float(rep0[0]), float(rep1[0])
    cv0, cv1 = float(rep0[1]), float(rep1[1])
    print(f"c4 max/mean load {m0:.2f} -> {m1:.2f}, CV {cv0:.3f} -> {cv1:.3f}")
    assert m0 > 3.0 and m1 < 1.6 and cv1 < 0.25 * cv0


@pytest.mark.parametrize("name", ["c4", "c5", "c2"])
def test_router_report_parity(name):
    p, inp, x, w = _setup(name)
    saved = B.alloc_saved(p, DEV)
    y, st = B.layer_fwd(p, w, x, saved=saved, stats=True)
    out = B.router_report(st["counts"], st["n_dropped"], saved["o"], saved["offsets"])
    torch.cuda.synchronize()
    counts = st["counts"].cpu().numpy()
    nd = int(st["n_dropped"].cpu()[0])
    ref = orc.load_report(counts, nd)
    offsets = saved["offsets"].cpu().numpy()
    R = int(offsets[-1])
    norms, ratio = orc.expert_output_norms(saved["o"][:R].cpu().numpy(), offsets)
    rep = out["report"].cpu().numpy()
    np.testing.assert_allclose(rep[:4], [ref["max_over_mean"], ref["cv"], ref["drop_rate"], ratio],
                               rtol=1e-5, atol=1e-7)
    assert int(rep[4]) == ref["n_empty"]
    np.testing.assert_allclose(out["expert_norm"].cpu().numpy(), norms, rtol=1e-5, atol=1e-7)
    print(f"{name}: max/mean {rep[0]:.2f}, CV {rep[1]:.3f}, drops {rep[2]:.4f}, "
          f"norm max/median {rep[3]:.2f}, empty {int(rep[4])}")
