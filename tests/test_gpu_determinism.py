"""Determinism and anomaly reporting of the layer on the GPU (through the C ABI).

* Bitwise repeatability: no atomics decide any order and every reduction runs
  in a fixed order, so ten training steps (forward + backward) of the
  256-expert layer, and steps issued on a second caller stream (which gets its
  own internal side stream), give identical bits in y, the router losses, dx
  and every weight gradient.
* Non-finite router logits are counted in moe_stats.n_nonfinite, never
  trapped: tokens with NaN or infinite inputs are reported one each.
"""

import numpy as np
import pytest
import torch

from top_routing_expert_amd import binding as B, presets, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _step(layer, x, dy):
    y = layer.fwd(x).clone()
    g = layer.bwd(x, dy)
    out = {"y": y, "losses": layer.saved["losses"].clone()}
    out.update({k: v.clone() for k, v in g.items() if v is not None})
    return out


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def test_training_step_bitwise_repeatable_across_runs_and_streams():
    p = presets.get("c5")
    print("[determinism] c5 inputs", flush=True)
    inp = synth.make_inputs(p, seed=0, with_dy=True)
    x = torch.from_numpy(inp["x"]).to(DEV).to(torch.bfloat16).contiguous()
    w = B.weights_to_device(p, inp, DEV)
    dy = torch.from_numpy(inp["dy"]).to(DEV)
    layer = B.Layer(p, w, DEV, train=True)
    ref = _step(layer, x, dy)
    torch.cuda.synchronize()
    names = sorted(ref)
    assert {"y", "losses", "dx", "dWg", "dW13", "dW2", "dWs13", "dWs2"} <= set(names)
    for i in range(9):
        got = _step(layer, x, dy)
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(_bits(got[n]), _bits(ref[n])), f"run {i + 2}: {n} differs"
    # a second caller stream, with a fresh layer object (own workspace)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer2 = B.Layer(p, w, DEV, train=True)
        got = _step(layer2, x, dy)
    torch.cuda.synchronize()
    for n in names:
        assert torch.equal(_bits(got[n]), _bits(ref[n])), f"second stream: {n} differs"
    print(f"[determinism] c5: 10 runs and a second stream bitwise equal in {names}")


def test_nonfinite_tokens_are_counted():
    p = presets.get("c4", T=2048)
    inp = synth.make_inputs(p, seed=3)
    x = torch.from_numpy(inp["x"]).to(DEV).to(torch.bfloat16).contiguous()
    bad = {3: float("nan"), 7: float("inf"), 100: float("-inf"), 1500: float("nan")}
    for t, v in bad.items():
        x[t, t % p.d] = v
    x[200, :] = float("nan")                       # a whole row
    w = B.weights_to_device(p, inp, DEV)
    y, st = B.layer_fwd(p, w, x, stats=True)
    torch.cuda.synchronize()
    assert int(st["n_nonfinite"].cpu()[0]) == len(bad) + 1
    good = np.ones(p.T, bool)
    good[list(bad) + [200]] = False
    assert torch.isfinite(y[torch.from_numpy(good).to(DEV)]).all()
    # a clean batch reports none
    x0 = torch.from_numpy(inp["x"]).to(DEV).to(torch.bfloat16).contiguous()
    _, st0 = B.layer_fwd(p, w, x0, stats=True)
    torch.cuda.synchronize()
    assert int(st0["n_nonfinite"].cpu()[0]) == 0
