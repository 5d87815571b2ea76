"""moe_permute_noalloc (the dispatch step without a workspace, for callers that
cannot allocate) against moe_permute, through the C ABI: counts, offsets,
row_of_slot, token_of_row and x_perm bit-exact (dispatch is integer and byte
work), on calls in a row on the same GPU, the second smaller than the first.

Collected last (the name): it shares the library's per-GPU scratch array with
nothing else, and a failure here cannot hide the tests before it."""

import numpy as np
import pytest
import torch

from top_routing_expert_amd import binding as B, presets

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _topk_ids(T, E, k, seed, skew):
    """Seeded top-k expert ids with skewed loads (a log-prior on the experts)."""
    rng = np.random.default_rng(seed)
    logits = rng.normal(size=(T, E)) + skew * np.log(np.arange(1, E + 1))[::-1]
    return np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)


def _same(p, x, idx_np):
    idx = torch.from_numpy(idx_np).to(DEV)
    ref = B.permute(p, x, idx)
    T = x.shape[0]
    # poisoned outputs: every entry the call must write starts as garbage
    out = dict(counts=torch.full((p.E,), -7, dtype=torch.int32, device=DEV),
               offsets=torch.full((p.E + 1,), -7, dtype=torch.int32, device=DEV),
               row_of_slot=torch.full((T, p.k), -7, dtype=torch.int32, device=DEV),
               token_of_row=torch.full((max(T * p.k, 1),), -7, dtype=torch.int32, device=DEV),
               x_perm=torch.zeros(max(T * p.k, 1), p.d, dtype=x.dtype, device=DEV))
    got = B.permute_noalloc(p, x, idx, out=out)
    torch.cuda.synchronize()
    R = int(ref["offsets"][-1])
    for n in ("counts", "offsets", "row_of_slot"):
        assert torch.equal(got[n], ref[n]), n
    assert torch.equal(got["token_of_row"][:R], ref["token_of_row"][:R])
    bits = torch.int16 if x.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(got["x_perm"][:R].view(bits), ref["x_perm"][:R].view(bits))
    return R


def test_noalloc_permute_matches_permute_on_calls_in_a_row():
    # 256 experts, top-8, 16384 tokens with skewed loads: the largest layer of
    # the workloads, 256 KiB of the 1 MiB scratch
    p1 = presets.get("c5")
    print(f"[no-alloc] {p1.T} tokens, E={p1.E}, k={p1.k}", flush=True)
    x1 = torch.randn(p1.T, p1.d, device=DEV).to(torch.bfloat16)
    R1 = _same(p1, x1, _topk_ids(p1.T, p1.E, p1.k, 1, 1.1))
    # then a smaller layer whose capacity drops slots (stale tables of the
    # first call still sit in the scratch)
    p2 = presets.get("c2", T=1000, E=8, k=2, capacity_factor=1.0)
    print(f"[no-alloc] {p2.T} tokens, E={p2.E}, k={p2.k}, capacity factor 1.0", flush=True)
    x2 = torch.randn(p2.T, p2.d, device=DEV).to(torch.bfloat16)
    R2 = _same(p2, x2, _topk_ids(p2.T, p2.E, p2.k, 2, 2.0))
    assert R1 == p1.T * p1.k and R2 < p2.T * p2.k
    # and slot priority, fp32 tokens
    p3 = presets.get("c1", T=777, priority="slot", capacity_factor=0.9)
    print(f"[no-alloc] {p3.T} fp32 tokens, slot priority", flush=True)
    x3 = torch.randn(p3.T, p3.d, device=DEV)
    _same(p3, x3, _topk_ids(p3.T, p3.E, p3.k, 3, 2.0))
