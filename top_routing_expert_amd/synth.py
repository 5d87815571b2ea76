"""Seeded synthetic inputs for the sparse MoE layer.

This module is shared by the tests, the benchmark and the oracle's callers.
It holds no arithmetic of the method itself: it only draws random tensors,
rounds them to the storage format the layer reads (bf16, round-to-nearest-even)
and builds the per-expert Zipf logit offset that skews expert popularity.

Every tensor has its own child stream of ``np.random.SeedSequence(seed)``, in a
fixed order (x, W_g, zipf permutation, selection bias, W13, W2, shared expert,
dy), and the expert weights have one grandchild stream per expert, so any one
expert can be regenerated alone.

Storage formats and layouts (row-major):
  x      [T, d]        float32 holding bf16-representable values when dtype=bf16
  Wg     [d, E]        float32 router weight (z = x @ Wg)
  offset [E] | None    float32 per-expert logit offset (Zipf skew)
  sel_bias [E] | None  float32 selection-only bias
  W13    [E, n_up, d]  expert up projection, nn.Linear [out, in]; for SwiGLU rows
                       0..F-1 are the gate and F..2F-1 the up projection
  W2     [E, d, F]     expert down projection
  Ws13   [2Fs, d], Ws2 [d, Fs]   shared SwiGLU expert, or None
  dy     [T, d]        float32 upstream gradient (training presets)
"""

from __future__ import annotations

import numpy as np

from .presets import Preset

_STREAMS = ("x", "Wg", "zipf_perm", "sel_bias", "W13", "W2", "shared", "dy",
            "W_noise", "noise", "uniform", "token_ids")
VOCAB = 65536   # token-id range of the hash-routing inputs


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32.

    A storage-format conversion: the result is exactly what a bf16 tensor holds.
    Inputs are finite Gaussian draws, so NaN handling is not needed here.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    out = np.empty_like(u)
    step = 1 << 24
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    for s in range(0, flat_u.size, step):
        v = flat_u[s:s + step]
        lsb = (v >> np.uint32(16)) & np.uint32(1)
        flat_o[s:s + step] = (v + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return out.view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float, bf16: bool) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return bf16_round(a) if bf16 else a


def zipf_offset(E: int, s: float, rng: np.random.Generator) -> np.ndarray:
    """Per-expert logit offset ln(E * p_r(e)) with p_r proportional to r^-s.

    r(e) is a seeded permutation of the ranks 1..E, so which experts are hot is
    random but the popularity profile is Zipf(s).  Added to the router logits
    this acts as a log-prior on expert selection.
    """
    ranks = rng.permutation(E) + 1
    w = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    p = w / w.sum()
    return np.log(E * p[ranks - 1]).astype(np.float32)


def make_inputs(p: Preset, seed: int = 0, with_dy: bool | None = None,
                experts: bool = True) -> dict:
    """Draw every input of preset ``p`` from ``SeedSequence(seed)``."""
    bf16 = p.dtype == "bf16"
    ss = dict(zip(_STREAMS, np.random.SeedSequence(seed).spawn(len(_STREAMS))))
    rng = {name: np.random.default_rng(s) for name, s in ss.items()}
    out: dict = {}
    out["x"] = _normal(rng["x"], (p.T, p.d), p.x_std, bf16)
    out["Wg"] = _normal(rng["Wg"], (p.d, p.E), p.wg_std, False)
    out["offset"] = (zipf_offset(p.E, p.zipf_s, rng["zipf_perm"])
                     if p.zipf_s is not None else None)
    out["sel_bias"] = (_normal(rng["sel_bias"], (p.E,), p.sel_bias_std, False)
                       if p.sel_bias_std is not None else None)
    if experts:
        out["W13"] = expert_weights(p, "W13", seed)
        out["W2"] = expert_weights(p, "W2", seed)
        if p.F_shared > 0:
            sh = [np.random.default_rng(c) for c in ss["shared"].spawn(2)]
            out["Ws13"] = _normal(sh[0], (2 * p.F_shared, p.d), p.w_std, bf16)
            out["Ws2"] = _normal(sh[1], (p.d, p.F_shared), p.w_std, bf16)
        else:
            out["Ws13"] = out["Ws2"] = None
    # inputs of the variant routers: the noise projection and its standard-normal
    # draws (noisy top-k), one uniform draw per token (random second expert),
    # token ids (hash routing)
    out["W_noise"] = out["noise"] = out["uniform"] = out["token_ids"] = None
    if p.routing == "noisy_topk":
        out["W_noise"] = _normal(rng["W_noise"], (p.d, p.E), p.wg_std, False)
        out["noise"] = rng["noise"].standard_normal((p.T, p.E), dtype=np.float32)
    elif p.routing == "gshard":
        out["uniform"] = rng["uniform"].random(p.T, dtype=np.float32)
    elif p.routing == "hash":
        out["token_ids"] = rng["token_ids"].integers(0, VOCAB, p.T, dtype=np.int32)
    if with_dy is None:
        with_dy = p.train
    out["dy"] = _normal(rng["dy"], (p.T, p.d), 1.0, False) if with_dy else None
    return out


def expert_weights(p: Preset, which: str, seed: int = 0, only=None) -> np.ndarray:
    """W13 [E, n_up, d] or W2 [E, d, F]; ``only`` regenerates a subset of experts."""
    bf16 = p.dtype == "bf16"
    root = np.random.SeedSequence(seed).spawn(len(_STREAMS))[_STREAMS.index(which)]
    kids = root.spawn(p.E)
    shape = (p.n_up, p.d) if which == "W13" else (p.d, p.F)
    ids = range(p.E) if only is None else list(only)
    out = np.empty((len(ids),) + shape, dtype=np.float32)
    for i, e in enumerate(ids):
        out[i] = _normal(np.random.default_rng(kids[e]), shape, p.w_std, bf16)
    return out
