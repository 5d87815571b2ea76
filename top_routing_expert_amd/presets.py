"""Workload presets for the sparse MoE layer.

Each preset is plain data: the layer's problem statement (tokens T, hidden d,
experts E, top-k, expert width F, scoring function, capacity factor, shared
expert) and the recipe for its seeded synthetic inputs.  Nothing here computes
any part of the method.

Sources for the shapes and rules:
  * The Ultimate MoE Training Handbook (digest, "what MoE saves"): the
    fine-grained example of 64 experts, top-8, expert width 1024, which has the
    active width of a dense 8192 FFN.
  * Hugging Face 30k-word MoE handbook news digest ("confirmed" bullets):
    sigmoid and sqrt(softplus) router scoring, a routing scale near sqrt(k),
    fixed-step loss-free bias updates, shared experts.
  * Mixture of Experts Explained, "Switch Transformers": top-1 routing, expert
    capacity from a capacity factor, bf16 experts with a full-precision router.
  * Mixture of Experts Explained, "What is sparsity?": softmax gating, keep the
    top-k, softmax over the kept logits.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional


@dataclass(frozen=True)
class Preset:
    name: str
    T: int                      # tokens in the batch
    d: int                      # hidden size
    E: int                      # routed experts
    k: int                      # experts kept per token
    F: int                      # routed expert FFN width
    act: str                    # "swiglu" | "gelu"
    score: str                  # "softmax" | "sigmoid" | "sqrt_softplus"
    renorm: bool                # renormalise the kept gates to sum to 1
    gate_scale: float           # multiplies the kept gates after renorm
    capacity_factor: float      # <= 0: no capacity limit
    F_shared: int = 0           # width of the one shared SwiGLU expert, 0 = none
    dtype: str = "bf16"         # "f32" | "bf16": x and expert weights
    aux_coef: float = 0.0       # load-balance loss coefficient (0 = off)
    z_coef: float = 0.0         # router z-loss coefficient (0 = off)
    bias_gamma: float = 0.0     # fixed step of the loss-free bias update (0 = off)
    routing: str = "topk"       # "topk" | "uniform" | "noisy_topk" | "gshard" | "hash"
    priority: str = "token"     # capacity overflow order: "token" (index) | "slot" (top-1 first)
    act_pair: bool = False      # routed activation into the down projection as a bf16 (hi, lo) pair
    # ---- synthetic input recipe (all standard deviations) ----
    x_std: float = 1.0
    wg_std: float = 0.02        # router weight W_g [d, E], fp32
    w_std: float = 0.02         # expert and shared-expert weights
    zipf_s: Optional[float] = None      # per-expert Zipf logit offset
    sel_bias_std: Optional[float] = None  # selection-only bias
    train: bool = False         # forward + backward

    def with_(self, **kw) -> "Preset":
        return replace(self, **kw)

    @property
    def n_up(self) -> int:
        """Rows of the fused up projection per expert: 2F for SwiGLU, F for GELU."""
        return 2 * self.F if self.act == "swiglu" else self.F


def _inv_sqrt(d: int) -> float:
    # "N(0, 1/d)" is read as variance 1/d, i.e. standard deviation 1/sqrt(d).
    return 1.0 / math.sqrt(d)


PRESETS = {
    # Tiny fp32 layer: softmax router renormalised over the top-2, SwiGLU
    # experts of width 128, capacity factor 1.25.
    "c1": Preset("c1", T=256, d=64, E=8, k=2, F=128, act="swiglu", score="softmax",
                 renorm=True, gate_scale=1.0, capacity_factor=1.25, dtype="f32",
                 wg_std=_inv_sqrt(64), w_std=_inv_sqrt(64)),
    # Switch-style top-1 layer: GELU experts of width 4096, capacity factor
    # 1.0, the raw softmax probability of the chosen expert as its gate,
    # aux load-balance and z losses on.  The raw gates peak at about four
    # times their RMS, which scales the single bf16 rounding of the activation
    # past 2e-2 of RMS(y) on a few tokens, so the activation enters the down
    # projection as a (hi, lo) bf16 pair.
    "c2": Preset("c2", T=8192, d=1024, E=32, k=1, F=4096, act="gelu", score="softmax",
                 renorm=False, gate_scale=1.0, capacity_factor=1.0, dtype="bf16",
                 aux_coef=1e-2, z_coef=1e-3, wg_std=0.02, w_std=0.02, act_pair=True),
    # Mixtral-shaped 8-expert top-2 layer, no capacity limit.
    "c3": Preset("c3", T=4096, d=4096, E=8, k=2, F=14336, act="swiglu", score="softmax",
                 renorm=True, gate_scale=1.0, capacity_factor=0.0, dtype="bf16",
                 wg_std=_inv_sqrt(4096), w_std=_inv_sqrt(4096)),
    # Fine-grained layer: 64 experts, top-8, width 1024, one shared expert of
    # width 1024, sigmoid scores plus a selection-only bias, gates normalised
    # over the top-8 and scaled by sqrt(8), Zipf-skewed router logits.
    "c4": Preset("c4", T=16384, d=2048, E=64, k=8, F=1024, act="swiglu", score="sigmoid",
                 renorm=True, gate_scale=math.sqrt(8.0), capacity_factor=0.0,
                 F_shared=1024, dtype="bf16", wg_std=_inv_sqrt(2048), w_std=_inv_sqrt(2048),
                 zipf_s=1.1, sel_bias_std=0.1),
    # Training step of the fine-grained layer with 256 experts of width 512
    # and sqrt(softplus) scoring; keeps c4's shared expert, skew, bias and
    # sqrt(k) scale.
    "c5": Preset("c5", T=16384, d=2048, E=256, k=8, F=512, act="swiglu",
                 score="sqrt_softplus", renorm=True, gate_scale=math.sqrt(8.0),
                 capacity_factor=0.0, F_shared=1024, dtype="bf16", aux_coef=1e-2,
                 z_coef=1e-3, bias_gamma=1e-3, wg_std=_inv_sqrt(2048),
                 w_std=_inv_sqrt(2048), zipf_s=1.1, sel_bias_std=0.1, train=True),
}


def get(name: str, **overrides) -> Preset:
    p = PRESETS[name]
    return p.with_(**overrides) if overrides else p
