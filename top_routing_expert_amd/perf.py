"""Algorithmic work of each step of the MoE layer (FLOPs and HBM bytes).

Only real work is counted: kept rows R (not tile padding), weights of experts
that received at least one row, each tensor read or written once.  These are
the figures the roofline fractions are computed from.

Peaks of one MI355X (AMD's published dense figures): HBM3E 8 TB/s; bf16 MFMA
2.5 PFLOP/s; fp8 MFMA 5.0 PFLOP/s (also the rate of the scaled FP8 x FP4
matrix instruction, whose issue rate is set by its wider operand); fp32 vector 157.3 TFLOP/s (packed), 78.6 TFLOP/s without packed
FP32 instructions.
"""

from __future__ import annotations

import hashlib
import os

from .presets import Preset

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP32_TFLOPS = 157.3


def eb(p: Preset) -> int:
    return 2 if p.dtype == "bf16" else 4


def n_mats(p: Preset) -> int:
    """Matrices per expert: gate, up, down for SwiGLU; up, down for GELU."""
    return 3 if p.act == "swiglu" else 2


def ffn_flops(p: Preset, R: int, shared: bool = True) -> float:
    f = 2.0 * n_mats(p) * p.d * p.F * R
    if shared and p.F_shared:
        f += 2.0 * 3 * p.d * p.F_shared * p.T
    return f


def ffn_bytes(p: Preset, R: int, active_experts: int, shared: bool = True) -> float:
    """Algorithmic HBM bytes of the routed expert FFN: the weights of the active
    experts read once, the x_perm rows read once and the fp32 output rows
    written once.  The activation between the two projections is an
    intermediate (a fused FFN keeps it on chip), so it is not counted."""
    b = active_experts * n_mats(p) * p.d * p.F * eb(p)
    b += R * p.d * eb(p) + R * p.d * 4
    if shared and p.F_shared:
        b += 3 * p.d * p.F_shared * eb(p) + p.T * p.d * eb(p) + p.T * p.d * 4
    return float(b)


def ffn_bytes_unfused(p: Preset, R: int, active_experts: int) -> float:
    """What the two-launch FFN moves at best: ffn_bytes plus the activation
    written by the up projection and read back by the down projection."""
    return ffn_bytes(p, R, active_experts, shared=False) + 2.0 * R * p.F * eb(p)


def ffn_roofline_s(p: Preset, R: int, active_experts: int) -> tuple:
    """(seconds, bound) of the routed expert FFN at the bf16 MFMA peak or the
    HBM peak, whichever is longer."""
    t_mfma = ffn_flops(p, R, shared=False) / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = ffn_bytes(p, R, active_experts, shared=False) / (PEAK_HBM_GBS * 1e9)
    return (t_mfma, "mfma") if t_mfma >= t_hbm else (t_hbm, "hbm")


def ffn_mx_bytes(p: Preset, R: int, active_experts: int) -> float:
    """MXFP4 routed expert FFN: FP4 weights (half a byte per element) and their
    E8M0 scales (one per 32) of active experts, FP8 x_perm and its scales (one
    per 64), FP8 activation and scales written then read, fp32 output written."""
    w = active_experts * n_mats(p) * p.d * p.F
    b = w // 2 + w // 32
    b += R * p.d + R * p.d // 64 + 2 * (R * p.F + R * p.F // 64) + R * p.d * 4
    return float(b)


def route_flops(p: Preset) -> float:
    return 2.0 * p.T * p.d * p.E


def route_roofline_s(p: Preset) -> float:
    """Binding roofline of the router: its HBM bytes at the HBM peak, or, for
    bf16 tokens, the logits contraction as three exact bf16 planes of Wg on the
    bf16 matrix cores (fp32 tokens: the fp32 vector peak), whichever is longer."""
    if p.dtype == "bf16":
        t_math = 3 * route_flops(p) / (PEAK_BF16_TFLOPS * 1e12)
    else:
        t_math = route_flops(p) / (PEAK_FP32_TFLOPS * 1e12)
    return max(route_bytes(p) / (PEAK_HBM_GBS * 1e9), t_math)


def route_bytes(p: Preset) -> float:
    """x read once, Wg read once, indices and gates written."""
    return float(p.T * p.d * eb(p) + p.d * p.E * 4 + p.T * p.k * 8)


def permute_bytes(p: Preset, R: int) -> float:
    """x read once, R rows written, indices read, slot/row maps written."""
    return float(p.T * p.d * eb(p) + R * p.d * eb(p) + p.T * p.k * 8 + R * 4)


def combine_bytes(p: Preset, R: int) -> float:
    """fp32 expert rows read once, y written, gates and rows read (+ shared)."""
    b = R * p.d * 4 + p.T * p.d * 4 + p.T * p.k * 8
    if p.F_shared:
        b += p.T * p.d * 4
    return float(b)


# Sources of the grouped-GEMM kernels: measured hardware byte counts of the
# expert FFN are valid only for the sources they were taken on.
GEMM_SOURCES = ("gemm_bf16.hip", "gemm_common.hpp", "common.hpp", "kernels.hpp")


def gemm_source_sha256() -> str:
    h = hashlib.sha256()
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    for f in GEMM_SOURCES:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()
