"""MI355X-native sparse MoE layer: HIP kernels for gfx950 behind a C ABI.

Importing the package loads nothing native; ``top_routing_expert_amd.binding``
loads ``libmoe.so`` on first use and raises if it is missing.
"""

__all__ = ["presets", "synth"]
