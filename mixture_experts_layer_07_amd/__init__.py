"""MI355X-native forward pass of a token-choice MoE FFN layer.

The layer runs in hand-written HIP kernels for gfx950 behind a C ABI
(include/moe.h, built into libmoe_mi355x.so next to this file). The Python
side only marshals arguments: ``mixture_experts_layer_07_amd.binding`` has the
four calls (moe_route, moe_permute, moe_expert_ffn, moe_combine) and
``layer.MoELayer`` strings them together on torch device buffers.

Importing this package does not load the library; ``binding`` loads it on
first use and raises if it is missing.
"""
from .configs import CONFIGS, LayerConfig, active_flops  # noqa: F401

__all__ = ["CONFIGS", "LayerConfig", "active_flops"]
