"""MI355X-native MoE-layer hot path: route, co-activation histogram, dispatch
layout, grouped SwiGLU expert FFN and combine, as hand-written gfx950 HIP
kernels behind the C ABI in include/moe.h.

Importing the package loads nothing; ``routing_dispatch_expert_top_amd.ops``
loads the HIP library on first use and fails loudly if it is missing.
"""
__all__ = ["synth", "ops"]
