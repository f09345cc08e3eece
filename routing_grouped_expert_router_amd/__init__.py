"""One MoE layer (router, GPU-resident routing metadata, row permute, grouped
SwiGLU expert GEMMs, weighted combine, and their backward) as hand-written HIP
kernels for AMD Instinct MI355X (gfx950), behind the C ABI in include/moe.h.

Import the binding with ``from routing_grouped_expert_router_amd import _lib``
and the layer driver with ``from routing_grouped_expert_router_amd.layer
import MoELayer``. The shared library is built by ``build.build()``.
"""
