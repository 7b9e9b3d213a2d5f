"""MI355X (gfx950) sparse mixture-of-experts FFN layer behind a C ABI.

The library (libmoe.so, built from csrc/ by ``build.py``) exports the calls
declared in include/moe.h: moe_route, moe_permute, moe_quantize_act,
moe_expert_ffn, moe_combine, their fused forms (moe_route_permute,
moe_expert_ffn_combine, moe_expert_ffn_combine_slots), expert packing and the
expert slot cache.  ``binding`` is a thin ctypes layer over them,
``layer.MoELayer`` runs one layer end to end and ``stack.ExpertStack`` the
48-layer stack over the slot pool.  Importing this package does not load the library; the
first call does, and fails loudly if it has not been built.
"""
from . import binding  # noqa: F401  (ctypes only; loads libmoe.so lazily)

__all__ = ["binding"]
