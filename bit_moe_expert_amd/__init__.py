"""Routed int4 mixture-of-experts FFN for AMD MI355X (gfx950).

The computation runs in libmoe_int4.so (hand-written HIP, C ABI in include/moe_int4.h);
``bit_moe_expert_amd.moe`` is its Python binding.
"""
from . import moe  # noqa: F401
from .moe import QProj, QuantFFN, Layer, debug_dequant, expert_ffn, forward_layer, route  # noqa: F401
