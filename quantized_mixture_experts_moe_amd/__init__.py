"""Routed int4 Mixture-of-Experts FFN layer for AMD Instinct MI355X (gfx950).

The compute path is libmoe.so (hand-written HIP kernels behind the C ABI in
include/moe.h); ``quantized_mixture_experts_moe_amd.moe`` is its Python
binding.  Build with ``python -m quantized_mixture_experts_moe_amd.build``.
"""
