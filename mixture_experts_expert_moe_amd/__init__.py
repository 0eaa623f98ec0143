"""Routed Mixture-of-Experts FFN layer for AMD MI355X (gfx950).

The compute path is libmoe_gfx950.so (HIP kernels behind the C ABI of
include/moe.h); `moe` is its thin ctypes binding.
"""
from . import moe  # noqa: F401
from .moe import (MoeLayer, make_desc, moe_buffer_sizes, moe_combine, moe_grouped_gemm_down,  # noqa: F401
                  moe_grouped_gemm_gu, moe_permute, moe_rmsnorm, moe_route_topk)
