"""Fused MoE routed-expert layer for AMD Instinct MI355X (gfx950).

The layer's steps run in the HIP kernels of ``libmoe_gfx950.so`` behind the
C ABI of ``include/moe.h``; this package is its thin Python binding plus a
small holder (``FusedMoE``) that keeps kernel-layout weights and a workspace
in torch-allocated device memory.
"""

from ._lib import (  # noqa: F401
    FMT, EXPORTS, Activation, MoEError, LIB_PATH, lib_handle,
    moe_get_block_m, moe_workspace_bytes, moe_transform_weights, moe_quantize_weights,
    moe_quantize_x, moe_dispatch, moe_forward, moe_route,
)
from .layer import FusedMoE  # noqa: F401
