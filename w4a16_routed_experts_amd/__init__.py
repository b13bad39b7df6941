"""Routed MoE FFN under W4A16 on MI355X: Python binding of libmoe_w4a16.so.

The binding only marshals arguments: torch tensors supply device memory and
the current HIP stream, and every step of the layer runs in the library's HIP
kernels.  There is no fallback: if the library is missing or the device is not
gfx950, calls raise.
"""
from .binding import (  # noqa: F401
    MoeDims,
    MoeWeights,
    MoeError,
    PATH_AUTO,
    PATH_DECODE,
    PATH_CHUNK,
    DEBUG_WAIT_GIVE_UP,
    FMT_AFFINE4,
    NORM_GAIN_PLUS_ONE,
    GIVE_UP_WORD_OFFSET,
    lib,
    library_path,
    moe_workspace_bytes,
    moe_status_string,
    moe_route,
    moe_experts_w4a16,
    moe_forward,
    moe_forward_noalloc,
    NOALLOC_SCRATCH_BYTES,
    moe_block_forward,
    moe_layers_workspace_bytes,
    moe_layers_forward,
    layers_workspace,
    LayerStack,
    DeviceWeights,
    make_dims,
    workspace,
)
