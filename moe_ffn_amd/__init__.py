"""MI355X-native ZONOS2 MoE feed-forward layer.

The layer runs in hand-written HIP kernels for gfx950 behind the C ABI of
include/moe_layer.h (libmoe_layer.so, built in-tree by ``python -m
moe_ffn_amd.build``).  This package holds the kernels' sources, the build
step and a ctypes binding; PyTorch is used only for device memory and streams.
"""

from .layer import (  # noqa: F401
    MoELayer, MoEStack, MoELayerError, load_library, LIB_PATH, EXPORTS,
    MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_OOM, MOE_ERR_HIP, MOE_ERR_UNSUPPORTED,
    LayerConfig, LayerWeights, RoutingOut, TIMED_SLOTS, fp8_quantize_rows,
)
