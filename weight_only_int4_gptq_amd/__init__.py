"""weight_only_int4_gptq_amd: weight-only INT4 (AWQ / GPTQ, W4A16) linear
layers for AMD Instinct MI355X (gfx950).

The product is the C-ABI library libw4hip (include/w4hip.h, sources in
csrc/).  ``_abi`` binds its calls under the same names; ``layer`` wraps the
create_weights / process_weights_after_loading / apply lifecycle with torch
allocations.  Build with ``python -m weight_only_int4_gptq_amd.build``.
"""
from ._abi import (  # noqa: F401
    W4Error, W4_OK, W4_ERR_INVALID_ARGUMENT, W4_ERR_UNSUPPORTED, W4_ERR_WORKSPACE, W4_ERR_HIP,
    W4_FP16, W4_BF16, w4_layer, w4_sizes_t, make_layer, lib,
    w4_check_layer, w4_sizes, w4_workspace_size, w4_kernel_name, w4_launch_dims, w4_status_str,
    w4_repack_awq, w4_repack_gptq, w4a16_linear, w4_dequant_dense, w4a16_moe_linear,
    w4a16_linear_noalloc, w4_noalloc_scratch_bytes,
    w4a8_quantize, w4a8_workspace_size, w4a8_linear, w4a8_kernel_name,
)


def __getattr__(name):
    # torch is imported lazily so that the host-only calls work without it
    if name in ("W4A16Linear", "W4A16MoELinear"):
        from . import layer
        return getattr(layer, name)
    raise AttributeError(name)
