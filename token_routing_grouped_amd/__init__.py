"""MI355X (gfx950) local MoE expert layer.

Python binding of the C ABI in ``include/moe.h`` (``libmoe.so``): argument
marshalling only. Every step runs in the HIP kernels of the library; PyTorch
provides device memory and the stream. There is no fallback: if the library is
not built, importing the binding raises.
"""
from ._binding import (  # noqa: F401
    MOE_BF16, MOE_FP32, MOE_GATEUP_INTERLEAVED, MOE_GATEUP_CONCAT, MOE_DEV_BAD_EXPERT, MOE_DEV_OVER_CAPACITY,
    MoeError, Metadata, lib, moe_build_metadata, moe_build_metadata_workspace,
    moe_expert_forward, moe_expert_forward_workspace, moe_expert_backward,
    moe_expert_backward_workspace, moe_status_string, EXPORTED_SYMBOLS, KERNELS,
    moe_time_kernel, moe_kernel_name, moe_route, moe_route_workspace, MOE_ROUTE_SOFTMAX_TOPK,
    MOE_ROUTE_TOPK_SOFTMAX, moe_build_metadata_noalloc, MOE_NOALLOC_SCRATCH_BYTES,
)
