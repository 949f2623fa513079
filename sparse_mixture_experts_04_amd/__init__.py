"""Sparse Mixture-of-Experts FFN layer forward on MI355X (gfx950).

The layer -- router, dispatcher, expert Linear-GELU-Linear, weighted combine --
runs in the HIP kernels of libmoe.so behind the C ABI of include/moe.h.  This
package is its thin Python binding (ctypes; torch supplies device memory and
streams) plus buffer plumbing.  Importing it fails loudly when libmoe.so is
missing: there is no CPU or PyTorch fallback.
"""
from ._lib import (MOE_BF16, MOE_ERR_HIP, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED,  # noqa: F401
                   MOE_ERR_WORKSPACE_TOO_SMALL, MOE_F32, MOE_OK, MOE_OP_DISPATCH, MOE_OP_EXPERT_FFN,
                   MOE_OP_FORWARD, MOE_OP_ROUTE, MOE_OP_ROUTE_STATS, MOE_OP_DISPATCH_REROUTE,
                   MOE_OP_FORWARD_REROUTE, EXPORTED, LIB, LIB_PATH, MoeConfig, MoeError,
                   config, moe_capacity_from_factor, moe_combine, moe_dispatch, moe_expert_down, moe_expert_ffn,
                   moe_expert_up,
                   moe_expert_up_gather, moe_expert_up_gather_supported, moe_forward, moe_route, moe_route_stats,
                   moe_workspace_size, moe_route_ranked, moe_dispatch_reroute, moe_forward_reroute, moe_forward_noalloc, NOALLOC_MAX_WORKSPACE_BYTES,
                   status_string, version)
from .layer import ForwardBuffers, MoELayer  # noqa: F401
