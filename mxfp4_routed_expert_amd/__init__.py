"""MI355X-native Kimi K3 Stable LatentMoE routed-expert layer (MXFP4 experts).

The layer runs in hand-written gfx950 HIP kernels behind the C-ABI of
include/k3moe.h (libk3moe.so); ``k3moe`` is its ctypes binding with the same names.
"""
from . import k3moe  # noqa: F401
from .k3moe import (k3moe_combine, k3moe_dispatch, k3moe_expert_glu_mxfp4, k3moe_latent_proj_bf16,  # noqa: F401
                    k3moe_layer, k3moe_route, k3moe_workspace_size)
