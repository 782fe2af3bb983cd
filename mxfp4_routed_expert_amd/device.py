"""Device-memory plumbing: torch allocates HBM, the generated host arrays are copied in,
and the ctypes views of the weights are assembled for the C-ABI. No arithmetic of the
layer happens here."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import k3moe


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


@dataclasses.dataclass
class DeviceLayer:
    dims: object
    w_router: torch.Tensor
    bias: torch.Tensor
    w_down: torch.Tensor
    w_up: torch.Tensor
    norm_w: torch.Tensor
    experts: torch.Tensor       # uint8 [E * blob_bytes]: per-expert records back to back
    blob_bytes: int
    offsets: dict
    gemm_scales: torch.Tensor | None = None  # the experts' scales turn-major (k3moe_prepare_gemm_scales)
    router_planes: torch.Tensor | None = None  # w_router as three bf16 planes (k3moe_prepare_router_planes)

    def experts_struct(self) -> k3moe.k3moe_experts:
        base = self.experts.data_ptr()
        B = self.blob_bytes

        def mx(p, s):
            return k3moe.k3moe_mxfp4(base + self.offsets[p], base + self.offsets[s], B, B)
        return k3moe.k3moe_experts(mx("w1p", "w1s"), mx("w3p", "w3s"), mx("w2p", "w2s"))

    def weights_struct(self, gemm_scales: bool = True, router_planes: bool = True) -> k3moe.k3moe_weights:
        """gemm_scales=False leaves the turn-major copy out (the GEMM then reads the plain scales);
        router_planes=False leaves the router plane copy out (split on every call instead)."""
        gs = self.gemm_scales.data_ptr() if (gemm_scales and self.gemm_scales is not None) else None
        rp = self.router_planes.data_ptr() if (router_planes and self.router_planes is not None) else None
        return k3moe.k3moe_weights(self.w_router.data_ptr(), self.bias.data_ptr(), self.w_down.data_ptr(),
                                   self.w_up.data_ptr(), self.norm_w.data_ptr(), self.experts_struct(), gs, rp)

    def prepare_router_planes(self):
        """Allocate and fill the router's three bf16 planes (once per router matrix)."""
        n = k3moe.k3moe_router_planes_size(self.dims)
        self.router_planes = torch.empty(max(n, 16) // 2, dtype=torch.int16, device=self.w_router.device)
        k3moe.k3moe_prepare_router_planes(self.dims, self.w_router, self.router_planes)
        torch.cuda.synchronize(self.w_router.device)

    def prepare_gemm_scales(self):
        """Allocate and fill the turn-major scale copy (once per set of expert weights)."""
        n = k3moe.k3moe_gemm_scales_size(self.dims)
        self.gemm_scales = torch.empty(max(n, 256), dtype=torch.uint8, device=self.experts.device)
        k3moe.k3moe_prepare_gemm_scales(self.dims, self.experts_struct(), self.gemm_scales)
        torch.cuda.synchronize(self.experts.device)


def upload_layer(dims, dense: dict, expert_chunks, blob_bytes: int, offsets: dict, device="cuda",
                 gemm_scales: bool = True, router_planes: bool = True) -> DeviceLayer:
    """dense: host arrays (w_router fp32 [E,H], bias fp32 [E], w_down/w_up bf16 bits, norm_w fp32).
    expert_chunks: iterable of (first expert, uint8 blob array) covering experts 0..E-1 in order;
    each chunk is copied into one preallocated device buffer, so host memory stays at one chunk.
    gemm_scales: also make the turn-major scale copy that the prefill GEMM reads.
    router_planes: also make the router's bf16 plane copy that the front's GEMM form reads."""
    E = dims.n_experts
    ex = torch.empty(E * blob_bytes, dtype=torch.uint8, device=device)
    for e0, arr in expert_chunks:
        n = arr.size
        ex[e0 * blob_bytes: e0 * blob_bytes + n].copy_(torch.from_numpy(arr), non_blocking=False)
    layer = DeviceLayer(
        dims=dims,
        w_router=_dev(dense["w_router"].astype(np.float32), device),
        bias=_dev(dense["bias"].astype(np.float32), device),
        w_down=_dev(dense["w_down"].view(np.int16), device),
        w_up=_dev(dense["w_up"].view(np.int16), device),
        norm_w=_dev(dense["norm_w"].astype(np.float32), device),
        experts=ex, blob_bytes=blob_bytes, offsets=dict(offsets))
    if gemm_scales:
        layer.prepare_gemm_scales()
    if router_planes:
        layer.prepare_router_planes()
    return layer


def workspace(dims, T: int, device="cuda") -> torch.Tensor:
    n = k3moe.k3moe_workspace_size(dims, T)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def shared_workspace(dims, n_shared: int, T: int, device="cuda") -> torch.Tensor:
    n = k3moe.k3moe_shared_workspace_size(dims, n_shared, T)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def upload_shared(sh: dict, device="cuda") -> dict:
    """The fused shared experts' sh1, sh3, sh2 (bf16 bits) as device tensors."""
    return {k: _dev(sh[k].view(np.int16), device) for k in ("sh1", "sh3", "sh2")}
