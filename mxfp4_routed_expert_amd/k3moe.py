"""ctypes binding of the k3moe C-ABI (include/k3moe.h). Argument marshalling only:
every step of the layer runs in the HIP kernels of libk3moe.so.

Pointers may be given as torch tensors (their data_ptr is passed) or as plain ints.
A stream may be a torch.cuda.Stream, a raw hipStream_t int, or None (the current
torch stream when torch is importable, else the default stream).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libk3moe.so")

K3MOE_OK = 0
K3MOE_EINVAL = -1
K3MOE_EUNSUPPORTED = -2
K3MOE_EWORKSPACE = -3
K3MOE_EHIP = -4


class K3MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} ({status})")
        self.status = status


class k3moe_dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("latent", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("topk", ctypes.c_int32), ("group", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("routed_scale", ctypes.c_float), ("eps", ctypes.c_float),
                ("b1", ctypes.c_float), ("b2", ctypes.c_float), ("topp", ctypes.c_float),
                ("idot", ctypes.c_int32)]


class k3moe_mxfp4(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("packed_expert_stride", ctypes.c_int64), ("scales_expert_stride", ctypes.c_int64)]


class k3moe_experts(ctypes.Structure):
    _fields_ = [("w1", k3moe_mxfp4), ("w3", k3moe_mxfp4), ("w2", k3moe_mxfp4)]


class k3moe_weights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("norm_w", ctypes.c_void_p), ("ex", k3moe_experts),
                ("gemm_scales", ctypes.c_void_p), ("router_planes", ctypes.c_void_p)]


EXPORTS = ["k3moe_workspace_size", "k3moe_route", "k3moe_latent_proj_bf16", "k3moe_dispatch",
           "k3moe_expert_glu_mxfp4", "k3moe_combine", "k3moe_layer", "k3moe_layer_noalloc",
           "k3moe_shared_workspace_size", "k3moe_shared_glu_bf16", "k3moe_gemm_scales_size",
           "k3moe_prepare_gemm_scales", "k3moe_router_planes_size", "k3moe_prepare_router_planes",
           "k3moe_status_str"]

_lib = None


def load(path: str | None = None):
    """Load libk3moe.so (built in place by mxfp4_routed_expert_amd.build). Raises if it
    is missing and cannot be built: there is no other implementation to fall back on."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    try:
        # torch ships a HIP runtime of its own: it must be the one loaded first, so that this
        # library binds to it and its kernels run on torch's streams and memory
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(p):
        from . import build as _build
        _build.build()
    L = ctypes.CDLL(p)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(k3moe_dims)
    L.k3moe_workspace_size.argtypes = [D, i32, ctypes.POINTER(sz)]
    L.k3moe_gemm_scales_size.argtypes = [D, ctypes.POINTER(sz)]
    L.k3moe_prepare_gemm_scales.argtypes = [D, ctypes.POINTER(k3moe_experts), vp, sz, vp]
    L.k3moe_router_planes_size.argtypes = [D, ctypes.POINTER(sz)]
    L.k3moe_prepare_router_planes.argtypes = [D, vp, vp, sz, vp]
    L.k3moe_route.argtypes = [D, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.k3moe_latent_proj_bf16.argtypes = [D, i32, vp, vp, vp, vp, sz, vp]
    L.k3moe_dispatch.argtypes = [D, i32, vp, vp, vp, vp, vp, sz, vp]
    L.k3moe_expert_glu_mxfp4.argtypes = [D, i32, vp, ctypes.POINTER(k3moe_experts), vp, vp, vp, vp, sz, vp]
    L.k3moe_combine.argtypes = [D, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.k3moe_layer.argtypes = [D, i32, vp, ctypes.POINTER(k3moe_weights), vp, vp, vp, vp, sz, vp]
    L.k3moe_layer_noalloc.argtypes = [D, i32, vp, ctypes.POINTER(k3moe_weights), vp, vp, vp, vp]
    L.k3moe_shared_workspace_size.argtypes = [D, i32, i32, ctypes.POINTER(sz)]
    L.k3moe_shared_glu_bf16.argtypes = [D, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.k3moe_shared_profiled.argtypes = [D, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp,
                                        ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    L.k3moe_shared_profiled.restype = ctypes.c_int
    L.k3moe_status_str.argtypes = [ctypes.c_int]
    L.k3moe_status_str.restype = ctypes.c_char_p
    L.k3moe_layer_profiled.argtypes = [D, i32, vp, ctypes.POINTER(k3moe_weights), vp, vp, vp, vp, sz, vp,
                                       ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    L.k3moe_layer_profiled.restype = ctypes.c_int
    L.k3moe_prof_name.argtypes = [ctypes.c_int]
    L.k3moe_prof_name.restype = ctypes.c_char_p
    ip = ctypes.POINTER(ctypes.c_int)
    L.k3moe_prof_gemm_tiling.argtypes = [ip, ip, ip, ip]
    L.k3moe_prof_gemm_tiling.restype = ctypes.c_int
    L.k3moe_set_expert_path.argtypes = [ctypes.c_int]
    L.k3moe_set_expert_path.restype = ctypes.c_int
    for n in EXPORTS[:-1]:
        getattr(L, n).restype = ctypes.c_int
    if path is None:
        _lib = L
    return L


def status_str(status: int) -> str:
    return load().k3moe_status_str(status).decode()


def make_dims(d) -> k3moe_dims:
    return k3moe_dims(d.hidden, d.latent, d.inter, d.n_experts, d.topk, d.group, d.renorm,
                      d.routed_scale, d.eps, d.b1, d.b2, getattr(d, "topp", 0.0), getattr(d, "idot", 0))


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(s):
    if s is None:
        try:
            import torch
            if torch.cuda.is_available():
                return torch.cuda.current_stream().cuda_stream
        except ImportError:
            pass
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _dims(d):
    return d if isinstance(d, k3moe_dims) else make_dims(d)


def _check(rc: int, where: str):
    if rc != K3MOE_OK:
        raise K3MoeError(rc, where)


def _ws(ws):
    if ws is None:
        return None, 0
    if isinstance(ws, tuple):
        return ws
    return ws.data_ptr(), ws.numel() * ws.element_size()


def k3moe_workspace_size(dims, T: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().k3moe_workspace_size(ctypes.byref(_dims(dims)), T, ctypes.byref(n)), "k3moe_workspace_size")
    return n.value


def k3moe_gemm_scales_size(dims) -> int:
    n = ctypes.c_size_t(0)
    _check(load().k3moe_gemm_scales_size(ctypes.byref(_dims(dims)), ctypes.byref(n)), "k3moe_gemm_scales_size")
    return n.value


def k3moe_prepare_gemm_scales(dims, experts: k3moe_experts, dst, stream=None, check=True):
    """dst: a device buffer (tensor, or (pointer, bytes)) of k3moe_gemm_scales_size bytes."""
    p, n = _ws(dst)
    rc = load().k3moe_prepare_gemm_scales(ctypes.byref(_dims(dims)), ctypes.byref(experts), p, n, _stream(stream))
    if check:
        _check(rc, "k3moe_prepare_gemm_scales")
    return rc


def k3moe_router_planes_size(dims) -> int:
    n = ctypes.c_size_t(0)
    _check(load().k3moe_router_planes_size(ctypes.byref(_dims(dims)), ctypes.byref(n)), "k3moe_router_planes_size")
    return n.value


def k3moe_prepare_router_planes(dims, w_router, dst, stream=None, check=True):
    """w_router: device fp32 [E][H]; dst: a device buffer (tensor, or (pointer, bytes)) of
    k3moe_router_planes_size bytes."""
    p, n = _ws(dst)
    rc = load().k3moe_prepare_router_planes(ctypes.byref(_dims(dims)), _ptr(w_router), p, n, _stream(stream))
    if check:
        _check(rc, "k3moe_prepare_router_planes")
    return rc


def k3moe_route(dims, T, x, w_router, bias, topk_idx, topk_w, ws, stream=None, check=True):
    p, n = _ws(ws)
    rc = load().k3moe_route(ctypes.byref(_dims(dims)), T, _ptr(x), _ptr(w_router), _ptr(bias),
                            _ptr(topk_idx), _ptr(topk_w), p, n, _stream(stream))
    if check:
        _check(rc, "k3moe_route")
    return rc


def k3moe_latent_proj_bf16(dims, T, x, w_down, z, ws, stream=None, check=True):
    p, n = _ws(ws)
    rc = load().k3moe_latent_proj_bf16(ctypes.byref(_dims(dims)), T, _ptr(x), _ptr(w_down), _ptr(z), p, n,
                                       _stream(stream))
    if check:
        _check(rc, "k3moe_latent_proj_bf16")
    return rc


def k3moe_dispatch(dims, T, topk_idx, expert_off, sorted_pair, pair_slot, ws, stream=None, check=True):
    p, n = _ws(ws)
    rc = load().k3moe_dispatch(ctypes.byref(_dims(dims)), T, _ptr(topk_idx), _ptr(expert_off),
                               _ptr(sorted_pair), _ptr(pair_slot), p, n, _stream(stream))
    if check:
        _check(rc, "k3moe_dispatch")
    return rc


def k3moe_expert_glu_mxfp4(dims, T, z, experts: k3moe_experts, expert_off, sorted_pair, edn, ws,
                           stream=None, check=True):
    p, n = _ws(ws)
    rc = load().k3moe_expert_glu_mxfp4(ctypes.byref(_dims(dims)), T, _ptr(z),
                                       ctypes.byref(experts) if experts is not None else None,
                                       _ptr(expert_off), _ptr(sorted_pair), _ptr(edn), p, n, _stream(stream))
    if check:
        _check(rc, "k3moe_expert_glu_mxfp4")
    return rc


def k3moe_combine(dims, T, edn, pair_slot, topk_w, norm_w, w_up, y, ws, stream=None, check=True):
    p, n = _ws(ws)
    rc = load().k3moe_combine(ctypes.byref(_dims(dims)), T, _ptr(edn), _ptr(pair_slot), _ptr(topk_w),
                              _ptr(norm_w), _ptr(w_up), _ptr(y), p, n, _stream(stream))
    if check:
        _check(rc, "k3moe_combine")
    return rc


def k3moe_layer(dims, T, x, weights: k3moe_weights, y, topk_idx_out, topk_w_out, ws, stream=None, check=True):
    p, n = _ws(ws)
    rc = load().k3moe_layer(ctypes.byref(_dims(dims)), T, _ptr(x),
                            ctypes.byref(weights) if weights is not None else None, _ptr(y),
                            _ptr(topk_idx_out), _ptr(topk_w_out), p, n, _stream(stream))
    if check:
        _check(rc, "k3moe_layer")
    return rc


NOALLOC_SCRATCH_BYTES = 64 << 20  # K3MOE_NOALLOC_SCRATCH_BYTES


def k3moe_layer_noalloc(dims, T, x, weights: k3moe_weights, y, topk_idx_out, topk_w_out, stream=None, check=True):
    """k3moe_layer with the library's own fixed device array as workspace (allocates nothing)."""
    rc = load().k3moe_layer_noalloc(ctypes.byref(_dims(dims)), T, _ptr(x),
                                    ctypes.byref(weights) if weights is not None else None, _ptr(y),
                                    _ptr(topk_idx_out), _ptr(topk_w_out), _stream(stream))
    if check:
        _check(rc, "k3moe_layer_noalloc")
    return rc


def k3moe_layer_profiled(dims, T, x, weights: k3moe_weights, y, topk_idx_out, topk_w_out, ws, events,
                         stream=None):
    """As k3moe_layer, each kernel launch i bound to the event pair events[2i], events[2i+1]
    (its own start and end). Returns the step name of each timed launch, in launch order."""
    p, n = _ws(ws)
    arr = (ctypes.c_void_p * len(events))(*events)
    nk = ctypes.c_int(0)
    rc = load().k3moe_layer_profiled(ctypes.byref(_dims(dims)), T, _ptr(x), ctypes.byref(weights), _ptr(y),
                                     _ptr(topk_idx_out), _ptr(topk_w_out), p, n, _stream(stream), arr,
                                     len(events), ctypes.byref(nk))
    _check(rc, "k3moe_layer_profiled")
    return [load().k3moe_prof_name(i).decode() for i in range(nk.value)]


def k3moe_shared_workspace_size(dims, n_shared: int, T: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().k3moe_shared_workspace_size(ctypes.byref(_dims(dims)), n_shared, T, ctypes.byref(n)),
           "k3moe_shared_workspace_size")
    return n.value


def k3moe_shared_glu_bf16(dims, n_shared, T, x, sh1, sh3, sh2, y, ws, stream=None, check=True):
    """y += the fused shared experts on x (y is read and written)."""
    p, n = _ws(ws)
    rc = load().k3moe_shared_glu_bf16(ctypes.byref(_dims(dims)), n_shared, T, _ptr(x), _ptr(sh1), _ptr(sh3),
                                      _ptr(sh2), _ptr(y), p, n, _stream(stream))
    if check:
        _check(rc, "k3moe_shared_glu_bf16")
    return rc


def k3moe_shared_profiled(dims, n_shared, T, x, sh1, sh3, sh2, y, ws, events, stream=None):
    """As k3moe_shared_glu_bf16 with each launch timed (see k3moe_layer_profiled)."""
    p, n = _ws(ws)
    arr = (ctypes.c_void_p * len(events))(*events)
    nk = ctypes.c_int(0)
    rc = load().k3moe_shared_profiled(ctypes.byref(_dims(dims)), n_shared, T, _ptr(x), _ptr(sh1), _ptr(sh3),
                                      _ptr(sh2), _ptr(y), p, n, _stream(stream), arr, len(events),
                                      ctypes.byref(nk))
    _check(rc, "k3moe_shared_profiled")
    return [load().k3moe_prof_name(i).decode() for i in range(nk.value)]


EXPERT_PATH_AUTO, EXPERT_PATH_GEMV, EXPERT_PATH_GEMM = 0, 1, 2


def k3moe_set_expert_path(mode: int) -> int:
    """Select the expert-pass kernels (0 by batch size, 1 grouped GEMV, 2 grouped GEMM
    where its shape limits allow); returns the previous mode."""
    rc = load().k3moe_set_expert_path(int(mode))
    if rc < 0:
        raise K3MoeError(rc, "k3moe_set_expert_path")
    return rc


def gemm_tiling():
    """(tokens per column tile, gate/up rows per block, down rows per block, the most pairs
    of an expert that the batch-size GEMM form leaves to the decode kernel) of the grouped
    GEMM form (k3moe_prof_gemm_tiling)."""
    a, b, c, n = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(load().k3moe_prof_gemm_tiling(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c), ctypes.byref(n)),
           "k3moe_prof_gemm_tiling")
    return a.value, b.value, c.value, n.value
