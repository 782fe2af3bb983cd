"""CPU oracle for the Kimi K3 Stable LatentMoE routed-expert layer (ctypes wrapper).

TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import this module. The GPU library never
imports, links or calls it, and it never calls the GPU library.

The arithmetic is in ``k3o.c``: the plain definition of each step in fp64 with fp32
results where the pages store fp32. This wrapper only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "k3o.c")
# K3_HOST_SANITIZE=1 selects a build with AddressSanitizer and UndefinedBehaviorSanitizer
# (host code only; the process must preload the ASan runtime)
SANITIZE = os.environ.get("K3_HOST_SANITIZE") == "1"
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
_LIB_PATH = os.path.join(_HERE, "libk3o_san.so" if SANITIZE else "libk3o.so")
_lib = None


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int), ("latent", ctypes.c_int), ("inter", ctypes.c_int),
                ("n_experts", ctypes.c_int), ("topk", ctypes.c_int), ("group", ctypes.c_int),
                ("renorm", ctypes.c_int), ("routed_scale", ctypes.c_float), ("eps", ctypes.c_float),
                ("b1", ctypes.c_float), ("b2", ctypes.c_float), ("topp", ctypes.c_float),
                ("idot", ctypes.c_int)]


class Mx(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("packed_stride", ctypes.c_int64), ("scales_stride", ctypes.c_int64)]


class Experts(ctypes.Structure):
    _fields_ = [("w1", Mx), ("w3", Mx), ("w2", Mx)]


class Weights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("norm_w", ctypes.c_void_p), ("ex", Experts)]


def build() -> str:
    opt = SAN_FLAGS if SANITIZE else ["-O2"]
    subprocess.check_call(["gcc", *opt, "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                           "-std=c99", "-Wall", "-Wextra", _SRC, "-o", _LIB_PATH, "-lm"])
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.k3o_e2m1.restype = f
        L.k3o_e2m1.argtypes = [i]
        L.k3o_e8m0.restype = f
        L.k3o_e8m0.argtypes = [i]
        L.k3o_bf16_to_f32.restype = f
        L.k3o_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.k3o_mxfp4_decode_row.argtypes = [vp, vp, vp, i, i]
        L.k3o_mxfp4_decode_row.restype = None
        L.k3o_mxfp4_matvec.argtypes = [vp, vp, vp, vp, i, i, i]
        L.k3o_mxfp4_matvec.restype = None
        L.k3o_bf16_matvec.argtypes = [vp, vp, vp, i, i]
        L.k3o_bf16_matvec.restype = None
        L.k3o_router.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f]
        L.k3o_router.restype = ctypes.c_double
        L.k3o_router_topp.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, f, vp]
        L.k3o_router_topp.restype = ctypes.c_double
        L.k3o_situ.argtypes = [f, f, f, f]
        L.k3o_situ.restype = f
        L.k3o_rmsnorm.argtypes = [vp, vp, vp, i, f]
        L.k3o_rmsnorm.restype = None
        L.k3o_expert.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(Experts), i, ctypes.POINTER(Dims)]
        L.k3o_expert.restype = None
        L.k3o_dispatch.argtypes = [vp, i, i, i, vp, vp, vp]
        L.k3o_dispatch.restype = i
        L.k3o_layer.argtypes = [ctypes.POINTER(Dims), i, vp, ctypes.POINTER(Weights), vp, vp, vp, vp, vp, vp, i]
        L.k3o_layer.restype = i
        L.k3o_route_batch.argtypes = [ctypes.POINTER(Dims), i, vp, vp, vp, vp, vp, vp, vp, i]
        L.k3o_route_batch.restype = None
        L.k3o_scores_batch.argtypes = [ctypes.POINTER(Dims), i, vp, vp, vp, i]
        L.k3o_scores_batch.restype = None
        L.k3o_expert_pairs.argtypes = [ctypes.POINTER(Dims), i, vp, vp, vp, ctypes.POINTER(Experts), vp, vp, i]
        L.k3o_expert_pairs.restype = None
        L.k3o_shared.argtypes = [ctypes.POINTER(Dims), i, i, vp, vp, vp, vp, vp, i]
        L.k3o_shared.restype = None
        L.k3o_q8_round.argtypes = [vp, vp, i]
        L.k3o_q8_round.restype = f
        L.k3o_mxfp4_matvec_q8.argtypes = [vp, vp, vp, vp, vp, i, i, i]
        L.k3o_mxfp4_matvec_q8.restype = None
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous numpy"
    return a.ctypes.data


def make_dims(d) -> Dims:
    """From any object with the layer's dimension fields (e.g. k3gen.Dims)."""
    return Dims(d.hidden, d.latent, d.inter, d.n_experts, d.topk, d.group, d.renorm,
                d.routed_scale, d.eps, d.b1, d.b2, getattr(d, "topp", 0.0), getattr(d, "idot", 0))


class ExpertSet:
    """Expert weights as one blob array plus byte offsets of the six tensors in a blob.

    ``blobs`` holds experts first..first+n-1; expert ids given to the oracle are global,
    so pointers are rebased by ``first``."""

    def __init__(self, blobs: np.ndarray, blob_bytes: int, offsets: dict, first: int = 0):
        self.blobs = blobs
        self.blob_bytes = blob_bytes
        self.offsets = offsets
        self.first = first
        base = blobs.ctypes.data - first * blob_bytes

        def mx(p, s):
            return Mx(base + offsets[p], base + offsets[s], blob_bytes, blob_bytes)
        self.c = Experts(mx("w1p", "w1s"), mx("w3p", "w3s"), mx("w2p", "w2s"))


def e2m1(code: int) -> float:
    return lib().k3o_e2m1(code)


def e8m0(byte: int) -> float:
    return lib().k3o_e8m0(byte)


def mxfp4_decode(packed: np.ndarray, scales: np.ndarray, cols: int, group: int = 32) -> np.ndarray:
    rows = packed.shape[0]
    out = np.empty((rows, cols), np.float32)
    packed = np.ascontiguousarray(packed)
    scales = np.ascontiguousarray(scales)
    for r in range(rows):
        lib().k3o_mxfp4_decode_row(_p(out[r]), _p(packed[r]), _p(scales[r]), cols, group)
    return out


def mxfp4_matvec(x: np.ndarray, packed: np.ndarray, scales: np.ndarray, cols: int, rows: int,
                 group: int = 32) -> np.ndarray:
    y = np.empty(rows, np.float32)
    x = np.ascontiguousarray(x, np.float32)
    lib().k3o_mxfp4_matvec(_p(y), _p(x), _p(np.ascontiguousarray(packed)),
                           _p(np.ascontiguousarray(scales)), cols, rows, group)
    return y


def bf16_matvec(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    out, inn = W.shape
    y = np.empty(out, np.float32)
    lib().k3o_bf16_matvec(_p(y), _p(np.ascontiguousarray(x, np.float32)), _p(np.ascontiguousarray(W)), inn, out)
    return y


def router(x: np.ndarray, Wr: np.ndarray, bias, topk: int, renorm: int = 1, routed_scale: float = 1.0):
    """One token. Returns (idx ascending, weights, selection order, gap)."""
    E, H = Wr.shape
    idx = np.empty(topk, np.int32)
    w = np.empty(topk, np.float32)
    sel = np.empty(topk, np.int32)
    gap = lib().k3o_router(_p(idx), _p(w), _p(sel), _p(np.ascontiguousarray(x, np.float32)),
                           _p(np.ascontiguousarray(Wr, np.float32)),
                           None if bias is None else _p(np.ascontiguousarray(bias, np.float32)),
                           H, E, topk, renorm, routed_scale)
    return idx, w, sel, gap


def router_topp(x: np.ndarray, Wr: np.ndarray, bias, topk: int, topp: float, renorm: int = 1,
                routed_scale: float = 1.0):
    """One token with the top-p tail drop (k3o_router_topp). Returns (idx, weights, gap,
    margin); dropped slots hold id -1 and weight 0."""
    E, H = Wr.shape
    idx = np.empty(topk, np.int32)
    w = np.empty(topk, np.float32)
    margin = np.empty(1, np.float64)
    gap = lib().k3o_router_topp(_p(idx), _p(w), None, _p(np.ascontiguousarray(x, np.float32)),
                                _p(np.ascontiguousarray(Wr, np.float32)),
                                None if bias is None else _p(np.ascontiguousarray(bias, np.float32)),
                                H, E, topk, renorm, routed_scale, topp, _p(margin))
    return idx, w, gap, float(margin[0])


def situ(g: float, u: float, b1: float = 4.0, b2: float = 25.0) -> float:
    return lib().k3o_situ(g, u, b1, b2)


def rmsnorm(x: np.ndarray, w=None, eps: float = 1e-5) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty_like(x)
    lib().k3o_rmsnorm(_p(out), _p(x), None if w is None else _p(np.ascontiguousarray(w, np.float32)),
                      x.size, eps)
    return out


def expert(dims, ex: ExpertSet, e: int, z: np.ndarray):
    """One expert on one latent vector. Returns (edn, g, u, act)."""
    L, I = dims.latent, dims.inter
    edn = np.empty(L, np.float32)
    g, u, act = (np.empty(I, np.float32) for _ in range(3))
    d = make_dims(dims)
    lib().k3o_expert(_p(edn), _p(g), _p(u), _p(act), _p(np.ascontiguousarray(z, np.float32)),
                     ctypes.byref(ex.c), e, ctypes.byref(d))
    return edn, g, u, act


def dispatch(topk_idx: np.ndarray, E: int):
    T, K = topk_idx.shape
    ti = np.ascontiguousarray(topk_idx, np.int32)
    off = np.empty(E + 1, np.int32)
    sp = np.empty(T * K, np.int32)
    ps = np.empty(T * K, np.int32)
    rc = lib().k3o_dispatch(_p(ti), T, K, E, _p(off), _p(sp), _p(ps))
    if rc != 0:
        raise ValueError("expert index out of range")
    return off, sp, ps


def _weights_struct(dense: dict, ex: ExpertSet) -> Weights:
    return Weights(_p(dense["w_router"]), _p(dense["bias"]), _p(dense["w_down"]), _p(dense["w_up"]),
                   _p(dense["norm_w"]) if dense.get("norm_w") is not None else None, ex.c)


def layer(dims, x: np.ndarray, dense: dict, ex: ExpertSet, nthreads: int = 0, want_inner: bool = False):
    """The whole layer on the rows of x (bf16 bits [T, H]). Returns a dict with y, idx, w
    (and z, acc, nrm when want_inner)."""
    T = x.shape[0]
    H, L, K = dims.hidden, dims.latent, dims.topk
    x = np.ascontiguousarray(x, np.uint16)
    out = {"y": np.empty((T, H), np.float32), "idx": np.empty((T, K), np.int32),
           "w": np.empty((T, K), np.float32)}
    if want_inner:
        for k in ("z", "acc", "nrm"):
            out[k] = np.empty((T, L), np.float32)
    d = make_dims(dims)
    ws = _weights_struct(dense, ex)
    lib().k3o_layer(ctypes.byref(d), T, _p(x), ctypes.byref(ws), _p(out["y"]), _p(out["idx"]), _p(out["w"]),
                    _p(out.get("z")), _p(out.get("acc")), _p(out.get("nrm")), nthreads)
    return out


def route_batch(dims, x: np.ndarray, Wr: np.ndarray, bias: np.ndarray, nthreads: int = 0,
                want_margins: bool = False):
    """Router only for rows of x (with dims.topp's tail drop). Returns (idx [T,K], w [T,K],
    gaps [T]), plus the top-p decision margins [T] when want_margins."""
    T = x.shape[0]
    K = dims.topk
    idx = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    gaps = np.empty(T, np.float64)
    margins = np.empty(T, np.float64) if want_margins else None
    d = make_dims(dims)
    lib().k3o_route_batch(ctypes.byref(d), T, _p(np.ascontiguousarray(x, np.uint16)),
                          _p(np.ascontiguousarray(Wr, np.float32)), _p(np.ascontiguousarray(bias, np.float32)),
                          _p(idx), _p(w), _p(gaps), _p(margins), nthreads)
    return (idx, w, gaps, margins) if want_margins else (idx, w, gaps)


def scores_batch(dims, x: np.ndarray, Wr: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """Unbiased router scores sigmoid(Wr x_t) [T, E] (fp32), as the router computes them."""
    T = x.shape[0]
    sc = np.empty((T, dims.n_experts), np.float32)
    d = make_dims(dims)
    lib().k3o_scores_batch(ctypes.byref(d), T, _p(np.ascontiguousarray(x, np.uint16)),
                           _p(np.ascontiguousarray(Wr, np.float32)), _p(sc), nthreads)
    return sc


def expert_pairs(dims, tok: np.ndarray, ex_id: np.ndarray, z: np.ndarray, ex: ExpertSet,
                 nthreads: int = 0, want_act: bool = False):
    n = len(tok)
    edn = np.empty((n, dims.latent), np.float32)
    act = np.empty((n, dims.inter), np.float32) if want_act else None
    d = make_dims(dims)
    lib().k3o_expert_pairs(ctypes.byref(d), n, _p(np.ascontiguousarray(tok, np.int32)),
                           _p(np.ascontiguousarray(ex_id, np.int32)), _p(np.ascontiguousarray(z, np.float32)),
                           ctypes.byref(ex.c), _p(edn), _p(act), nthreads)
    return (edn, act) if want_act else edn


def shared(dims, x: np.ndarray, sh: dict, y: np.ndarray, n_shared: int = 2, nthreads: int = 0) -> np.ndarray:
    """y [T][H] plus the shared experts' output (k3o_shared); x [T][H] bf16 bits; sh as
    k3gen.gen_shared. Returns a new array."""
    x = np.ascontiguousarray(x, np.uint16)
    T = x.shape[0]
    out = np.ascontiguousarray(y, np.float32).copy()
    sh1, sh3, sh2 = (np.ascontiguousarray(sh[k], np.uint16) for k in ("sh1", "sh3", "sh2"))
    SI = n_shared * dims.inter
    assert sh1.shape == (SI, dims.hidden) and sh3.shape == (SI, dims.hidden) and sh2.shape == (dims.hidden, SI)
    lib().k3o_shared(ctypes.byref(make_dims(dims)), n_shared, T, _p(x), _p(sh1), _p(sh3), _p(sh2), _p(out),
                     nthreads)
    return out


def q8_round(v: np.ndarray):
    """One group (n <= 32) of activations to int8 (k3o_q8_round). Returns (q, d)."""
    v = np.ascontiguousarray(v, np.float32)
    q = np.empty(v.size, np.int8)
    d = lib().k3o_q8_round(_p(q), _p(v), v.size)
    return q, float(d)


def mxfp4_matvec_q8(q: np.ndarray, d: np.ndarray, packed: np.ndarray, scales: np.ndarray, cols: int, rows: int,
                    group: int = 32) -> np.ndarray:
    """k3o_mxfp4_matvec_q8: int8 activations q [cols] with group scales d."""
    y = np.empty(rows, np.float32)
    lib().k3o_mxfp4_matvec_q8(_p(y), _p(np.ascontiguousarray(q, np.int8)), _p(np.ascontiguousarray(d, np.float32)),
                              _p(np.ascontiguousarray(packed, np.uint8)), _p(np.ascontiguousarray(scales, np.uint8)),
                              cols, rows, group)
    return y
