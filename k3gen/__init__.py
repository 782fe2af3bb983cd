"""Seeded synthetic inputs for the Kimi K3 LatentMoE routed-expert layer.

This module only draws random numbers and lays them out in the layer's storage
formats; it holds none of the layer's arithmetic. Both the CPU oracle's tests and
the GPU path's tests and benchmark take their inputs from here.

Input recipe (shapes and distributions of the five workloads):
  * x ~ N(0, 1) per element, rounded to bf16.
  * router weight Wr [E, H] fp32 ~ N(0, 1/H); score-correction bias [E] ~ U(-0.1, 0.1).
  * W_down [L, H] bf16 ~ N(0, 1/H); W_up [H, L] bf16 ~ N(0, 1/L).
  * MXFP4 experts: packed bytes uniform (so each nibble is uniform over the 16 E2M1
    codes), ue8m0 scale bytes uniform in {118, ..., 124}.
  * RMSNorm weight gamma = 1.
  * Shared experts (n_shared fused GLU experts of width inter, SI = n_shared * inter):
    gate and up [SI, H] bf16 ~ N(0, 1/H); down [H, SI] bf16 ~ N(0, 1/SI).
Expert storage follows the pages' per-expert record: the six tensors of expert e
(w1 packed, w1 scales, w3 packed, w3 scales, w2 packed, w2 scales) lie back to back
in one blob of ``blob_bytes`` bytes, blob e at byte e * blob_bytes.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "k3gen.c")
# K3_HOST_SANITIZE=1 selects a build with AddressSanitizer and UndefinedBehaviorSanitizer
# (host code only; the process must preload the ASan runtime)
SANITIZE = os.environ.get("K3_HOST_SANITIZE") == "1"
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
_LIB_PATH = os.path.join(_HERE, "libk3gen_san.so" if SANITIZE else "libk3gen.so")
_lib = None

# tensor ids of the counter-based streams
T_X, T_WR, T_BIAS, T_WDOWN, T_WUP = 1, 2, 3, 4, 5
T_W1P, T_W1S, T_W3P, T_W3S, T_W2P, T_W2S = 6, 7, 8, 9, 10, 11
T_ZPROBE, T_GAMMA = 12, 13
T_SH1, T_SH3, T_SH2 = 14, 15, 16  # the shared experts (fused gate, up and down)
_ATTEMPT_SHIFT = 40  # x row counter: (attempt << 40) + t * H + i


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
        vp, sz, u64, u32, dbl = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double
        L.k3g_hash.restype = u64
        L.k3g_hash.argtypes = [u64, u32, u64]
        for name in ("k3g_normal_f32", "k3g_normal_bf16"):
            getattr(L, name).argtypes = [vp, sz, u64, u32, u64, dbl]
            getattr(L, name).restype = None
        L.k3g_uniform_f32.argtypes = [vp, sz, u64, u32, u64, dbl, dbl]
        L.k3g_uniform_f32.restype = None
        L.k3g_bytes.argtypes = [vp, sz, u64, u32, u64]
        L.k3g_bytes.restype = None
        L.k3g_int_range_u8.argtypes = [vp, sz, u64, u32, u64, ctypes.c_int, ctypes.c_int]
        L.k3g_int_range_u8.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal_f32(n, seed, tensor, idx0=0, std=1.0, out=None):
    out = np.empty(n, np.float32) if out is None else out
    lib().k3g_normal_f32(_ptr(out), n, seed, tensor, idx0, std)
    return out


def normal_bf16(n, seed, tensor, idx0=0, std=1.0, out=None):
    out = np.empty(n, np.uint16) if out is None else out
    lib().k3g_normal_bf16(_ptr(out), n, seed, tensor, idx0, std)
    return out


def uniform_f32(n, seed, tensor, lo, hi, idx0=0, out=None):
    out = np.empty(n, np.float32) if out is None else out
    lib().k3g_uniform_f32(_ptr(out), n, seed, tensor, idx0, lo, hi)
    return out


def random_bytes(n, seed, tensor, idx0=0, out=None):
    out = np.empty(n, np.uint8) if out is None else out
    lib().k3g_bytes(_ptr(out), n, seed, tensor, idx0)
    return out


def int_range_u8(n, seed, tensor, lo, hi, idx0=0, out=None):
    out = np.empty(n, np.uint8) if out is None else out
    lib().k3g_int_range_u8(_ptr(out), n, seed, tensor, idx0, lo, hi)
    return out


@dataclasses.dataclass(frozen=True)
class Dims:
    hidden: int
    latent: int
    inter: int
    n_experts: int
    topk: int
    eps: float
    group: int = 32
    renorm: int = 1
    routed_scale: float = 1.0
    b1: float = 4.0
    b2: float = 25.0
    topp: float = 0.0  # top-p tail drop of the chosen experts (0 = off)
    idot: int = 0      # 1: int8-per-32 activations in the expert products


# Kimi K3 MoE fields as the pages' config reader lists them (hidden 7168, 896
# experts, top 16, latent 3584, inter 3072, rms_eps 1e-5, SiTU caps 4 and 25).
K3 = Dims(hidden=7168, latent=3584, inter=3072, n_experts=896, topk=16, eps=1e-5)
TINY = Dims(hidden=256, latent=128, inter=96, n_experts=32, topk=4, eps=1e-6)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    T: int
    seed: int
    skewed: bool = False


WORKLOADS = [
    Workload("tiny T=4 H=256 L=128 I=96 E=32 K=4", TINY, 4, 0),
    Workload("K3 decode T=1", K3, 1, 1),
    Workload("K3 decode batch T=64", K3, 64, 2),
    Workload("K3 prefill T=4096", K3, 4096, 3),
    Workload("K3 skewed prefill T=8192", K3, 8192, 4, skewed=True),
]


@dataclasses.dataclass(frozen=True)
class ExpertLayout:
    """Byte offsets of the six tensors inside one expert blob."""
    dims: Dims

    @property
    def sizes(self):
        d = self.dims
        p13 = d.inter * (d.latent // 2)
        s13 = d.inter * (d.latent // d.group)
        p2 = d.latent * (d.inter // 2)
        s2 = d.latent * (d.inter // d.group)
        return [("w1p", p13), ("w1s", s13), ("w3p", p13), ("w3s", s13), ("w2p", p2), ("w2s", s2)]

    @property
    def offsets(self):
        off, o = {}, 0
        for name, n in self.sizes:
            off[name] = o
            o += n
        return off

    @property
    def blob_bytes(self) -> int:
        return sum(n for _, n in self.sizes)


_EXPERT_STREAMS = {"w1p": T_W1P, "w1s": T_W1S, "w3p": T_W3P, "w3s": T_W3S, "w2p": T_W2P, "w2s": T_W2S}


def gen_experts(dims: Dims, seed: int, e0: int, e1: int, out: np.ndarray | None = None) -> np.ndarray:
    """Blobs of experts e0..e1-1 as one uint8 array [(e1-e0) * blob_bytes]."""
    lay = ExpertLayout(dims)
    B = lay.blob_bytes
    out = np.empty((e1 - e0) * B, np.uint8) if out is None else out
    assert out.size == (e1 - e0) * B
    offs = lay.offsets
    for e in range(e0, e1):
        base = (e - e0) * B
        for name, n in lay.sizes:
            view = out[base + offs[name]: base + offs[name] + n]
            if name.endswith("p"):
                random_bytes(n, seed, _EXPERT_STREAMS[name], idx0=e * n, out=view)
            else:
                int_range_u8(n, seed, _EXPERT_STREAMS[name], 118, 124, idx0=e * n, out=view)
    return out


def gen_dense(dims: Dims, seed: int) -> dict:
    H, L, E = dims.hidden, dims.latent, dims.n_experts
    return {
        "w_router": normal_f32(E * H, seed, T_WR, std=1.0 / np.sqrt(H)).reshape(E, H),
        "bias": uniform_f32(E, seed, T_BIAS, -0.1, 0.1),
        "w_down": normal_bf16(L * H, seed, T_WDOWN, std=1.0 / np.sqrt(H)).reshape(L, H),
        "w_up": normal_bf16(H * L, seed, T_WUP, std=1.0 / np.sqrt(L)).reshape(H, L),
        "norm_w": np.ones(L, np.float32),
    }


def gen_shared(dims: Dims, seed: int, n_shared: int = 2) -> dict:
    """The fused shared experts: sh1 (gate) and sh3 (up) [SI][H], sh2 (down) [H][SI], bf16."""
    H, SI = dims.hidden, n_shared * dims.inter
    return {
        "sh1": normal_bf16(SI * H, seed, T_SH1, std=1.0 / np.sqrt(H)).reshape(SI, H),
        "sh3": normal_bf16(SI * H, seed, T_SH3, std=1.0 / np.sqrt(H)).reshape(SI, H),
        "sh2": normal_bf16(H * SI, seed, T_SH2, std=1.0 / np.sqrt(SI)).reshape(H, SI),
    }


def gen_x_rows(dims: Dims, seed: int, tokens, attempts=None) -> np.ndarray:
    """bf16 bits [len(tokens), H]; token t's row at attempt a (default 0)."""
    H = dims.hidden
    tokens = np.asarray(tokens, np.int64)
    attempts = np.zeros(len(tokens), np.int64) if attempts is None else np.asarray(attempts, np.int64)
    out = np.empty((len(tokens), H), np.uint16)
    for r, (t, a) in enumerate(zip(tokens.tolist(), attempts.tolist())):
        normal_bf16(H, seed, T_X, idx0=(a << _ATTEMPT_SHIFT) + t * H, std=1.0, out=out[r])
    return out


def gen_x(dims: Dims, seed: int, T: int, attempts=None) -> np.ndarray:
    if attempts is None:
        return normal_bf16(T * dims.hidden, seed, T_X, std=1.0).reshape(T, dims.hidden)
    return gen_x_rows(dims, seed, np.arange(T), attempts)


def skew_bias(base: np.ndarray, beta: float, tail_offset: float, hot_every: int = 10,
              tail_from: int = 4) -> np.ndarray:
    """Skewed score-correction bias. Hot experts (e % hot_every == 0: 90 of 896) keep
    their bias plus beta. The cold experts' own bias is replaced, so that the offset alone
    decides their rank: 0 for the warm ones (1 <= e % hot_every < tail_from) and
    -tail_offset for the tail (e % hot_every >= tail_from)."""
    E = base.size
    r = np.arange(E) % hot_every
    out = np.where(r == 0, base.astype(np.float64) + beta, np.where(r < tail_from, 0.0, -tail_offset))
    return out.astype(np.float32)

