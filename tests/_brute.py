"""An independent, brute-force statement of the layer, used to pin the oracle.

It shares nothing with oracle/k3o.c: the E2M1 values are derived from the element
format's bit fields (OCP Microscaling Formats v1.0, E2M1: 1 sign bit, 2 exponent
bits with bias 1, 1 mantissa bit; exponent field 0 is subnormal), not read from a
table; MXFP4 matrices are decoded whole with numpy; the logistic is taken through tanh;
routing ranks with numpy's lexsort; products are numpy fp64 matmuls.
"""
from __future__ import annotations

import numpy as np


def e2m1_from_bits(code: int) -> float:
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:
        mag = man * 0.5                      # subnormal: 2^(1-bias) * (m / 2)
    else:
        mag = 2.0 ** (exp - 1) * (1.0 + man / 2.0)
    return sign * mag


E2M1_BITS = np.array([e2m1_from_bits(c) for c in range(16)], np.float64)


def e8m0_bits(s: np.ndarray) -> np.ndarray:
    s = np.asarray(s, np.int64)
    v = np.ldexp(1.0, (s - 127).astype(np.int64))
    return np.where(s == 255, 0.0, v)


def decode_mxfp4(packed: np.ndarray, scales: np.ndarray, group: int = 32) -> np.ndarray:
    """[rows, cols/2] bytes + [rows, cols/group] scales -> fp64 [rows, cols]."""
    rows, half = packed.shape
    codes = np.empty((rows, half * 2), np.int64)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    vals = E2M1_BITS[codes]
    sc = np.repeat(e8m0_bits(scales), group, axis=1)[:, : half * 2]
    return vals * sc


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)


def expert_views(blob: np.ndarray, dims, offsets: dict):
    L, I, G = dims.latent, dims.inter, dims.group

    def mat(p, s, rows, cols):
        pk = blob[offsets[p]: offsets[p] + rows * cols // 2].reshape(rows, cols // 2)
        sc = blob[offsets[s]: offsets[s] + rows * cols // G].reshape(rows, cols // G)
        return pk, sc
    return mat("w1p", "w1s", I, L), mat("w3p", "w3s", I, L), mat("w2p", "w2s", L, I)


def route(xf: np.ndarray, Wr: np.ndarray, bias: np.ndarray, K: int, renorm=1, routed_scale=1.0):
    logit = Wr.astype(np.float64) @ xf
    sc = (0.5 * (1.0 + np.tanh(0.5 * logit))).astype(np.float32)   # logistic via tanh
    ch = sc.astype(np.float64) + bias.astype(np.float64)
    order = np.lexsort((np.arange(ch.size), -ch))   # by ch descending, then id ascending
    chosen = np.sort(order[:K])
    s = sc[chosen].astype(np.float64)
    w = s / s.sum() if renorm else s
    return chosen, (w * routed_scale).astype(np.float32)


def topp_drop(chosen: np.ndarray, sc_chosen: np.ndarray, p: float, renorm=1, routed_scale=1.0):
    """The top-p tail drop on a routed token: fractions of the chosen total (fp32), walked
    by (fraction descending, id ascending) with an fp32 running sum; kept while the sum
    before is below p. Returns (ids with -1 for dropped, weights with 0 for dropped)."""
    s = sc_chosen.astype(np.float64)
    f = (s / s.sum()).astype(np.float32)
    order = np.lexsort((chosen, -f))
    before = np.zeros(len(f), np.float32)
    run = np.float32(0.0)
    for r, j in enumerate(order):
        before[r] = run
        run = np.float32(run + f[j])
    keep = np.zeros(len(f), bool)
    keep[order[before < np.float32(p)]] = True
    sk = s[keep].sum()
    w = np.where(keep, (s / sk if renorm else s) * routed_scale, 0.0).astype(np.float32)
    return np.where(keep, chosen, -1).astype(np.int32), w


def q8_dequant(v: np.ndarray, group: int = 32) -> np.ndarray:
    """Activations rounded to int8 per group (symmetric absmax scale, nearest with ties away
    from zero), returned as the values the integer dot stands for: q * d in fp64."""
    v = np.asarray(v, np.float32)
    out = np.empty(v.size, np.float64)
    for g0 in range(0, v.size, group):
        x = v[g0:g0 + group]
        d = np.float32(np.max(np.abs(x))) / np.float32(127.0)
        if d == 0:
            out[g0:g0 + group] = 0.0
            continue
        r = (x / d).astype(np.float32)
        q = np.clip(np.sign(r) * np.floor(np.abs(r) + np.float32(0.5)), -127, 127)
        out[g0:g0 + group] = q.astype(np.float64) * np.float64(d)
    return out


def situ(g: np.ndarray, u: np.ndarray, b1=4.0, b2=25.0) -> np.ndarray:
    g = g.astype(np.float64)
    u = u.astype(np.float64)
    return (b1 * np.tanh(g / b1) * (0.5 * (1.0 + np.tanh(0.5 * g))) * b2 * np.tanh(u / b2)).astype(np.float32)


def layer_token(dims, x_bf16: np.ndarray, dense: dict, expert_blob_fn, offsets: dict):
    """One token through the layer; expert_blob_fn(e) returns expert e's blob bytes."""
    xf = bf16_bits_to_f64(x_bf16)
    idx, w = route(xf, dense["w_router"], dense["bias"], dims.topk, dims.renorm, dims.routed_scale)
    if getattr(dims, "topp", 0.0) > 0.0:
        logit = dense["w_router"].astype(np.float64) @ xf
        sc = (0.5 * (1.0 + np.tanh(0.5 * logit))).astype(np.float32)
        idx, w = topp_drop(idx, sc[idx], dims.topp, dims.renorm, dims.routed_scale)
    z = (bf16_bits_to_f64(dense["w_down"]) @ xf).astype(np.float32)
    acc = np.zeros(dims.latent, np.float64)
    for e, wj in zip(idx, w):
        if e < 0:
            continue
        (p1, s1), (p3, s3), (p2, s2) = expert_views(expert_blob_fn(int(e)), dims, offsets)
        idot = getattr(dims, "idot", 0)
        zin = q8_dequant(z, dims.group) if idot else z.astype(np.float64)
        g = (decode_mxfp4(p1, s1, dims.group) @ zin).astype(np.float32)
        u = (decode_mxfp4(p3, s3, dims.group) @ zin).astype(np.float32)
        a = situ(g, u, dims.b1, dims.b2)
        ain = q8_dequant(a, dims.group) if idot else a.astype(np.float64)
        edn = (decode_mxfp4(p2, s2, dims.group) @ ain).astype(np.float32)
        acc += np.float64(wj) * edn.astype(np.float64)
    accf = acc.astype(np.float32).astype(np.float64)
    gam = dense["norm_w"].astype(np.float64)
    nrm = (accf / np.sqrt(np.mean(accf * accf) + dims.eps) * gam).astype(np.float32)
    y = (bf16_bits_to_f64(dense["w_up"]) @ nrm.astype(np.float64)).astype(np.float32)
    return {"y": y, "idx": idx.astype(np.int32), "w": w, "z": z, "acc": accf.astype(np.float32), "nrm": nrm}


def shared_token(dims, x_bf16: np.ndarray, sh: dict, n_shared: int = 2) -> np.ndarray:
    """The fused shared experts on one token's original input: numpy fp64 products
    rounded to fp32 at the same points as the routed experts."""
    xf = bf16_bits_to_f64(x_bf16)
    g = (bf16_bits_to_f64(sh["sh1"]) @ xf).astype(np.float32)
    u = (bf16_bits_to_f64(sh["sh3"]) @ xf).astype(np.float32)
    a = situ(g, u, dims.b1, dims.b2)
    return (bf16_bits_to_f64(sh["sh2"]) @ a.astype(np.float64)).astype(np.float32)
