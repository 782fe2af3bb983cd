"""Test inputs: the generator's seeded tensors plus the 1e-3 selection-gap rule.

A token whose 16th and 17th selection scores (as the oracle computes them) lie closer
than MIN_GAP is redrawn from its next sub-stream (attempt + 1), so that the expert set
is unique under any fp32 evaluation order. This needs the oracle's router, so it lives
with the tests, not in the generator.
"""
from __future__ import annotations

import functools
import json
import os

import numpy as np

import k3gen
import oracle

MIN_GAP = 1e-3
# with the top-p tail drop on, a token whose walk passes within this of p is redrawn too
# (the GPU's fractions and running sum agree with the oracle's to about 1e-6)
MIN_TOPP_MARGIN = 1e-4
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _gaps(dims, x, w_router, bias, nthreads):
    if getattr(dims, "topp", 0.0) > 0.0:
        _, _, g, m = oracle.route_batch(dims, x, w_router, bias, nthreads, want_margins=True)
        return np.where(m < MIN_TOPP_MARGIN, 0.0, g)
    return oracle.route_batch(dims, x, w_router, bias, nthreads)[2]


def gap_fixed_x(dims, seed, T, w_router, bias, nthreads=0, max_rounds=200):
    attempts = np.zeros(T, np.int64)
    x = k3gen.gen_x(dims, seed, T)
    gaps = _gaps(dims, x, w_router, bias, nthreads)
    for _ in range(max_rounds):
        bad = np.flatnonzero(gaps < MIN_GAP)
        if bad.size == 0:
            return x, attempts
        attempts[bad] += 1
        x[bad] = k3gen.gen_x_rows(dims, seed, bad, attempts[bad])
        gaps[bad] = _gaps(dims, x[bad], w_router, bias, nthreads)
    raise RuntimeError("gap rule not met")


def skew_params():
    with open(os.path.join(GOLDEN, "skew_bias.json")) as f:
        return json.load(f)


def skewed_bias(base: np.ndarray) -> np.ndarray:
    """The skewed workload's bias on a layer's own bias (parameters in skew_bias.json)."""
    p = skew_params()
    return k3gen.skew_bias(base, p["beta"], p["tail_offset"], p["hot_every"], p["tail_from"])


def layer_seed(wl: k3gen.Workload) -> int:
    """All K3-shape workloads share one layer (the decode layer's seed); tiny has its own."""
    return wl.seed if wl.dims is k3gen.TINY else 1


@functools.lru_cache(maxsize=4)
def dense_for(wl_index: int):
    wl = k3gen.WORKLOADS[wl_index]
    dense = k3gen.gen_dense(wl.dims, layer_seed(wl))
    if wl.skewed:
        p = skew_params()
        dense["bias"] = skewed_bias(dense["bias"])
    return dense


def expert_chunks(dims, seed, chunk=64):
    lay = k3gen.ExpertLayout(dims)
    for e0 in range(0, dims.n_experts, chunk):
        e1 = min(dims.n_experts, e0 + chunk)
        yield e0, k3gen.gen_experts(dims, seed, e0, e1)
