"""GPU parity on seeded random shapes inside the supported set (include/k3moe.h): widths
that are multiples of 32 but not of 64 or 128, expert counts that are not multiples of
64, every top-k from 1 up, batches across the GEMV/GEMM thresholds (so some layers mix a
GEMV gate/up pass with a GEMM down pass), with and without renormalisation and the top-p
tail drop. Same bar as the other parity tests."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import k3gen
from tests import _inputs
from tests.test_gpu_parity import Host, compare_idot, compare_layer, say

pytestmark = pytest.mark.gpu


def random_case(seed: int):
    r = np.random.default_rng(1000 + seed)
    H = 32 * int(r.integers(2, 33))
    L = 32 * int(r.integers(1, 33))
    I = 32 * int(r.integers(1, 17))
    E = int(r.integers(2, 257))
    K = int(r.integers(1, min(16, E) + 1))
    T = int(r.integers(1, 160))
    topp = float(r.choice([0.0, 0.0, r.uniform(0.3, 0.95)]))
    renorm = int(r.integers(0, 2))
    d = dataclasses.replace(k3gen.TINY, hidden=H, latent=L, inter=I, n_experts=E, topk=K, topp=topp,
                            renorm=renorm)
    return d, T


@pytest.mark.parametrize("one", [False, True], ids=["T", "T1"])
@pytest.mark.parametrize("seed", range(16))
def test_random_shape_layer(seed, one):
    # T1: the same shape at one token (the selection inside the gate/up pass)
    d, T = random_case(seed)
    T = 1 if one else T
    say(f"random shape {seed}: {d}, T={T}")
    h = Host(d, 70 + seed)
    x, _ = _inputs.gap_fixed_x(d, 80 + seed, T, h.dense["w_router"], h.dense["bias"])
    compare_layer(h, x, what=f"random shape {seed} T={T}")


@pytest.mark.parametrize("seed", range(6))
def test_random_shape_shared_experts(seed):
    import oracle
    from mxfp4_routed_expert_amd import device
    from tests.test_gpu_parity import check_rows, run_shared
    r = np.random.default_rng(2000 + seed)
    n_shared = int(r.integers(1, 4))
    inter = 64 * int(r.integers(1, 9))  # a multiple of 64, so n_shared * inter is too
    H = 32 * int(r.integers(2, 49))
    T = int(r.choice([1, int(r.integers(2, 40)), int(r.integers(40, 300))]))
    d = dataclasses.replace(k3gen.TINY, hidden=H, inter=inter)
    say(f"random shared experts {seed}: H={H} inter={inter} n_shared={n_shared} T={T}")
    sh = k3gen.gen_shared(d, 90 + seed, n_shared)
    x = k3gen.gen_x(d, 95 + seed, T)
    y0 = np.random.default_rng(seed).standard_normal((T, H)).astype(np.float32)
    got = run_shared(d, n_shared, x, device.upload_shared(sh), y0)
    check_rows(got, oracle.shared(d, x, sh, y0, n_shared), f"random shared {seed}")


@pytest.mark.parametrize("seed", range(6))
def test_random_shape_int8_activations(seed):
    # the int8-activation variant on the random shapes (its own bar: compare_idot)
    d, T = random_case(100 + seed)
    say(f"random shape {100 + seed} with int8 activations: {d}, T={T}")
    h = Host(d, 170 + seed)
    compare_idot(h, T, 180 + seed, f"random shape {100 + seed} int8 T={T}")


@pytest.mark.parametrize("E,K,p", [(32, 1, 0.5), (8, 8, 0.6), (8, 8, 0.0)])
@pytest.mark.parametrize("T", [1, 40])
def test_degenerate_routing(E, K, p, T):
    # one expert per token (top-p keeps it, weight 1); every expert chosen (the top-k is
    # the whole set; top-p drops its tail)
    d = dataclasses.replace(k3gen.TINY, n_experts=E, topk=K, topp=p)
    h = Host(d, 60 + E + K)
    x, _ = _inputs.gap_fixed_x(d, 61 + T, T, h.dense["w_router"], h.dense["bias"])
    compare_layer(h, x, what=f"E={E} K={K} top-p {p} T={T}")
