"""Host-side checks of the C-ABI: the library loads, exports every entry point the
header declares, and refuses bad arguments before launching anything (so these run
without a GPU)."""
import ctypes
import os
import re

import pytest

import k3gen
from mxfp4_routed_expert_amd import k3moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def header_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = open(os.path.join(INCLUDE, h)).read()
            names |= set(re.findall(r"^\s*(?:int|const char \*)\s*(k3moe_\w+)\s*\(", text, re.M))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = header_functions()
    assert set(names) >= set(k3moe.EXPORTS[:-1])
    lib = ctypes.CDLL(k3moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert k3moe.status_str(0) == "ok"
    for c in (-1, -2, -3, -4):
        assert k3moe.status_str(c) != "unknown status"


def _d(**kw):
    base = dict(hidden=256, latent=128, inter=96, n_experts=32, topk=4, group=32, renorm=1,
                routed_scale=1.0, eps=1e-6, b1=4.0, b2=25.0)
    base.update(kw)
    return k3moe.k3moe_dims(**base)


def test_workspace_size_grows_with_T_and_refuses_bad_dims():
    a = k3moe.k3moe_workspace_size(k3gen.TINY, 4)
    b = k3moe.k3moe_workspace_size(k3gen.TINY, 400)
    assert 0 < a < b
    assert k3moe.k3moe_workspace_size(k3gen.TINY, 0) >= 0
    n = ctypes.c_size_t()
    L = k3moe.load()
    bad = {
        k3moe.K3MOE_EINVAL: [dict(hidden=0), dict(topk=0), dict(renorm=2), dict(eps=-1.0), dict(b1=0.0)],
        k3moe.K3MOE_EUNSUPPORTED: [dict(group=16), dict(latent=100), dict(inter=40), dict(hidden=250),
                                   dict(topk=33, n_experts=64), dict(topk=8, n_experts=4),
                                   dict(n_experts=1025)],
    }
    for code, cases in bad.items():
        for kw in cases:
            assert L.k3moe_workspace_size(ctypes.byref(_d(**kw)), 4, ctypes.byref(n)) == code, kw
    assert L.k3moe_workspace_size(ctypes.byref(_d()), -1, ctypes.byref(n)) == k3moe.K3MOE_EINVAL
    assert L.k3moe_workspace_size(None, 4, ctypes.byref(n)) == k3moe.K3MOE_EINVAL
    assert L.k3moe_workspace_size(ctypes.byref(_d()), 4, None) == k3moe.K3MOE_EINVAL
    # T * topk must fit in int32
    assert L.k3moe_workspace_size(ctypes.byref(_d(topk=4)), 2 ** 29, ctypes.byref(n)) == k3moe.K3MOE_EUNSUPPORTED


FAKE = 1 << 20          # an aligned, never dereferenced address
WS = (1 << 24, 1 << 40)  # aligned fake workspace, large


def test_route_refuses_before_launch():
    d = _d()
    f = k3moe.k3moe_route
    assert f(d, 4, None, FAKE, FAKE, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_EINVAL
    assert f(d, 4, FAKE, FAKE, None, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_EINVAL
    assert f(d, 4, FAKE + 2, FAKE, FAKE, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_EUNSUPPORTED
    assert f(d, 4, FAKE, FAKE, FAKE, FAKE, FAKE, (1 << 24, 100), check=False) == k3moe.K3MOE_EWORKSPACE
    assert f(d, 4, FAKE, FAKE, FAKE, FAKE, FAKE, (None, 0), check=False) == k3moe.K3MOE_EWORKSPACE
    assert f(d, 4, FAKE, FAKE, FAKE, FAKE, FAKE, ((1 << 24) + 64, 1 << 40), check=False) == k3moe.K3MOE_EUNSUPPORTED
    assert f(_d(topk=40), 4, FAKE, FAKE, FAKE, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_EUNSUPPORTED
    assert f(d, -3, FAKE, FAKE, FAKE, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_EINVAL
    # T == 0 is a no-op that launches nothing
    assert f(d, 0, FAKE, FAKE, FAKE, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_OK


def _experts(packed=FAKE, stride=1 << 16):
    m = k3moe.k3moe_mxfp4(packed, FAKE, stride, 4096)
    return k3moe.k3moe_experts(m, m, m)


def test_expert_stage_refuses_before_launch():
    d = _d()
    f = k3moe.k3moe_expert_glu_mxfp4
    assert f(d, 4, FAKE, None, FAKE, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_EINVAL
    assert f(d, 4, FAKE, _experts(packed=FAKE + 8), FAKE, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_EUNSUPPORTED
    assert f(d, 4, FAKE, _experts(stride=(1 << 16) + 4), FAKE, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_EUNSUPPORTED
    assert f(d, 4, FAKE, _experts(stride=-16), FAKE, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_EINVAL
    assert f(d, 4, FAKE + 4, _experts(), FAKE, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_EUNSUPPORTED
    assert f(d, 4, FAKE, _experts(), None, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_EINVAL
    assert f(d, 0, FAKE, _experts(), FAKE, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_OK


def test_gemm_scales_size_and_refusals():
    d = _d()
    n = k3moe.k3moe_gemm_scales_size(d)
    # three 256-byte aligned regions of E experts x ceil(ng / 12) turns x rows x 12 bytes
    up = lambda v: (v + 255) // 256 * 256
    gu = -(-(d.latent // 32) // 12) * d.inter * 12
    dn = -(-(d.inter // 32) // 12) * d.latent * 12
    assert n == 2 * up(d.n_experts * gu) + up(d.n_experts * dn)
    f = k3moe.k3moe_prepare_gemm_scales
    assert f(d, _experts(), None, check=False) == k3moe.K3MOE_EINVAL
    assert f(d, _experts(), (FAKE, n - 1), check=False) == k3moe.K3MOE_EWORKSPACE
    assert f(d, _experts(), (FAKE + 16, n), check=False) == k3moe.K3MOE_EUNSUPPORTED
    assert f(d, _experts(stride=-16), (FAKE, n), check=False) == k3moe.K3MOE_EINVAL
    # the layer refuses a copy that is not 256-byte aligned
    w = k3moe.k3moe_weights(FAKE, FAKE, FAKE, FAKE, FAKE, _experts(), FAKE + 16)
    assert k3moe.k3moe_layer(d, 4, FAKE, w, FAKE, None, None, WS, check=False) == k3moe.K3MOE_EUNSUPPORTED


def test_router_planes_size_and_refusals():
    d = _d()
    n = k3moe.k3moe_router_planes_size(d)
    assert n == 3 * d.n_experts * d.hidden * 2  # three bf16 planes of [E][H]
    f = k3moe.k3moe_prepare_router_planes
    assert f(d, FAKE, None, check=False) == k3moe.K3MOE_EINVAL
    assert f(d, None, (FAKE, n), check=False) == k3moe.K3MOE_EINVAL
    assert f(d, FAKE, (FAKE, n - 1), check=False) == k3moe.K3MOE_EWORKSPACE
    assert f(d, FAKE, (FAKE + 8, n), check=False) == k3moe.K3MOE_EUNSUPPORTED
    assert f(d, FAKE + 4, (FAKE, n), check=False) == k3moe.K3MOE_EUNSUPPORTED
    # the layer refuses a plane copy that is not 16-byte aligned
    w = k3moe.k3moe_weights(FAKE, FAKE, FAKE, FAKE, FAKE, _experts(), None, FAKE + 8)
    assert k3moe.k3moe_layer(d, 4, FAKE, w, FAKE, None, None, WS, check=False) == k3moe.K3MOE_EUNSUPPORTED


def test_other_entry_points_refuse_before_launch():
    d = _d()
    assert k3moe.k3moe_latent_proj_bf16(d, 4, FAKE, None, FAKE, WS, check=False) == k3moe.K3MOE_EINVAL
    assert k3moe.k3moe_latent_proj_bf16(d, 4, FAKE, FAKE + 2, FAKE, WS, check=False) == k3moe.K3MOE_EUNSUPPORTED
    assert k3moe.k3moe_dispatch(d, 4, None, FAKE, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_EINVAL
    assert k3moe.k3moe_dispatch(d, 4, FAKE, FAKE, FAKE, FAKE, (FAKE, 8), check=False) == k3moe.K3MOE_EWORKSPACE
    assert k3moe.k3moe_combine(d, 4, FAKE, FAKE, FAKE, None, FAKE, FAKE, WS, check=False) == k3moe.K3MOE_EINVAL
    assert k3moe.k3moe_combine(d, 4, FAKE, FAKE, FAKE, FAKE, FAKE + 2, FAKE, WS, check=False) == k3moe.K3MOE_EUNSUPPORTED
    w = k3moe.k3moe_weights(FAKE, FAKE, FAKE, FAKE, FAKE, _experts())
    assert k3moe.k3moe_layer(d, 4, FAKE, None, FAKE, None, None, WS, check=False) == k3moe.K3MOE_EINVAL
    assert k3moe.k3moe_layer(d, 4, FAKE, w, None, None, None, WS, check=False) == k3moe.K3MOE_EINVAL
    wb = k3moe.k3moe_weights(FAKE, None, FAKE, FAKE, FAKE, _experts())
    assert k3moe.k3moe_layer(d, 4, FAKE, wb, FAKE, None, None, WS, check=False) == k3moe.K3MOE_EINVAL
    assert k3moe.k3moe_layer(d, 0, FAKE, w, FAKE, None, None, WS, check=False) == k3moe.K3MOE_OK
    with pytest.raises(k3moe.K3MoeError):
        k3moe.k3moe_layer(d, 4, FAKE, None, FAKE, None, None, WS)


def test_expert_path_switch_host_only():
    prev = k3moe.k3moe_set_expert_path(k3moe.EXPERT_PATH_GEMM)
    try:
        assert k3moe.k3moe_set_expert_path(k3moe.EXPERT_PATH_GEMV) == k3moe.EXPERT_PATH_GEMM
        assert k3moe.load().k3moe_set_expert_path(3) == k3moe.K3MOE_EINVAL
        assert k3moe.load().k3moe_set_expert_path(-1) == k3moe.K3MOE_EINVAL
        assert k3moe.k3moe_set_expert_path(k3moe.EXPERT_PATH_AUTO) == k3moe.EXPERT_PATH_GEMV
    finally:
        k3moe.k3moe_set_expert_path(prev)


def test_shared_workspace_size_grows_with_T():
    # a workspace sized for a batch serves every smaller batch
    lib = k3moe
    for d in (k3gen.K3, k3gen.TINY):
        prev = 0
        for T in list(range(0, 300)) + list(range(300, 5000, 7)):
            n = lib.k3moe_shared_workspace_size(d, 2, T)
            assert n >= prev, (d, T)
            prev = n


def test_layer_workspace_size_grows_with_T():
    lib = k3moe
    for d in (k3gen.K3, k3gen.TINY):
        prev = 0
        for T in list(range(0, 300)) + list(range(300, 5000, 7)):
            n = lib.k3moe_workspace_size(d, T)
            assert n >= prev, (d, T)
            prev = n


def test_variant_fields_checked_on_the_host():
    # the approximation switches are validated before anything runs (host-only size query)
    import dataclasses
    lib = k3moe
    base = k3gen.TINY
    assert lib.k3moe_workspace_size(dataclasses.replace(base, topp=0.7, idot=1), 4) > 0
    for bad in (dict(topp=-0.1), dict(topp=float("nan")), dict(topp=float("inf")), dict(idot=2), dict(idot=-1)):
        with pytest.raises(lib.K3MoeError) as e:
            lib.k3moe_workspace_size(dataclasses.replace(base, **bad), 4)
        assert e.value.status == lib.K3MOE_EINVAL, bad
    # the shared experts' own checks
    assert lib.k3moe_shared_workspace_size(base, 2, 5) > 0
    for n_shared, T, code in ((0, 5, lib.K3MOE_EINVAL), (1, 5, lib.K3MOE_EUNSUPPORTED), (2, -1, lib.K3MOE_EINVAL)):
        with pytest.raises(lib.K3MoeError) as e:
            lib.k3moe_shared_workspace_size(base, n_shared, T)
        assert e.value.status == code, (n_shared, T)


def test_shared_workspace_covers_the_gemm_form_at_one_token():
    # a shared-expert width whose one-token activations do not fit the GEMV form's LDS
    # (SI * 4 > 64 KB, or H * 4 > 64 KB) runs the GEMM form even at T = 1: its workspace
    # must then hold the GEMM's buffers (gate|up products, act's two bf16 pieces, the
    # down product), not only the one-token act row
    import dataclasses
    lib = k3moe
    cases = [(dataclasses.replace(k3gen.TINY, inter=6144), 3),      # SI = 18432
             (dataclasses.replace(k3gen.TINY, hidden=20480), 2)]    # H * 4 = 80 KB
    for d, n_shared in cases:
        SI, H = n_shared * d.inter, d.hidden
        one = lib.k3moe_shared_workspace_size(d, n_shared, 1)
        # at least the gate|up product (2 SI fp32), the two pieces of act (2 SI bf16) and
        # the down product (H fp32), each region 256-byte aligned
        need = 2 * SI * 4 + 2 * (SI * 2) + H * 4
        assert one >= need, (d, n_shared, one, need)
        prev = 0
        for T in range(0, 40):
            n = lib.k3moe_shared_workspace_size(d, n_shared, T)
            assert n >= prev, (d, T)
            prev = n
    # the narrow shape keeps the one-token GEMV form's single act row
    assert lib.k3moe_shared_workspace_size(k3gen.TINY, 2, 1) < 2 * 2 * k3gen.TINY.inter * 4


def test_expert_path_switch_is_per_thread():
    import threading
    prev = k3moe.k3moe_set_expert_path(k3moe.EXPERT_PATH_GEMV)
    seen = []
    try:
        def other():
            # another thread starts from the default and its setting stays its own
            seen.append(k3moe.k3moe_set_expert_path(k3moe.EXPERT_PATH_GEMM))
        th = threading.Thread(target=other)
        th.start()
        th.join()
        assert seen == [k3moe.EXPERT_PATH_AUTO]
        assert k3moe.k3moe_set_expert_path(k3moe.EXPERT_PATH_AUTO) == k3moe.EXPERT_PATH_GEMV
    finally:
        k3moe.k3moe_set_expert_path(prev)


def test_noalloc_refuses_on_the_host():
    # the no-allocation layer: bad arguments and batches whose workspace exceeds its fixed
    # device array are refused before any HIP call
    L = k3moe.load()
    fake = FAKE
    w = k3moe.k3moe_weights(fake, fake, fake, fake, fake, _experts())
    hdr = open(os.path.join(INCLUDE, "k3moe.h")).read()
    m = re.search(r"#define K3MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and k3moe.NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))
    assert k3moe.k3moe_workspace_size(k3gen.K3, 39) <= k3moe.NOALLOC_SCRATCH_BYTES
    assert k3moe.k3moe_workspace_size(k3gen.K3, 64) > k3moe.NOALLOC_SCRATCH_BYTES
    assert k3moe.k3moe_layer_noalloc(k3gen.K3, 64, fake, w, fake, None, None, check=False) == k3moe.K3MOE_EWORKSPACE
    assert k3moe.k3moe_layer_noalloc(_d(hidden=0), 4, fake, w, fake, None, None, check=False) == k3moe.K3MOE_EINVAL
    assert k3moe.k3moe_layer_noalloc(_d(), -1, fake, w, fake, None, None, check=False) == k3moe.K3MOE_EINVAL
    assert L.k3moe_layer_noalloc(None, 4, fake, ctypes.byref(w), fake, None, None, None) == k3moe.K3MOE_EINVAL
