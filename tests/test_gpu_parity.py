"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle, on the same
seeded inputs. Expert indices and all integer outputs bit-exact; floating outputs per
token row within rel-L2 <= 1e-5 and max-abs <= 1e-4 * max|ref| (the layer's stated
tolerance; stage outputs are held to the same bar)."""
from __future__ import annotations

import copy
import dataclasses
import sys

import numpy as np
import pytest

import k3gen
import oracle
from tests import _inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from mxfp4_routed_expert_amd import device, k3moe  # noqa: E402

REL = 1e-5
ABSF = 1e-4


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def check_rows(got: np.ndarray, ref: np.ndarray, what: str, rel=REL, absf=ABSF):
    got = np.asarray(got, np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    assert np.all(np.isfinite(got)), what
    err = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    mabs = np.max(np.abs(got - ref), axis=1) / np.maximum(np.max(np.abs(ref), axis=1), 1e-30)
    say(f"  {what}: max row rel-L2 {err.max():.3e}, max abs/max|ref| {mabs.max():.3e}")
    assert err.max() <= rel, (what, float(err.max()))
    assert mabs.max() <= absf, (what, float(mabs.max()))
    return float(err.max())


class Host:
    def __init__(self, dims, seed, dense=None, blobs=None):
        self.dims = dims
        self.dense = dense if dense is not None else k3gen.gen_dense(dims, seed)
        self.lay = k3gen.ExpertLayout(dims)
        self.blobs = blobs if blobs is not None else k3gen.gen_experts(dims, seed, 0, dims.n_experts)
        self.ex = oracle.ExpertSet(self.blobs, self.lay.blob_bytes, self.lay.offsets)
        B = self.lay.blob_bytes
        chunks = ((e0, self.blobs[e0 * B:min(dims.n_experts, e0 + 64) * B])
                  for e0 in range(0, dims.n_experts, 64))
        self.dev = device.upload_layer(dims, self.dense, chunks, B, self.lay.offsets)


@pytest.fixture(scope="module")
def tiny():
    return Host(k3gen.TINY, 0)


# a tiny shape whose expert passes both have K % 128 == 0 (both can run as grouped
# GEMMs) and whose expert count is a multiple of 64 (the router can run as a GEMM)
TINY_MM = dataclasses.replace(k3gen.TINY, inter=128, n_experts=64)


@pytest.fixture(scope="module")
def tiny_mm():
    return Host(TINY_MM, 0)


def nan_scale_blobs(dims, seed, frac=0.03):
    """Expert blobs with a seeded fraction of every weight-scale tensor set to the ue8m0
    NaN code 255 (each such 32-column group contributes zero)."""
    lay = k3gen.ExpertLayout(dims)
    blobs = k3gen.gen_experts(dims, seed, 0, dims.n_experts).copy()
    rng = np.random.default_rng(seed + 1000)
    sizes = dict(lay.sizes)
    per = blobs.reshape(dims.n_experts, lay.blob_bytes)
    for name in ("w1s", "w3s", "w2s"):
        o, n = lay.offsets[name], sizes[name]
        sel = rng.random((dims.n_experts, n)) < frac
        per[:, o:o + n][sel] = 255
    return blobs


@pytest.fixture(scope="module")
def tiny_mm_nan():
    return Host(TINY_MM, 0, blobs=nan_scale_blobs(TINY_MM, 0))


@pytest.fixture
def expert_path():
    """Set the expert-pass form for one test; the default is restored afterwards."""
    prev = k3moe.k3moe_set_expert_path(k3moe.EXPERT_PATH_AUTO)
    yield k3moe.k3moe_set_expert_path
    k3moe.k3moe_set_expert_path(prev)


@pytest.fixture(scope="module")
def k3():
    say("generating and uploading the K3-shape layer (896 experts, 15.7 GB)")
    return Host(k3gen.K3, 1)


def t_(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


def run_layer(h: Host, x: np.ndarray, gemm_scales: bool = True, router_planes: bool = True):
    d = h.dims
    T = x.shape[0]
    xd = t_(x.view(np.int16))
    y = torch.empty((T, d.hidden), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, d.topk), dtype=torch.int32, device="cuda")
    w = torch.empty((T, d.topk), dtype=torch.float32, device="cuda")
    ws = device.workspace(d, T)
    k3moe.k3moe_layer(d, T, xd, h.dev.weights_struct(gemm_scales, router_planes), y, idx, w, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def compare_layer(h: Host, x: np.ndarray, rows=None, what="layer"):
    y, idx, w = run_layer(h, x)
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    ref = oracle.layer(h.dims, x[rows], h.dense, h.ex)
    assert np.array_equal(idx[rows], ref["idx"]), f"{what}: expert ids differ"
    check_rows(w[rows], ref["w"], f"{what} weights", rel=1e-6, absf=1e-6)
    return check_rows(y[rows], ref["y"], f"{what} y")


def stages(h: Host, x: np.ndarray):
    """Each ABI stage alone, fed the oracle's own inputs for that stage."""
    d = h.dims
    T, K, L, E = x.shape[0], d.topk, d.latent, d.n_experts
    ws = device.workspace(d, T)
    ref = oracle.layer(d, x, h.dense, h.ex, want_inner=True)
    xd = t_(x.view(np.int16))
    # route
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    k3moe.k3moe_route(d, T, xd, h.dev.w_router, h.dev.bias, idx, w, ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    check_rows(w.cpu().numpy(), ref["w"], "route weights", rel=1e-6, absf=1e-6)
    # latent projection
    z = torch.empty((T, L), dtype=torch.float32, device="cuda")
    k3moe.k3moe_latent_proj_bf16(d, T, xd, h.dev.w_down, z, ws)
    torch.cuda.synchronize()
    check_rows(z.cpu().numpy(), ref["z"], "latent z", rel=1e-6, absf=1e-6)
    # dispatch on the oracle's ids
    off_r, sp_r, ps_r = oracle.dispatch(ref["idx"], E)
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * K, dtype=torch.int32, device="cuda")
    ps = torch.empty(T * K, dtype=torch.int32, device="cuda")
    k3moe.k3moe_dispatch(d, T, t_(ref["idx"]), off, sp, ps, ws)
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), off_r)
    assert np.array_equal(sp.cpu().numpy(), sp_r)
    assert np.array_equal(ps.cpu().numpy(), ps_r)
    # experts on the oracle's z, in the oracle's sorted order
    edn = torch.empty((T * K, L), dtype=torch.float32, device="cuda")
    k3moe.k3moe_expert_glu_mxfp4(d, T, t_(ref["z"]), h.dev.experts_struct(), t_(off_r), t_(sp_r), edn, ws)
    torch.cuda.synchronize()
    tok = sp_r // K
    exid = ref["idx"].reshape(-1)[sp_r]
    edn_ref = oracle.expert_pairs(d, tok, exid, ref["z"], h.ex)
    check_rows(edn.cpu().numpy(), edn_ref, "expert edn")
    # combine on the oracle's edn
    y = torch.empty((T, d.hidden), dtype=torch.float32, device="cuda")
    k3moe.k3moe_combine(d, T, t_(edn_ref), t_(ps_r), t_(ref["w"]), h.dev.norm_w, h.dev.w_up, y, ws)
    torch.cuda.synchronize()
    check_rows(y.cpu().numpy(), ref["y"], "combine y")


# ------------------------------------------------------------------ tiny (config 0)
def test_tiny_stages(tiny):
    x, _ = _inputs.gap_fixed_x(tiny.dims, 0, 4, tiny.dense["w_router"], tiny.dense["bias"])
    stages(tiny, x)


def test_tiny_layer_config0(tiny):
    x, _ = _inputs.gap_fixed_x(tiny.dims, 0, 4, tiny.dense["w_router"], tiny.dense["bias"])
    compare_layer(tiny, x, what="tiny T=4")


@pytest.mark.parametrize("T", [1, 2, 3, 4, 16, 64, 65, 129, 300])
def test_tiny_layer_ragged_T(tiny, T):
    say(f"tiny layer T={T}")
    x, _ = _inputs.gap_fixed_x(tiny.dims, 100 + T, T, tiny.dense["w_router"], tiny.dense["bias"])
    compare_layer(tiny, x, what=f"tiny T={T}")


@pytest.mark.parametrize("mode", [k3moe.EXPERT_PATH_GEMV, k3moe.EXPERT_PATH_GEMM])
@pytest.mark.parametrize("T", [1, 64, 300])
def test_tiny_mm_nan_scales_both_expert_forms(tiny_mm_nan, expert_path, mode, T):
    """Weight groups whose scale byte is the NaN code contribute zero in both forms."""
    expert_path(mode)
    say(f"tiny (inter 128) layer with NaN weight scales T={T} expert form {mode}")
    x, _ = _inputs.gap_fixed_x(TINY_MM, 20 + T, T, tiny_mm_nan.dense["w_router"], tiny_mm_nan.dense["bias"])
    compare_layer(tiny_mm_nan, x, what=f"nan scales T={T} form {mode}")


@pytest.mark.parametrize("mode", [k3moe.EXPERT_PATH_GEMV, k3moe.EXPERT_PATH_GEMM])
@pytest.mark.parametrize("T", [1, 5, 16, 64, 65, 300, 700])
def test_tiny_mm_shape_both_expert_forms(tiny_mm, expert_path, mode, T):
    """Both expert-pass forms on the same inputs; T = 700 gives experts of more than one
    64-token column tile, T = 1 and 5 experts with a single token."""
    expert_path(mode)
    say(f"tiny (inter 128) layer T={T} expert form {mode}")
    x, _ = _inputs.gap_fixed_x(tiny_mm.dims, 200 + T, T, tiny_mm.dense["w_router"], tiny_mm.dense["bias"])
    compare_layer(tiny_mm, x, what=f"tiny-mm T={T} form {mode}")


def test_tiny_mm_stages_gemm(tiny_mm, expert_path):
    expert_path(k3moe.EXPERT_PATH_GEMM)
    x, _ = _inputs.gap_fixed_x(tiny_mm.dims, 7, 200, tiny_mm.dense["w_router"], tiny_mm.dense["bias"])
    stages(tiny_mm, x)


# a shape whose expert passes have several 256-column steps with a partial last one
# (latent 384: 12 groups; inter 160: 5 groups) and row blocks that end inside M
RAGGED_STEPS = dataclasses.replace(k3gen.TINY, latent=384, inter=160, n_experts=24)


@pytest.fixture(scope="module")
def ragged_steps():
    return Host(RAGGED_STEPS, 5)


def crafted_pairs(E: int, K: int, counts, seed: int) -> np.ndarray:
    """Expert ids [T, K] whose per-expert pair counts start with `counts` (experts 0, 1,
    ...) and are filled up to a multiple of K with one pair each on the later experts, in
    a seeded random order over the pairs."""
    ids = [e for e, c in enumerate(counts) for _ in range(c)]
    e = len(counts)
    while len(ids) % K:
        ids.append(e % E)
        e += 1
    rng = np.random.default_rng(seed)
    return rng.permutation(np.asarray(ids, np.int32)).reshape(-1, K)


@pytest.mark.parametrize("mode", [k3moe.EXPERT_PATH_GEMV, k3moe.EXPERT_PATH_GEMM])
@pytest.mark.parametrize("shape", ["tiny_mm", "ragged_steps"])
def test_expert_pass_counts_around_the_gemv_split(request, expert_path, shape, mode):
    """The expert stage on a dispatch whose experts hold 0, 1, 4 (the most the decode
    kernel takes in one pass), 5 (the fewest the rows-split kernel takes), 12 and 13 (one
    and two of its passes), 24, 25 and 61 pairs: every pair's output row against the
    oracle's, in the GEMV form and in the GEMM form where the shape allows it (the ragged
    shape's down pass, K = 160, stays a GEMV)."""
    h = request.getfixturevalue(shape)
    d = h.dims
    expert_path(mode)
    counts = [0, 1, 4, 5, 12, 13, 24, 25, 61, 0, 3]
    idx = crafted_pairs(d.n_experts, d.topk, counts, 17)
    T, K = idx.shape
    say(f"{shape}: crafted dispatch, T={T}, expert form {mode}")
    z = k3gen.normal_f32(T * d.latent, 900 + T, k3gen.T_ZPROBE).reshape(T, d.latent)
    off, sp, _ = oracle.dispatch(idx, d.n_experts)
    assert list(np.diff(off)[:len(counts)]) == counts
    ws = device.workspace(d, T)
    edn = torch.empty((T * K, d.latent), dtype=torch.float32, device="cuda")
    k3moe.k3moe_expert_glu_mxfp4(d, T, t_(z), h.dev.experts_struct(), t_(off), t_(sp), edn, ws)
    torch.cuda.synchronize()
    ref = oracle.expert_pairs(d, sp // K, idx.reshape(-1)[sp], z, h.ex)
    check_rows(edn.cpu().numpy(), ref, f"{shape} crafted expert edn")


# a latent width whose gate/up pass does not fit the rows-split kernel's LDS (224 scale
# bytes per row) and makes the decode kernel take one token per pass, with an inter
# width (64) that the grouped GEMM form cannot take for the down pass (K % 128 != 0)
WIDE_LATENT = dataclasses.replace(k3gen.TINY, latent=7168, inter=64, n_experts=8, topk=2)


@pytest.fixture(scope="module")
def wide_latent():
    return Host(WIDE_LATENT, 6)


@pytest.mark.parametrize("mode", [k3moe.EXPERT_PATH_AUTO, k3moe.EXPERT_PATH_GEMV, k3moe.EXPERT_PATH_GEMM])
@pytest.mark.parametrize("T", [3, 40])
def test_wide_latent_form_fallbacks(wide_latent, expert_path, mode, T):
    """At T = 40 the 80 pairs over 8 experts take the GEMM form's gate/up pass (auto and
    forced) next to a GEMV-form down pass, or with the GEMV form forced the decode kernel
    over every expert, several passes each (the rows-split kernel does not fit)."""
    expert_path(mode)
    say(f"wide latent (7168) layer T={T} expert form {mode}")
    x, _ = _inputs.gap_fixed_x(WIDE_LATENT, 60 + T, T, wide_latent.dense["w_router"], wide_latent.dense["bias"])
    compare_layer(wide_latent, x, what=f"wide latent T={T} form {mode}")


# a shape whose up-projection (1024 x 1024) splits its K among blocks from 8 tokens on
MID_UP = dataclasses.replace(k3gen.TINY, hidden=1024, latent=1024, inter=256, n_experts=64)


@pytest.fixture(scope="module")
def mid_up():
    return Host(MID_UP, 3)


@pytest.mark.parametrize("T", [7, 8, 37, 128, 200])
def test_layer_up_projection_split_k(mid_up, T):
    say(f"mid shape layer T={T} (up-projection K parts)")
    x, _ = _inputs.gap_fixed_x(mid_up.dims, 50 + T, T, mid_up.dense["w_router"], mid_up.dense["bias"])
    compare_layer(mid_up, x, what=f"mid T={T}")


def test_tiny_dispatch_chunked_and_invalid_ids(tiny):
    d = tiny.dims
    rng = np.random.default_rng(7)
    for T in (1, 63, 64, 65, 200, 1000):
        ids = np.stack([rng.choice(d.n_experts, d.topk, replace=False) for _ in range(T)]).astype(np.int32)
        ids.sort(axis=1)
        ws = device.workspace(d, T)
        off = torch.empty(d.n_experts + 1, dtype=torch.int32, device="cuda")
        sp = torch.empty(T * d.topk, dtype=torch.int32, device="cuda")
        ps = torch.empty(T * d.topk, dtype=torch.int32, device="cuda")
        k3moe.k3moe_dispatch(d, T, t_(ids), off, sp, ps, ws)
        torch.cuda.synchronize()
        o, s, p = oracle.dispatch(ids, d.n_experts)
        assert np.array_equal(off.cpu().numpy(), o) and np.array_equal(sp.cpu().numpy(), s)
        assert np.array_equal(ps.cpu().numpy(), p)
    # out-of-range ids are dropped: pair_slot -1, the rest still a stable sort
    ids = np.array([[0, 5, 40, 2], [1, -3, 5, 9]], np.int32)
    ws = device.workspace(d, 2)
    off = torch.empty(d.n_experts + 1, dtype=torch.int32, device="cuda")
    sp = torch.full((8,), -7, dtype=torch.int32, device="cuda")
    ps = torch.empty(8, dtype=torch.int32, device="cuda")
    k3moe.k3moe_dispatch(d, 2, t_(ids), off, sp, ps, ws)
    torch.cuda.synchronize()
    ps = ps.cpu().numpy()
    assert ps[2] == -1 and ps[5] == -1
    assert off.cpu().numpy()[-1] == 6
    valid = [p for p in range(8) if ps[p] >= 0]
    assert sorted(ps[valid].tolist()) == list(range(6))
    flat = ids.reshape(-1)
    order = sp.cpu().numpy()[:6]
    assert list(order) == sorted(valid, key=lambda p: (flat[p], p))


# 128 experts (two slots per selection lane), top-8, and a router with no x dependence:
# the selection scores are 0.5 + bias, with many equal values
TINY_TIES = dataclasses.replace(k3gen.TINY, n_experts=128, topk=8)


def ties_bias(kind: str) -> np.ndarray:
    e = np.arange(TINY_TIES.n_experts)
    if kind == "all_equal":        # every key equal: the 8 lowest ids
        b = np.zeros(e.shape)
    elif kind == "few_values":     # 5 values; the top one held by 26 experts
        b = ((e * 7) % 5) * 0.01
    elif kind == "above_and_ties":  # 3 above, then ties at the 8th place
        b = ((e * 7) % 5) * 0.01
        b[[3, 50, 100]] = 0.05
    else:                          # 2 above, 126 equal below them
        b = np.zeros(e.shape)
        b[[100, 120]] = 0.05
    return b.astype(np.float32)


@pytest.fixture(scope="module", params=["all_equal", "few_values", "above_and_ties", "two_above_rest_equal"])
def tiny_ties(request):
    dense = k3gen.gen_dense(TINY_TIES, 5)
    dense["w_router"][:] = 0.0
    dense["bias"][:] = ties_bias(request.param)
    return request.param, Host(TINY_TIES, 5, dense=dense)


@pytest.mark.parametrize("T", [1, 4, 300])
def test_tiny_selection_ties_lowest_ids(tiny_ties, T):
    """Equal selection scores go to the lower id, in every top-k path (the one-token
    launch, one wave per token, the GEMM-form router) and in both branches of the
    selection (few keys at the bound, and more than 64 of them)."""
    kind, h = tiny_ties
    say(f"selection ties {kind} T={T}")
    x = k3gen.gen_x(TINY_TIES, 7, T)
    compare_layer(h, x, what=f"ties {kind} T={T}")


# the largest expert count and top-k the library takes (1024 experts, top-32), on the
# tiny layer widths
TINY_MAX = dataclasses.replace(k3gen.TINY, n_experts=1024, topk=32)


@pytest.fixture(scope="module")
def tiny_max():
    return Host(TINY_MAX, 11)


@pytest.mark.parametrize("T", [1, 5, 180, 256])
def test_tiny_max_experts_and_topk(tiny_max, T):
    """16 selection slots per lane, 32 chosen per token; at T = 180 the 5760 pairs run the
    GEMV form's two kernels over 1024 experts, at T = 256 (8192 pairs) the grouped GEMM
    form (the experts of at most four pairs on the decode kernel)."""
    say(f"1024 experts, top-32, T={T}")
    x, _ = _inputs.gap_fixed_x(TINY_MAX, 30 + T, T, tiny_max.dense["w_router"], tiny_max.dense["bias"])
    compare_layer(tiny_max, x, what=f"max experts T={T}")


def test_tiny_combine_random_gamma_and_scale(tiny):
    """RMSNorm weight and routed_scale other than 1 reach the result."""
    import dataclasses
    d = dataclasses.replace(tiny.dims, routed_scale=2.5, renorm=1)
    dense = dict(tiny.dense)
    dense["norm_w"] = k3gen.uniform_f32(d.latent, 3, k3gen.T_GAMMA, 0.5, 1.5)
    h = tiny
    x, _ = _inputs.gap_fixed_x(d, 5, 8, dense["w_router"], dense["bias"])
    ref = oracle.layer(d, x, dense, h.ex)
    T = 8
    y = torch.empty((T, d.hidden), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, d.topk), dtype=torch.int32, device="cuda")
    w = torch.empty((T, d.topk), dtype=torch.float32, device="cuda")
    ws = device.workspace(d, T)
    ww = h.dev.weights_struct()
    gam = t_(dense["norm_w"])
    ww.norm_w = gam.data_ptr()
    k3moe.k3moe_layer(d, T, t_(x.view(np.int16)), ww, y, idx, w, ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    check_rows(w.cpu().numpy(), ref["w"], "scaled weights", rel=1e-6, absf=1e-6)
    check_rows(y.cpu().numpy(), ref["y"], "gamma y")


# ------------------------------------------------------------------ K3 shape
def test_k3_stages_T1(k3):
    x, _ = _inputs.gap_fixed_x(k3.dims, 1, 1, k3.dense["w_router"], k3.dense["bias"])
    stages(k3, x)


def test_k3_layer_config1_T1(k3):
    x, _ = _inputs.gap_fixed_x(k3.dims, 1, 1, k3.dense["w_router"], k3.dense["bias"])
    compare_layer(k3, x, what="K3 T=1")


@pytest.mark.parametrize("T", [2, 3, 4])
def test_k3_layer_few_tokens(k3, T):
    # two to four tokens: the front and the up-projection take every token against one
    # weight stream (three and four: 84 and 112 KB of staged activations)
    x, _ = _inputs.gap_fixed_x(k3.dims, 6 + T, T, k3.dense["w_router"], k3.dense["bias"])
    compare_layer(k3, x, what=f"K3 T={T}")


def test_k3_layer_config2_T64(k3):
    x, _ = _inputs.gap_fixed_x(k3.dims, 2, 64, k3.dense["w_router"], k3.dense["bias"])
    compare_layer(k3, x, what="K3 T=64")


def turn_major_reference(dims, blobs: np.ndarray) -> np.ndarray:
    """The turn-major scale copy written out from the expert blobs' scale bytes (numpy):
    regions for w1, w3, w2 at 256-byte aligned offsets, each [E][ceil(ng/12)][rows][12]
    holding bytes 12j .. 12j+11 of each row (zeros past ng)."""
    lay = k3gen.ExpertLayout(dims)
    per = blobs.reshape(dims.n_experts, lay.blob_bytes)
    sizes = dict(lay.sizes)
    out = []
    for name, rows, ng in (("w1s", dims.inter, dims.latent // 32), ("w3s", dims.inter, dims.latent // 32),
                           ("w2s", dims.latent, dims.inter // 32)):
        o = lay.offsets[name]
        s = per[:, o:o + sizes[name]].reshape(dims.n_experts, rows, ng)
        nt = -(-ng // 12)
        pad = np.zeros((dims.n_experts, rows, nt * 12), np.uint8)
        pad[:, :, :ng] = s
        region = pad.reshape(dims.n_experts, rows, nt, 12).transpose(0, 2, 1, 3).reshape(-1)
        out.append(np.concatenate([region, np.zeros((-region.size) % 256, np.uint8)]))
    return np.concatenate(out)


@pytest.mark.parametrize("which", ["tiny_mm", "tiny_mm_nan"])
def test_turn_major_scales_bytes(which, request):
    """k3moe_prepare_gemm_scales writes exactly the turn-major relayout of the blobs'
    scale bytes (NaN codes and padding included)."""
    h = request.getfixturevalue(which)
    say(f"turn-major scale copy of {which}")
    ref = turn_major_reference(h.dims, h.blobs)
    got = h.dev.gemm_scales.cpu().numpy()
    assert got.size >= ref.size == k3moe.k3moe_gemm_scales_size(h.dims)
    assert np.array_equal(got[:ref.size], ref)


@pytest.mark.parametrize("which,T", [("tiny_mm", 700), ("tiny_mm", 300), ("tiny_mm_nan", 300), ("k3", 64)])
def test_gemm_scales_copy_or_not_same_result(which, T, expert_path, request):
    """The grouped GEMM reading the turn-major copy or the plain scale bytes gives the same
    bits; the plain path is checked against the oracle as well."""
    h = request.getfixturevalue(which)
    expert_path(k3moe.EXPERT_PATH_GEMM)
    say(f"{which} T={T} GEMM form with and without the turn-major scales")
    x, _ = _inputs.gap_fixed_x(h.dims, 300 + T, T, h.dense["w_router"], h.dense["bias"])
    y1, i1, w1 = run_layer(h, x, gemm_scales=True)
    y0, i0, w0 = run_layer(h, x, gemm_scales=False)
    assert np.array_equal(i0, i1) and np.array_equal(w0, w1)
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    rows = np.arange(T) if T <= 300 else np.arange(0, T, 7)
    ref = oracle.layer(h.dims, x[rows], h.dense, h.ex)
    assert np.array_equal(i0[rows], ref["idx"])
    check_rows(y0[rows], ref["y"], f"{which} T={T} plain scales y")


def test_gemm_scales_ignored_by_gemv_form(tiny_mm, expert_path):
    """The GEMV form never reads the copy: the same bits with or without it."""
    expert_path(k3moe.EXPERT_PATH_GEMV)
    x, _ = _inputs.gap_fixed_x(TINY_MM, 77, 64, tiny_mm.dense["w_router"], tiny_mm.dense["bias"])
    y1, _, _ = run_layer(tiny_mm, x, gemm_scales=True)
    y0, _, _ = run_layer(tiny_mm, x, gemm_scales=False)
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))


def bf16_round_bits(v: np.ndarray) -> np.ndarray:
    """The bf16 nearest to each finite fp32 value (ties to the even significand), as the
    upper 16 bits of its fp32 pattern."""
    u = v.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("which", ["tiny_mm", "k3"])
def test_router_planes_exact_split(which, request):
    """k3moe_prepare_router_planes: plane 0 is each router weight rounded to the nearest
    bf16, plane 1 the remainder rounded to bf16, and the three planes sum to the fp32
    weight exactly."""
    h = request.getfixturevalue(which)
    say(f"router planes of {which}")
    E, H = h.dims.n_experts, h.dims.hidden
    assert k3moe.k3moe_router_planes_size(h.dims) == 3 * E * H * 2
    p = h.dev.router_planes.cpu().numpy().view(np.uint16)[:3 * E * H].reshape(3, E, H)
    w = h.dense["w_router"].astype(np.float32)
    assert np.array_equal(p[0], bf16_round_bits(w))
    r1 = (w.astype(np.float64) - bf16_to_f64(p[0])).astype(np.float32)  # exact in fp32
    assert np.array_equal(p[1], bf16_round_bits(r1))
    total = bf16_to_f64(p[0]) + bf16_to_f64(p[1]) + bf16_to_f64(p[2])
    assert np.array_equal(total, w.astype(np.float64))


@pytest.mark.parametrize("which,T", [("tiny_mm", 64), ("tiny_mm", 300), ("k3", 64)])
def test_router_planes_copy_or_not_same_result(which, T, request):
    """The front's GEMM form (40 tokens and more) reading the caller's plane copy or
    splitting the router weights itself gives the same bits; the split path is checked
    against the oracle as well."""
    h = request.getfixturevalue(which)
    say(f"{which} T={T} front GEMM with and without the router plane copy")
    x, _ = _inputs.gap_fixed_x(h.dims, 400 + T, T, h.dense["w_router"], h.dense["bias"])
    y1, i1, w1 = run_layer(h, x, router_planes=True)
    y0, i0, w0 = run_layer(h, x, router_planes=False)
    assert np.array_equal(i0, i1) and np.array_equal(w0.view(np.uint32), w1.view(np.uint32))
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    rows = np.arange(T) if T <= 64 else np.arange(0, T, 5)
    ref = oracle.layer(h.dims, x[rows], h.dense, h.ex)
    assert np.array_equal(i0[rows], ref["idx"])
    check_rows(y0[rows], ref["y"], f"{which} T={T} split router planes y")


@pytest.mark.parametrize("which,T", [("tiny_mm", 15), ("tiny_mm", 39), ("k3", 16), ("k3", 32)])
def test_front_form_by_plane_copy(which, T, request):
    """Below 40 tokens the front runs as a GEMM only when the caller gives the router
    plane copy (from 16 tokens), else as the GEMV forms: both against the oracle."""
    h = request.getfixturevalue(which)
    x, _ = _inputs.gap_fixed_x(h.dims, 500 + T, T, h.dense["w_router"], h.dense["bias"])
    ref = oracle.layer(h.dims, x, h.dense, h.ex)
    for planes in (True, False):
        say(f"{which} T={T} front with router plane copy={planes}")
        y, idx, w = run_layer(h, x, router_planes=planes)
        assert np.array_equal(idx, ref["idx"])
        check_rows(w, ref["w"], f"{which} T={T} planes={planes} weights", rel=1e-6, absf=1e-6)
        check_rows(y, ref["y"], f"{which} T={T} planes={planes} y")


def test_k3_layer_T64_grouped_gemm(k3, expert_path):
    expert_path(k3moe.EXPERT_PATH_GEMM)
    x, _ = _inputs.gap_fixed_x(k3.dims, 2, 64, k3.dense["w_router"], k3.dense["bias"])
    compare_layer(k3, x, what="K3 T=64 grouped GEMM")


@pytest.mark.parametrize("mode", [k3moe.EXPERT_PATH_GEMV, k3moe.EXPERT_PATH_GEMM])
def test_k3_layer_T256_both_expert_forms(k3, expert_path, mode):
    expert_path(mode)
    x, _ = _inputs.gap_fixed_x(k3.dims, 5, 256, k3.dense["w_router"], k3.dense["bias"])
    compare_layer(k3, x, what=f"K3 T=256 form {mode}")


# ------------------------------------------------------------------ top-p tail drop
def with_topp(h: Host, p: float) -> Host:
    """The same uploaded layer with the top-p tail drop set in its dims."""
    v = copy.copy(h)
    v.dims = dataclasses.replace(h.dims, topp=p)
    return v


def compare_topp(h: Host, p: float, T: int, seed: int, what: str):
    v = with_topp(h, p)
    x, _ = _inputs.gap_fixed_x(v.dims, seed, T, v.dense["w_router"], v.dense["bias"])
    compare_layer(v, x, what=what)
    ids = run_layer(v, x)[1]
    say(f"  {what}: kept {np.mean(np.sum(ids >= 0, axis=1)):.2f} of {v.dims.topk} experts per token")
    return ids


@pytest.mark.parametrize("p", [0.5, 0.8])
@pytest.mark.parametrize("T", [1, 2, 3, 64, 300])
def test_tiny_topp_layer(tiny, p, T):
    ids = compare_topp(tiny, p, T, 20 + T, f"tiny top-p {p} T={T}")
    if T >= 64:
        assert (ids < 0).any()


@pytest.mark.parametrize("mode", ["gemv", "gemm"])
@pytest.mark.parametrize("T", [1, 5, 300])
def test_tiny_mm_topp_both_expert_forms(tiny_mm, expert_path, mode, T):
    expert_path(k3moe.EXPERT_PATH_GEMV if mode == "gemv" else k3moe.EXPERT_PATH_GEMM)
    # T = 1: forced GEMV selects in the gate/up pass (positional dispatch), forced GEMM
    # selects in its own launch (compacted dispatch)
    ids = compare_topp(tiny_mm, 0.7, T, 30 + T, f"tiny-mm top-p 0.7 T={T} {mode}")
    if T > 1:
        assert (ids < 0).any()


@pytest.mark.parametrize("T", [1, 50])
def test_tiny_topp_without_renorm_and_scaled(tiny, T):
    # renorm off: the kept weights are the raw scores times routed_scale
    v = copy.copy(tiny)
    v.dims = dataclasses.replace(tiny.dims, topp=0.55, renorm=0, routed_scale=2.5)
    x, _ = _inputs.gap_fixed_x(v.dims, 60 + T, T, v.dense["w_router"], v.dense["bias"])
    compare_layer(v, x, what=f"tiny top-p 0.55 renorm 0 scale 2.5 T={T}")


def test_tiny_topp_route_and_dispatch(tiny):
    # k3moe_route alone writes -1 in place; k3moe_dispatch drops those slots as the oracle does
    v = with_topp(tiny, 0.6)
    d, T = v.dims, 37
    x, _ = _inputs.gap_fixed_x(d, 9, T, v.dense["w_router"], v.dense["bias"])
    ws = device.workspace(d, T)
    idx = torch.empty((T, d.topk), dtype=torch.int32, device="cuda")
    w = torch.empty((T, d.topk), dtype=torch.float32, device="cuda")
    k3moe.k3moe_route(d, T, t_(x.view(np.int16)), v.dev.w_router, v.dev.bias, idx, w, ws)
    torch.cuda.synchronize()
    ridx, rw, _ = oracle.route_batch(d, x, v.dense["w_router"], v.dense["bias"])
    assert np.array_equal(idx.cpu().numpy(), ridx)
    check_rows(w.cpu().numpy(), rw, "tiny top-p route weights", rel=1e-6, absf=1e-6)
    check_dispatch_of(v, ridx, "tiny top-p dispatch")


def test_k3_topp_layer_T1(k3):
    compare_topp(k3, 0.9, 1, 1, "K3 top-p 0.9 T=1")


def test_k3_topp_layer_T64(k3):
    compare_topp(k3, 0.8, 64, 2, "K3 top-p 0.8 T=64")


# ------------------------------------------------------------------ int8 activations
# The int8 rounding of z and act is a float decision on values the GPU and the oracle
# compute about 1e-6 apart (fp32 matrix-core sums against fp64), so a value lying that
# close to a half-step boundary may round the other way on one side. Such a value moves
# its group's input by d = max/127: an act value moves the row's output by about 1e-4
# relative, a z value (it feeds all 16 experts) by up to about 2e-3. At the K3 shape a
# token has a few such act values (measured: most rows near 1e-4), at the tiny shapes
# almost none (rows at the exact bar). The bar for this approximation, from that: rel-L2
# <= 5e-3 and max-abs <= 1e-2 * max|ref| per row, the median row within 5e-4; and the
# rule's own effect, about 1e-2 from the exact layer, must be there (median above 3e-3).
IDOT_REL, IDOT_ABSF, IDOT_MEDIAN = 5e-3, 1e-2, 5e-4


def compare_idot(h: Host, T: int, seed: int, what: str):
    v = copy.copy(h)
    v.dims = dataclasses.replace(h.dims, idot=1)
    x, _ = _inputs.gap_fixed_x(v.dims, seed, T, v.dense["w_router"], v.dense["bias"])
    y, idx, w = run_layer(v, x)
    ref = oracle.layer(v.dims, x, v.dense, v.ex)
    assert np.array_equal(idx, ref["idx"]), f"{what}: expert ids differ"
    check_rows(w, ref["w"], f"{what} weights", rel=1e-6, absf=1e-6)
    check_rows(y, ref["y"], f"{what} y", rel=IDOT_REL, absf=IDOT_ABSF)
    err = np.linalg.norm(y.astype(np.float64) - ref["y"], axis=1) / np.linalg.norm(ref["y"].astype(np.float64), axis=1)
    exact = oracle.layer(h.dims, x, h.dense, h.ex)["y"].astype(np.float64)
    gap = np.linalg.norm(y - exact, axis=1) / np.linalg.norm(exact, axis=1)
    say(f"  {what}: rows past 1e-5 {np.mean(err > 1e-5):.2f}, median distance from the exact layer {np.median(gap):.2e}")
    assert np.median(err) <= IDOT_MEDIAN
    assert np.median(gap) > 3e-3


@pytest.mark.parametrize("T", [1, 2, 3, 64, 300])
def test_tiny_idot_layer(tiny, T):
    compare_idot(tiny, T, 120 + T, f"tiny int8 activations T={T}")


@pytest.mark.parametrize("mode", ["gemv", "gemm"])
@pytest.mark.parametrize("T", [5, 300])
def test_tiny_mm_idot_both_expert_forms(tiny_mm, expert_path, mode, T):
    expert_path(k3moe.EXPERT_PATH_GEMV if mode == "gemv" else k3moe.EXPERT_PATH_GEMM)
    compare_idot(tiny_mm, T, 130 + T, f"tiny-mm int8 activations T={T} {mode}")


@pytest.mark.parametrize("mode", ["gemv", "gemm"])
@pytest.mark.parametrize("T", [3, 64, 300])
def test_tiny_mm_idot_expert_stage_exact_bar(tiny_mm, expert_path, mode, T):
    """The int8-activation expert products alone, on the oracle's own z (so both sides
    round z to int8 identically): edn against the oracle's int8 expert at the exact bar.
    The one decision the two sides can take apart is the rounding of an act value whose
    scaled value a / d lies within the GPU's act error of a half step (the GPU's act is
    about 1e-6 from the fp64 oracle's, so its a / d is within about 1e-4 of it). Pairs with
    such a value (margin 5e-4, by the oracle's act) take the variant's relaxed bar; every
    other pair is held to the exact bar, and they are most pairs."""
    expert_path(k3moe.EXPERT_PATH_GEMV if mode == "gemv" else k3moe.EXPERT_PATH_GEMM)
    d = dataclasses.replace(tiny_mm.dims, idot=1)
    K, L, E = d.topk, d.latent, d.n_experts
    x, _ = _inputs.gap_fixed_x(d, 140 + T, T, tiny_mm.dense["w_router"], tiny_mm.dense["bias"])
    ref = oracle.layer(d, x, tiny_mm.dense, tiny_mm.ex, want_inner=True)
    off, sp, _ = oracle.dispatch(ref["idx"], E)
    ws = device.workspace(d, T)
    edn = torch.empty((T * K, L), dtype=torch.float32, device="cuda")
    k3moe.k3moe_expert_glu_mxfp4(d, T, t_(ref["z"]), tiny_mm.dev.experts_struct(), t_(off), t_(sp), edn, ws)
    torch.cuda.synchronize()
    got = edn.cpu().numpy()
    tok = sp // K
    exid = ref["idx"].reshape(-1)[sp]
    edn_ref, act = oracle.expert_pairs(d, tok, exid, ref["z"], tiny_mm.ex, want_act=True)
    # each act value's distance from a rounding boundary, in steps of its group's scale
    g = act.reshape(act.shape[0], -1, 32)
    dq = (np.max(np.abs(g), axis=2, keepdims=True) / np.float32(127.0)).astype(np.float32)
    r = np.divide(g, dq, out=np.zeros_like(g), where=dq > 0).astype(np.float32)
    dist = np.abs(np.abs(r - np.floor(r)) - np.float32(0.5))
    clean = np.all(dist.reshape(act.shape[0], -1) > 5e-4, axis=1)
    say(f"  int8 expert stage T={T} {mode}: {clean.mean():.2f} of {clean.size} pairs at the exact bar")
    assert clean.mean() >= 0.8
    check_rows(got[clean], edn_ref[clean], f"int8 expert stage T={T} {mode} (exact bar)")
    check_rows(got, edn_ref, f"int8 expert stage T={T} {mode} (all pairs)", rel=IDOT_REL, absf=IDOT_ABSF)


def test_k3_idot_layer_T1(k3):
    compare_idot(k3, 1, 1, "K3 int8 activations T=1")


def test_k3_idot_layer_T64(k3):
    compare_idot(k3, 64, 2, "K3 int8 activations T=64")


# ------------------------------------------------------------------ shared experts
def run_shared(d, n_shared, x: np.ndarray, shd: dict, y0: np.ndarray):
    T = x.shape[0]
    y = t_(y0.astype(np.float32))
    ws = device.shared_workspace(d, n_shared, T)
    k3moe.k3moe_shared_glu_bf16(d, n_shared, T, t_(x.view(np.int16)), shd["sh1"], shd["sh3"], shd["sh2"], y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.fixture(scope="module")
def tiny_shared():
    d = k3gen.TINY
    sh = {n: k3gen.gen_shared(d, 7, n) for n in (2, 4)}
    return d, sh, {n: device.upload_shared(v) for n, v in sh.items()}


@pytest.mark.parametrize("n_shared", [2, 4])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 64, 300])
def test_tiny_shared_experts(tiny_shared, n_shared, T):
    d, sh, shd = tiny_shared
    say(f"tiny shared experts n_shared={n_shared} T={T}")
    x = k3gen.gen_x(d, 11 + T, T)
    zero = np.zeros((T, d.hidden), np.float32)
    got = run_shared(d, n_shared, x, shd[n_shared], zero)
    check_rows(got, oracle.shared(d, x, sh[n_shared], zero, n_shared), f"shared n={n_shared} T={T} alone")
    # added to an existing output, unweighted
    y0 = np.random.default_rng(T).standard_normal((T, d.hidden)).astype(np.float32)
    got = run_shared(d, n_shared, x, shd[n_shared], y0)
    check_rows(got, oracle.shared(d, x, sh[n_shared], y0, n_shared), f"shared n={n_shared} T={T} added")


# a shape whose batches split both shared-expert products along K (gate/up 4 parts,
# down 8 parts below 129 tokens)
SHARED_SPLIT = dataclasses.replace(k3gen.TINY, hidden=1024, inter=1024)


@pytest.fixture(scope="module")
def split_shared():
    d = SHARED_SPLIT
    sh = k3gen.gen_shared(d, 8, 2)
    return d, sh, device.upload_shared(sh)


@pytest.mark.parametrize("T", [2, 37, 128, 129, 300])
def test_shared_experts_split_k(split_shared, T):
    d, sh, shd = split_shared
    say(f"shared experts split-K shape T={T}")
    x = k3gen.gen_x(d, 40 + T, T)
    y0 = np.random.default_rng(T).standard_normal((T, d.hidden)).astype(np.float32)
    got = run_shared(d, 2, x, shd, y0)
    check_rows(got, oracle.shared(d, x, sh, y0, 2), f"shared split-K T={T}")


def test_tiny_shared_host_checks(tiny_shared):
    d, sh, shd = tiny_shared
    x = t_(k3gen.gen_x(d, 1, 2).view(np.int16))
    y0 = np.random.default_rng(0).standard_normal((2, d.hidden)).astype(np.float32)
    y = t_(y0)
    ws = device.shared_workspace(d, 2, 2)
    lib = k3moe
    # inter 96: one shared expert is 96 rows, not a multiple of 64
    assert lib.k3moe_shared_glu_bf16(d, 1, 2, x, shd[2]["sh1"], shd[2]["sh3"], shd[2]["sh2"], y, ws,
                                     check=False) == lib.K3MOE_EUNSUPPORTED
    assert lib.k3moe_shared_glu_bf16(d, 0, 2, x, shd[2]["sh1"], shd[2]["sh3"], shd[2]["sh2"], y, ws,
                                     check=False) == lib.K3MOE_EINVAL
    small = device.shared_workspace(d, 2, 1)
    assert lib.k3moe_shared_glu_bf16(d, 2, 2, x, shd[2]["sh1"], shd[2]["sh3"], shd[2]["sh2"], y, small,
                                     check=False) == lib.K3MOE_EWORKSPACE
    assert lib.k3moe_shared_glu_bf16(d, 2, 2, x, None, shd[2]["sh3"], shd[2]["sh2"], y, ws,
                                     check=False) == lib.K3MOE_EINVAL
    # T = 0 is a no-op; refused calls launched nothing
    lib.k3moe_shared_glu_bf16(d, 2, 0, x, shd[2]["sh1"], shd[2]["sh3"], shd[2]["sh2"], y, ws)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), y0)


# shared-expert widths whose one-token activations do not fit the GEMV form's LDS: one
# token runs the GEMM form (its workspace carved for it)
@pytest.mark.parametrize("kind", ["wide_inter", "wide_hidden"])
@pytest.mark.parametrize("T", [1, 2])
def test_shared_experts_gemm_form_at_one_token(kind, T):
    if kind == "wide_inter":
        d, n_shared = dataclasses.replace(k3gen.TINY, inter=6144), 3   # SI = 18432
    else:
        d, n_shared = dataclasses.replace(k3gen.TINY, hidden=20480), 2  # H * 4 = 80 KB
    say(f"shared experts {kind} (H {d.hidden}, SI {n_shared * d.inter}) T={T}")
    sh = k3gen.gen_shared(d, 9, n_shared)
    shd = device.upload_shared(sh)
    x = k3gen.gen_x(d, 70 + T, T)
    y0 = np.random.default_rng(T).standard_normal((T, d.hidden)).astype(np.float32)
    got = run_shared(d, n_shared, x, shd, y0)
    check_rows(got, oracle.shared(d, x, sh, y0, n_shared), f"shared {kind} T={T}")


@pytest.fixture(scope="module")
def k3_shared():
    say("generating and uploading the K3 shared experts (2 x 3072 wide, 264 MB)")
    sh = k3gen.gen_shared(k3gen.K3, 1, 2)
    return sh, device.upload_shared(sh)


def layer_plus_shared(h: Host, sh, shd, x: np.ndarray, rows, what: str):
    d = h.dims
    T = x.shape[0]
    y, idx, w = run_layer(h, x)
    y = run_shared(d, 2, x, shd, y)
    ref = oracle.layer(d, x[rows], h.dense, h.ex)
    assert np.array_equal(idx[rows], ref["idx"]), f"{what}: expert ids differ"
    check_rows(y[rows], oracle.shared(d, x[rows], sh, ref["y"]), f"{what} y with shared experts")
    # the shared part alone, on a zero output
    zero = np.zeros((T, d.hidden), np.float32)
    alone = run_shared(d, 2, x, shd, zero)
    check_rows(alone[rows], oracle.shared(d, x[rows], sh, zero[rows]), f"{what} shared experts alone")


def test_k3_layer_with_shared_T1(k3, k3_shared):
    x = k3gen.gen_x(k3.dims, 1, 1)
    layer_plus_shared(k3, *k3_shared, x, np.arange(1), "K3 T=1")


def test_k3_layer_with_shared_T2(k3, k3_shared):
    # two tokens: the shared experts' two-token GEMV form
    x = k3gen.gen_x(k3.dims, 3, 2)
    layer_plus_shared(k3, *k3_shared, x, np.arange(2), "K3 T=2")


def test_k3_layer_with_shared_T4(k3, k3_shared):
    # four tokens: the shared experts' GEMV form with 112 KB of staged activations
    x = k3gen.gen_x(k3.dims, 4, 4)
    layer_plus_shared(k3, *k3_shared, x, np.arange(4), "K3 T=4")


def test_k3_layer_with_shared_T64(k3, k3_shared):
    x = k3gen.gen_x(k3.dims, 2, 64)
    layer_plus_shared(k3, *k3_shared, x, np.arange(64), "K3 T=64")


def test_k3_shared_T4096_sampled(k3_shared):
    sh, shd = k3_shared
    d = k3gen.K3
    T = 4096
    x = k3gen.gen_x(d, 3, T)
    y0 = np.random.default_rng(3).standard_normal((T, d.hidden)).astype(np.float32) * 0.05
    got = run_shared(d, 2, x, shd, y0)
    # the first and last token of every 128-token tile of the GEMMs, then random tokens up
    # to 512
    tiles = np.arange(0, T, 128)
    edge = np.unique(np.concatenate([tiles, np.minimum(tiles + 127, T - 1)]))
    rng = np.random.default_rng(4)
    rows = np.sort(np.concatenate([edge, rng.choice(np.setdiff1d(np.arange(T), edge), 512 - edge.size,
                                                    replace=False)]))
    ref = np.concatenate([oracle.shared(d, x[rows[i:i + 128]], sh, y0[rows[i:i + 128]])
                          for i in range(0, rows.size, 128)])
    check_rows(got[rows], ref, f"K3 T=4096 shared on {rows.size} rows")


def check_dispatch_of(h: Host, ids: np.ndarray, what: str):
    d = h.dims
    T = ids.shape[0]
    ws = device.workspace(d, T)
    off = torch.empty(d.n_experts + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * d.topk, dtype=torch.int32, device="cuda")
    ps = torch.empty(T * d.topk, dtype=torch.int32, device="cuda")
    k3moe.k3moe_dispatch(d, T, t_(ids), off, sp, ps, ws)
    torch.cuda.synchronize()
    o, s_, p = oracle.dispatch(ids, d.n_experts)
    n = int(o[-1])  # positions past the dispatched pairs (dropped slots) are unspecified
    assert np.array_equal(off.cpu().numpy(), o), what
    assert np.array_equal(sp.cpu().numpy()[:n], s_[:n]), what
    assert np.array_equal(ps.cpu().numpy(), p), what
    return o


def cover_rows(idx: np.ndarray, off: np.ndarray, sp: np.ndarray, total: int, seed: int, unit: int = 32):
    """Tokens whose y rows are compared at full-batch sizes. Every run of `unit` consecutive
    dispatched slots of every expert (so every column tile of the grouped GEMM, whose
    tiles are whole multiples of 32 slots, and every expert's partial last tile) holds a
    pair of a chosen token: a greedy cover, each step taking, for the first slot run not
    yet covered, its token that covers the most runs not yet covered. Then random tokens
    up to `total`, and the first and last token."""
    T, K = idx.shape
    n = int(off[-1])
    slot_of = np.empty(T * K, np.int64)
    slot_of[sp[:n]] = np.arange(n)
    e_of = idx.reshape(-1).astype(np.int64)
    runs_e = (np.diff(off).astype(np.int64) + unit - 1) // unit
    first_run = np.concatenate([[0], np.cumsum(runs_e)])
    run_of = first_run[e_of] + (slot_of - off[e_of]) // unit     # each pair's slot run
    tok_runs = run_of.reshape(T, K)
    covered = np.zeros(int(first_run[-1]), bool)
    by_run = np.argsort(run_of, kind="stable")
    starts = np.searchsorted(run_of[by_run], np.arange(covered.size + 1))
    chosen = {0, T - 1}
    for t in chosen:
        covered[tok_runs[t]] = True
    for u in range(covered.size):
        if covered[u]:
            continue
        cand = by_run[starts[u]:starts[u + 1]] // K
        gain = [np.count_nonzero(~covered[tok_runs[t]]) for t in cand]
        t = int(cand[int(np.argmax(gain))])
        chosen.add(t)
        covered[tok_runs[t]] = True
    assert covered.all()
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(T), np.fromiter(chosen, np.int64))
    extra = rng.choice(rest, max(0, min(total - len(chosen), rest.size)), replace=False)
    return np.sort(np.concatenate([np.fromiter(chosen, np.int64), extra]))


def oracle_rows(dims, x: np.ndarray, rows: np.ndarray, dense: dict, ex, what: str, chunk: int = 64):
    """The oracle's layer on x[rows], in chunks, printing progress (a few seconds each)."""
    outs = []
    for i in range(0, len(rows), chunk):
        outs.append(oracle.layer(dims, x[rows[i:i + chunk]], dense, ex))
        say(f"  {what}: oracle rows {min(i + chunk, len(rows))}/{len(rows)}")
    return {k: np.concatenate([o[k] for o in outs]) for k in outs[0]}


def prefill_case(h: Host, dense: dict, T: int, x_seed: int, nrows: int, what: str):
    say(f"{what}: gap rule over all tokens (oracle router)")
    x, _ = _inputs.gap_fixed_x(h.dims, x_seed, T, dense["w_router"], dense["bias"])
    xd = t_(x.view(np.int16))
    y = torch.empty((T, h.dims.hidden), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, h.dims.topk), dtype=torch.int32, device="cuda")
    w = torch.empty((T, h.dims.topk), dtype=torch.float32, device="cuda")
    ws = device.workspace(h.dims, T)
    wts = h.dev.weights_struct()
    bias_d = t_(dense["bias"].astype(np.float32))
    wts.bias = bias_d.data_ptr()
    k3moe.k3moe_layer(h.dims, T, xd, wts, y, idx, w, ws)
    torch.cuda.synchronize()
    y, idx, w = y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    ridx, rw, _ = oracle.route_batch(h.dims, x, dense["w_router"], dense["bias"])
    assert np.array_equal(idx, ridx), f"{what}: expert ids differ"
    check_rows(w, rw, f"{what} weights", rel=1e-6, absf=1e-6)
    off = check_dispatch_of(h, ridx, what)
    _, sp, _ = oracle.dispatch(ridx, h.dims.n_experts)
    rows = cover_rows(ridx, off, sp, nrows, x_seed)
    say(f"{what}: y compared on {len(rows)} rows covering every 32-slot run of every expert")
    ref = oracle_rows(h.dims, x, rows, dense, h.ex, what)
    assert np.array_equal(ref["idx"], ridx[rows])
    check_rows(y[rows], ref["y"], f"{what} y on the covering rows")
    return off


# the oracle's rows take about 10 s per 64 on 16 host threads
@pytest.mark.timeout(400)
def test_k3_layer_config3_T4096_sampled(k3):
    off = prefill_case(k3, k3.dense, 4096, 3, 512, "K3 T=4096")
    counts = np.diff(off)
    say(f"  experts touched {np.count_nonzero(counts)}/{k3.dims.n_experts}, max tokens {counts.max()}")
    # the bias spread makes routing uneven: both empty experts and experts whose token
    # list spans several tiles occur, so both edges of the grouped stage are exercised
    assert (counts == 0).any() and counts.max() > 64


# the oracle's rows take about 10 s per 64 on 16 host threads
@pytest.mark.timeout(400)
def test_k3_layer_config4_T8192_skewed_sampled(k3):
    dense = dict(k3.dense)
    p = _inputs.skew_params()
    dense["bias"] = _inputs.skewed_bias(k3.dense["bias"])
    off = prefill_case(k3, dense, 8192, 4, 512, "K3 skewed T=8192")
    counts = np.diff(off)
    hot = (np.arange(k3.dims.n_experts) % p["hot_every"]) == 0
    share = counts[hot].sum() / counts.sum()
    tail15 = np.mean((counts[~hot] >= 1) & (counts[~hot] <= 5))
    say(f"  skewed routing: hot share {share:.3f}, hot tokens max {counts[hot].max()}, "
        f"cold tokens median {np.median(counts[~hot]):.0f}, cold with 1-5 tokens {tail15:.2f}, "
        f"cold with 0 tokens {np.mean(counts[~hot] == 0):.2f}")
    # the workload: 90 experts take about 80% of the pairs, a long tail of 1-5 tokens
    assert 0.78 <= share <= 0.82
    assert tail15 >= 0.5
