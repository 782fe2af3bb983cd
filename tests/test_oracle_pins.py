"""Pins of the CPU oracle against facts that do not come from the oracle itself:
values printed on the pages (tests/golden/mxfp4_format.json), hand-worked decodes,
the E2M1 element format's bit-field definition, closed forms and limits, invariants,
and brute force (tests/_brute.py: dense numpy decode, full sort, fp64 matmul).

Each test is chosen so that a plausible slip in the oracle (a swapped nibble, a
dropped scale, a wrong sign, the capped gate fed to the sigmoid, eps outside the
root, biased scores used as weights, a transposed weight) fails at least one.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest

import k3gen
import oracle
from tests import _brute

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mxfp4_format.json")))


# ---------------------------------------------------------------- decode tables
def test_e2m1_table_matches_page_lut():
    vals = [oracle.e2m1(c) for c in range(16)]
    assert vals == GOLDEN["e2m1_lut"]
    # -0.0 for code 8: sign bit kept
    assert math.copysign(1.0, oracle.e2m1(8)) == -1.0


def test_e2m1_table_matches_bit_field_definition():
    for c in range(16):
        assert oracle.e2m1(c) == _brute.e2m1_from_bits(c)


@pytest.mark.parametrize("s", [118, 124, 127, 130])
def test_all_codes_at_scale(s):
    # every code at four scales against the format definition: value * 2^(s-127)
    for c in range(16):
        packed = np.array([[c | (c << 4)] * 16], np.uint8)      # 32 columns, all code c
        scales = np.array([[s]], np.uint8)
        row = oracle.mxfp4_decode(packed, scales, 32)[0]
        want = _brute.e2m1_from_bits(c) * 2.0 ** (s - 127)
        assert np.all(row == np.float32(want)), (c, s)


def test_e8m0_special_bytes():
    assert oracle.e8m0(127) == 1.0
    assert oracle.e8m0(255) == 0.0                       # NaN byte zeroes the group
    assert oracle.e8m0(254) == 2.0 ** 127
    assert oracle.e8m0(0) == 2.0 ** -127                 # fp32 subnormal, still exact


def test_hand_worked_decodes():
    for byte, s, even, odd in GOLDEN["hand_decodes"]:
        packed = np.full((1, 16), byte, np.uint8)
        row = oracle.mxfp4_decode(packed, np.array([[s]], np.uint8), 32)[0]
        assert row[0] == even and row[1] == odd, (byte, s, row[:2])
        assert math.copysign(1.0, row[0]) == math.copysign(1.0, even)
        assert math.copysign(1.0, row[1]) == math.copysign(1.0, odd)


def test_nibble_order_one_hot():
    # A one-hot x = e_c must read column c. Treating the low nibble as the odd
    # element has the same statistics and fails here.
    rng = np.random.default_rng(5)
    rows, cols = 8, 64
    packed = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(120, 130, (rows, cols // 32), dtype=np.uint8)
    for c in (0, 1, 2, 31, 32, 33, 62, 63):
        x = np.zeros(cols, np.float32)
        x[c] = 1.0
        y = oracle.mxfp4_matvec(x, packed, scales, cols, rows)
        byte = packed[:, c // 2]
        code = (byte & 15) if c % 2 == 0 else (byte >> 4)
        want = np.array([_brute.e2m1_from_bits(int(k)) for k in code]) * 2.0 ** (scales[:, c // 32].astype(np.int64) - 127)
        assert np.array_equal(y, want.astype(np.float32)), c


def test_scale_255_zeroes_only_its_group():
    packed = np.full((1, 32), 0x22, np.uint8)             # 64 columns of 1.0
    scales = np.array([[255, 127]], np.uint8)
    y = oracle.mxfp4_matvec(np.ones(64, np.float32), packed, scales, 64, 1)
    assert y[0] == 32.0


def test_odd_width_tail():
    # 33 columns: 17 bytes, the last high nibble unused; 2 groups of 32 + 1
    packed = np.full((1, 17), 0x2F, np.uint8)            # even -6, odd +1
    packed[0, 16] = 0xF2                                 # column 32 = 1.0, high nibble ignored
    scales = np.array([[127, 127]], np.uint8)
    y = oracle.mxfp4_matvec(np.ones(33, np.float32), packed, scales, 33, 1)
    assert y[0] == 16 * (-6.0) + 16 * 1.0 + 1.0


def test_expert_byte_count_closed_form():
    lay = k3gen.ExpertLayout(k3gen.K3)
    assert lay.blob_bytes == GOLDEN["bytes_per_expert"]
    d = k3gen.K3
    params = 3 * d.inter * d.latent
    assert params == GOLDEN["params_per_expert"]
    assert lay.blob_bytes == params * GOLDEN["bytes_per_param"]
    # the fixture's shape: one w1 slice of 64 rows at width 3584
    fs = GOLDEN["fixture_shape"]
    assert fs["packed_cols"] == d.latent // 2 and fs["scale_cols"] == d.latent // d.group
    assert k3gen.ExpertLayout(k3gen.TINY).blob_bytes == 3 * (96 * 64 + 96 * 4)


# ---------------------------------------------------------------- matvecs
def test_mxfp4_matvec_vs_dense_decode():
    rng = np.random.default_rng(11)
    for rows, cols in [(5, 32), (7, 96), (16, 256)]:
        packed = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
        scales = rng.integers(110, 135, (rows, cols // 32), dtype=np.uint8)
        x = rng.standard_normal(cols).astype(np.float32)
        y = oracle.mxfp4_matvec(x, packed, scales, cols, rows)
        W = _brute.decode_mxfp4(packed, scales)
        ref = (W @ x.astype(np.float64)).astype(np.float32)
        assert np.max(np.abs(y - ref)) <= 1e-6 * np.max(np.abs(ref)), (rows, cols)


def test_bf16_matvec_layout_out_by_in():
    rng = np.random.default_rng(3)
    out, inn = 6, 10
    W = k3gen.normal_bf16(out * inn, 9, 99).reshape(out, inn)
    x = rng.standard_normal(inn).astype(np.float32)
    y = oracle.bf16_matvec(x, W)
    ref = (_brute.bf16_bits_to_f64(W) @ x.astype(np.float64)).astype(np.float32)
    assert np.allclose(y, ref, rtol=1e-6, atol=0)
    # a one-hot x picks column i of W (not row i): catches a transposed operand
    x1 = np.zeros(inn, np.float32)
    x1[3] = 1.0
    assert np.array_equal(oracle.bf16_matvec(x1, W), _brute.bf16_bits_to_f64(W[:, 3]).astype(np.float32))


def test_bf16_widening_is_a_shift():
    assert oracle.lib().k3o_bf16_to_f32(0x3F80) == 1.0
    assert oracle.lib().k3o_bf16_to_f32(0xC040) == -3.0
    assert oracle.lib().k3o_bf16_to_f32(0x0001) == 2.0 ** -133


# ---------------------------------------------------------------- router
def _logit_case(logits, bias, K):
    """H = 1, x = [1]: each expert's logit is its single router weight."""
    Wr = np.array(logits, np.float32).reshape(-1, 1)
    x = np.ones(1, np.float32)
    return oracle.router(x, Wr, np.array(bias, np.float32), K)


def test_router_bias_steers_selection_only():
    logits = [2.0, 1.0, 0.0, -1.0, 0.5, 3.0]
    bias = [0.0, 0.0, 0.6, 0.0, 0.0, -0.5]
    idx, w, sel, gap = _logit_case(logits, bias, 2)
    # selection scores: sigma + bias = [.8808, .7311, 1.1, .2689, .6225, .4526]
    assert list(sel) == [2, 0]                       # expert 5 (largest sigma) is NOT chosen
    assert list(idx) == [0, 2]
    s0 = 1.0 / (1.0 + math.exp(-2.0))                # unbiased scores weight the winners
    s2 = 0.5
    assert w[0] == pytest.approx(s0 / (s0 + s2), rel=1e-7)
    assert w[1] == pytest.approx(s2 / (s0 + s2), rel=1e-7)
    assert gap == pytest.approx(s0 - (1.0 / (1.0 + math.exp(-1.0))), rel=1e-6)


def test_router_tie_lowest_index_wins():
    idx, w, sel, gap = _logit_case([0.3] * 6, [0.0] * 6, 3)
    assert list(sel) == [0, 1, 2]
    assert gap == 0.0
    assert np.allclose(w, 1.0 / 3.0, rtol=1e-7)


def test_router_renorm_off_and_routed_scale():
    Wr = np.array([[1.0], [0.0], [-1.0]], np.float32)
    x = np.ones(1, np.float32)
    idx, w, _, _ = oracle.router(x, Wr, np.zeros(3, np.float32), 2, renorm=0, routed_scale=2.5)
    assert list(idx) == [0, 1]
    assert w[0] == pytest.approx(2.5 / (1.0 + math.exp(-1.0)), rel=1e-7)
    assert w[1] == pytest.approx(1.25, rel=1e-7)


def test_router_brute_force_and_invariants():
    d = k3gen.TINY
    dense = k3gen.gen_dense(d, 0)
    x = k3gen.gen_x(d, 0, 32)
    idx, w, gaps = oracle.route_batch(d, x, dense["w_router"], dense["bias"])
    for t in range(32):
        xf = _brute.bf16_bits_to_f64(x[t])
        bi, bw = _brute.route(xf, dense["w_router"], dense["bias"], d.topk)
        if gaps[t] > 1e-9:
            assert np.array_equal(idx[t], bi)
            assert np.allclose(w[t], bw, rtol=1e-6)
        assert len(set(idx[t].tolist())) == d.topk
        assert np.all((idx[t] >= 0) & (idx[t] < d.n_experts))
        assert np.all(np.diff(idx[t]) > 0)
        assert np.all(w[t] > 0)
        assert abs(float(np.sum(w[t].astype(np.float64))) - 1.0) < 1e-6


def test_router_scores_vs_tanh_logistic_and_weights():
    """The unbiased scores are the logistic of the fp64 logit (checked against the tanh
    form of the logistic), and the router's weights are exactly those scores renormalised
    over the chosen ids (weights use the raw scores, not the biased ones)."""
    d = k3gen.TINY
    dense = k3gen.gen_dense(d, 0)
    x = k3gen.gen_x(d, 1, 24)
    sc = oracle.scores_batch(d, x, dense["w_router"])
    idx, w, _ = oracle.route_batch(d, x, dense["w_router"], dense["bias"])
    for t in range(24):
        logit = dense["w_router"].astype(np.float64) @ _brute.bf16_bits_to_f64(x[t])
        ref = 0.5 * (1.0 + np.tanh(0.5 * logit))
        assert np.allclose(sc[t], ref, rtol=2 ** -23, atol=0)
        s = sc[t, idx[t]].astype(np.float64)
        assert np.allclose(w[t], (s / s.sum()).astype(np.float32), rtol=2 ** -23, atol=0)


# ---------------------------------------------------------------- SiTU, RMSNorm
def test_situ_zero_and_sign():
    assert oracle.situ(0.0, 7.0) == 0.0
    assert oracle.situ(3.0, 0.0) == 0.0
    assert oracle.situ(2.0, -5.0) == -oracle.situ(2.0, 5.0)     # odd in u


def test_situ_bound_reached():
    bound = GOLDEN["situ_bound"]
    assert oracle.situ(1000.0, 1000.0) == bound
    assert oracle.situ(1000.0, -1000.0) == -bound
    for g in (0.1, 1.0, 10.0, 100.0, 1000.0):
        for u in (0.1, 1.0, 10.0, 100.0, 1000.0):
            assert abs(oracle.situ(g, u)) <= bound


def test_situ_sigmoid_reads_uncapped_gate():
    # g = -40: sigmoid(-40) ~ 4e-18 gives ~0; a sigmoid fed the capped gate
    # 4*tanh(-10) ~ -4 would give about -4 * 0.018 * 19 = -1.37.
    assert abs(oracle.situ(-40.0, 25.0)) < 1e-12
    # g large: gate factor -> b1 = 4 and sigmoid -> 1, so y -> 4 * 25 tanh(u/25)
    assert oracle.situ(1000.0, 25.0) == pytest.approx(100.0 * 0.7615941559557649, rel=1e-7)


def test_situ_small_argument_limit():
    # near 0: 4 tanh(g/4) ~ g, sigmoid ~ 1/2, 25 tanh(u/25) ~ u  =>  y ~ g*u/2
    g = u = 1e-4
    assert oracle.situ(g, u) == pytest.approx(0.5 * g * u, rel=1e-3)


def test_rmsnorm_constant_vector_closed_form():
    c, n, eps = 3.0, 128, 1e-5
    out = oracle.rmsnorm(np.full(n, c, np.float32), None, eps)
    assert np.allclose(out, c / math.sqrt(c * c + eps), rtol=1e-7)
    gam = np.linspace(-2, 2, n).astype(np.float32)
    out = oracle.rmsnorm(np.full(n, c, np.float32), gam, eps)
    assert np.allclose(out, gam * (c / math.sqrt(c * c + eps)), rtol=1e-6, atol=1e-7)


def test_rmsnorm_eps_inside_root():
    # x = [3, 4]: mean square 12.5. With a large eps the two placements differ a lot.
    out = oracle.rmsnorm(np.array([3.0, 4.0], np.float32), None, 12.5)
    assert out[0] == pytest.approx(3.0 / 5.0, rel=1e-7)          # 3 / sqrt(12.5 + 12.5)
    assert out[1] == pytest.approx(4.0 / 5.0, rel=1e-7)


# ---------------------------------------------------------------- dispatch
def test_dispatch_is_stable_counting_sort():
    rng = np.random.default_rng(2)
    T, K, E = 50, 4, 13
    ti = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    off, sp, ps = oracle.dispatch(ti, E)
    flat = ti.reshape(-1)
    order = np.argsort(flat, kind="stable")          # library stable sort
    assert np.array_equal(sp, order)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(ps[sp], np.arange(T * K))
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([[0, E]], np.int32), E)


# ---------------------------------------------------------------- whole layer
def _tiny_layer(seed=0, T=4):
    d = k3gen.TINY
    dense = k3gen.gen_dense(d, seed)
    lay = k3gen.ExpertLayout(d)
    blobs = k3gen.gen_experts(d, seed, 0, d.n_experts)
    ex = oracle.ExpertSet(blobs, lay.blob_bytes, lay.offsets)
    x = k3gen.gen_x(d, seed, T)
    return d, dense, lay, blobs, ex, x


def _brute_expert(d, blob, offsets, z):
    """One expert on one latent row by numpy: whole-matrix decode, fp64 products."""
    (p1, s1), (p3, s3), (p2, s2) = _brute.expert_views(blob, d, offsets)
    zin = z.astype(np.float64)
    g = (_brute.decode_mxfp4(p1, s1, d.group) @ zin).astype(np.float32)
    u = (_brute.decode_mxfp4(p3, s3, d.group) @ zin).astype(np.float32)
    a = _brute.situ(g, u, d.b1, d.b2)
    return (_brute.decode_mxfp4(p2, s2, d.group) @ a.astype(np.float64)).astype(np.float32), a


def test_expert_pairs_reads_z_by_token():
    """The expert stage's checker (k3o_expert_pairs): pair q runs expert ex_id[q] on z row
    tok[q]. Pinned to a numpy expert per pair, on pairs whose token differs from their
    position and whose order is shuffled; reading z by pair position instead of by token
    would give other rows, so the pin tells the two apart."""
    d, dense, lay, blobs, ex, x = _tiny_layer(0, 4)
    B = lay.blob_bytes
    n = 24
    T = n  # as many z rows as pairs, so a by-position reading stays in bounds
    rng = np.random.default_rng(11)
    z = rng.standard_normal((T, d.latent)).astype(np.float32)
    tok = ((np.arange(n) + 1 + rng.integers(0, T - 1, n)) % T).astype(np.int32)  # tok[q] != q
    exid = rng.integers(0, d.n_experts, n).astype(np.int32)
    edn, act = oracle.expert_pairs(d, tok, exid, z, ex, want_act=True)
    for q in range(n):
        bref, aref = _brute_expert(d, blobs[exid[q] * B:(exid[q] + 1) * B], lay.offsets, z[tok[q]])
        err = np.linalg.norm(edn[q] - bref.astype(np.float64)) / np.linalg.norm(bref.astype(np.float64))
        assert err < 1e-6, (q, err)
        assert np.allclose(act[q], aref, rtol=1e-6, atol=1e-7), q
        # the same as the one-expert oracle call, bit for bit
        assert np.array_equal(edn[q], oracle.expert(d, ex, int(exid[q]), z[tok[q]])[0]), q
    # shuffled pairs: the same rows, permuted
    perm = rng.permutation(n)
    assert np.array_equal(oracle.expert_pairs(d, tok[perm], exid[perm], z, ex), edn[perm])
    # a by-position reading of z differs from the by-token result
    assert np.all(tok != np.arange(n))
    by_pos = np.stack([oracle.expert(d, ex, int(exid[q]), z[q])[0] for q in range(n)])
    assert not np.any([np.allclose(by_pos[q], edn[q]) for q in range(n)])


def test_layer_matches_brute_force_tiny():
    d, dense, lay, blobs, ex, x = _tiny_layer(0, 8)
    r = oracle.layer(d, x, dense, ex, want_inner=True)
    B = lay.blob_bytes
    for t in range(x.shape[0]):
        b = _brute.layer_token(d, x[t], dense, lambda e: blobs[e * B:(e + 1) * B], lay.offsets)
        assert np.array_equal(r["idx"][t], b["idx"])
        for k in ("z", "acc", "nrm", "y"):
            ref = b[k].astype(np.float64)
            err = np.linalg.norm(r[k][t] - ref) / np.linalg.norm(ref)
            assert err < 1e-6, (t, k, err)


def test_layer_thread_count_invariant():
    d, dense, lay, blobs, ex, x = _tiny_layer(0, 6)
    a = oracle.layer(d, x, dense, ex, nthreads=1)
    b = oracle.layer(d, x, dense, ex, nthreads=4)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["idx"], b["idx"])


def test_combine_identical_experts_and_order():
    # all experts identical => sum_j w_j edn_j = edn (weights sum to 1)
    d, dense, lay, blobs, ex, x = _tiny_layer(0, 3)
    B = lay.blob_bytes
    same = np.tile(blobs[:B], d.n_experts)
    exs = oracle.ExpertSet(same, B, lay.offsets)
    r = oracle.layer(d, x, dense, exs, want_inner=True)
    for t in range(3):
        edn, _, _, _ = oracle.expert(d, exs, 0, r["z"][t])
        assert np.allclose(r["acc"][t], edn, rtol=2e-6, atol=1e-6 * np.max(np.abs(edn)))
    # order invariance: recombining the per-expert outputs in reverse id order
    r = oracle.layer(d, x, dense, ex, want_inner=True)
    for t in range(3):
        edns = [oracle.expert(d, ex, int(e), r["z"][t])[0].astype(np.float64) for e in r["idx"][t]]
        rev = sum(float(w) * e for w, e in reversed(list(zip(r["w"][t], edns))))
        assert np.max(np.abs(rev.astype(np.float32) - r["acc"][t])) <= np.max(np.abs(r["acc"][t])) * 2 ** -23


def test_layer_per_expert_norm_would_differ():
    # the norm is applied to the aggregate: norming each expert first gives another function
    d, dense, lay, blobs, ex, x = _tiny_layer(0, 2)
    r = oracle.layer(d, x, dense, ex, want_inner=True)
    t = 0
    per = sum(float(w) * oracle.rmsnorm(oracle.expert(d, ex, int(e), r["z"][t])[0], None, d.eps).astype(np.float64)
              for w, e in zip(r["w"][t], r["idx"][t]))
    assert np.linalg.norm(per - r["nrm"][t]) / np.linalg.norm(r["nrm"][t]) > 1e-2
    assert np.allclose(r["nrm"][t], oracle.rmsnorm(r["acc"][t], None, d.eps))


@pytest.mark.slow
def test_layer_matches_brute_force_k3_shape_subproblem():
    # K3 widths (H 7168, L 3584, I 3072, K 16) with 24 experts, one token.
    d = k3gen.Dims(hidden=7168, latent=3584, inter=3072, n_experts=24, topk=16, eps=1e-5)
    dense = k3gen.gen_dense(d, 1)
    lay = k3gen.ExpertLayout(d)
    blobs = k3gen.gen_experts(d, 1, 0, d.n_experts)
    ex = oracle.ExpertSet(blobs, lay.blob_bytes, lay.offsets)
    x = k3gen.gen_x(d, 1, 1)
    r = oracle.layer(d, x, dense, ex, want_inner=True)
    B = lay.blob_bytes
    b = _brute.layer_token(d, x[0], dense, lambda e: blobs[e * B:(e + 1) * B], lay.offsets)
    assert np.array_equal(r["idx"][0], b["idx"])
    for k in ("z", "acc", "nrm", "y"):
        ref = b[k].astype(np.float64)
        assert np.linalg.norm(r[k][0] - ref) / np.linalg.norm(ref) < 1e-6, k


# ---------------------------------------------------------------- shared experts
def _tiny_shared(seed, T, n_shared=2):
    d = k3gen.TINY
    return d, k3gen.gen_shared(d, seed, n_shared), k3gen.gen_x(d, seed, T)


def test_shared_matches_brute_force_tiny():
    d, sh, x = _tiny_shared(0, 7)
    y0 = np.asarray(np.random.default_rng(5).standard_normal((7, d.hidden)), np.float32)
    y = oracle.shared(d, x, sh, y0)
    for t in range(7):
        ref = y0[t].astype(np.float64) + _brute.shared_token(d, x[t], sh).astype(np.float64)
        err = np.linalg.norm(y[t] - ref) / np.linalg.norm(ref)
        assert err < 1e-6, (t, err)


def test_shared_zero_down_leaves_y_unchanged():
    d, sh, x = _tiny_shared(1, 4)
    sh = dict(sh, sh2=np.zeros_like(sh["sh2"]))
    y0 = np.asarray(np.random.default_rng(6).standard_normal((4, d.hidden)), np.float32)
    assert np.array_equal(oracle.shared(d, x, sh, y0), y0)


def test_shared_fused_is_sum_of_its_experts():
    # the fused [SI] layout is n_shared experts side by side: row block j of sh1/sh3 and
    # column block j of sh2 form expert j; their outputs add
    d, sh, x = _tiny_shared(2, 3)
    I = d.inter
    zero = np.zeros((3, d.hidden), np.float32)
    fused = oracle.shared(d, x, sh, zero).astype(np.float64)
    parts = sum(oracle.shared(d, x, {"sh1": sh["sh1"][j * I:(j + 1) * I], "sh3": sh["sh3"][j * I:(j + 1) * I],
                                     "sh2": np.ascontiguousarray(sh["sh2"][:, j * I:(j + 1) * I])},
                              zero, n_shared=1).astype(np.float64) for j in range(2))
    assert np.max(np.abs(fused - parts)) <= 1e-5 * np.max(np.abs(fused))
    # and a transposed down matrix (or the gate/up roles swapped) gives another function
    swp = oracle.shared(d, x, {"sh1": sh["sh3"], "sh3": sh["sh1"], "sh2": sh["sh2"]}, zero)
    assert np.linalg.norm(swp - fused) / np.linalg.norm(fused) > 1e-2


def test_shared_one_hot_input_reads_one_column():
    # x = e_c: g and u are column c of sh1 and sh3 exactly; the output is sh2 . SiTU(g, u)
    d, sh, _ = _tiny_shared(3, 1)
    c = 5
    x = np.zeros((1, d.hidden), np.uint16)
    x[0, c] = 0x3F80                      # bf16 1.0
    y = oracle.shared(d, x, sh, np.zeros((1, d.hidden), np.float32))
    g = _brute.bf16_bits_to_f64(sh["sh1"][:, c])
    u = _brute.bf16_bits_to_f64(sh["sh3"][:, c])
    a = _brute.situ(g, u, d.b1, d.b2).astype(np.float64)
    ref = _brute.bf16_bits_to_f64(sh["sh2"]) @ a
    assert np.max(np.abs(y[0] - ref)) <= 1e-6 * np.max(np.abs(ref))


# ---------------------------------------------------------------- top-p tail drop
def _one_hot_router(logits, K):
    """A router whose scores are sigmoid(logits) exactly in fp64 terms: x = e_0."""
    E = len(logits)
    Wr = np.zeros((E, 4), np.float32)
    Wr[:, 0] = logits
    x = np.zeros(4, np.float32)
    x[0] = 1.0
    return x, Wr


def test_topp_hand_case():
    # scores sigmoid(2, 1, 0, -1) = .8808, .7311, .5, .2689: fractions .370, .307, .210, .113
    logits = np.array([2.0, 1.0, 0.0, -1.0], np.float32)
    x, Wr = _one_hot_router(logits, 4)
    sc = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    for p, kept in ((0.3, [0]), (0.6, [0, 1]), (0.7, [0, 1, 2]), (0.95, [0, 1, 2, 3])):
        idx, w, _, margin = oracle.router_topp(x, Wr, np.zeros(4, np.float32), 4, p)
        assert idx.tolist() == [e if e in kept else -1 for e in range(4)], p
        ref = np.array([sc[e] / sc[kept].sum() if e in kept else 0.0 for e in range(4)])
        assert np.allclose(w, ref, rtol=1e-6, atol=1e-7), p
        assert margin > 1e-3
    # without renorm the kept weights are the raw scores
    idx, w, _, _ = oracle.router_topp(x, Wr, np.zeros(4, np.float32), 4, 0.6, renorm=0, routed_scale=2.0)
    assert np.allclose(w, [2 * sc[0], 2 * sc[1], 0, 0], rtol=1e-6)


def test_topp_equal_fractions_keep_lowest_ids():
    x, Wr = _one_hot_router(np.zeros(6, np.float32), 4)
    idx, w, _, _ = oracle.router_topp(x, Wr, np.zeros(6, np.float32), 4, 0.3)
    # the four lowest ids are chosen; fractions all 1/4: 0 < .3 keeps id 0, .25 < .3 keeps id 1
    assert idx.tolist() == [0, 1, -1, -1]
    assert np.allclose(w, [0.5, 0.5, 0, 0])


def test_topp_one_or_more_keeps_all():
    d = k3gen.TINY
    dense = k3gen.gen_dense(d, 0)
    x = k3gen.gen_x(d, 0, 16)
    a = oracle.route_batch(d, x, dense["w_router"], dense["bias"])
    b = oracle.route_batch(dataclasses.replace(d, topp=1.0), x, dense["w_router"], dense["bias"])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("p", [0.3, 0.5, 0.8, 0.95])
def test_topp_brute_force_and_invariants(p):
    d = dataclasses.replace(k3gen.TINY, n_experts=64, topk=8, topp=p)
    dense = k3gen.gen_dense(d, 3)
    x = k3gen.gen_x(d, 3, 200)
    idx, w, _, margins = oracle.route_batch(d, x, dense["w_router"], dense["bias"], want_margins=True)
    full, _, _ = oracle.route_batch(dataclasses.replace(d, topp=0.0), x, dense["w_router"], dense["bias"])
    checked = 0
    for t in range(x.shape[0]):
        xf = _brute.bf16_bits_to_f64(x[t])
        ch, _ = _brute.route(xf, dense["w_router"], dense["bias"], d.topk)
        logit = dense["w_router"].astype(np.float64) @ xf
        sc = (0.5 * (1.0 + np.tanh(0.5 * logit))).astype(np.float32)
        bi, bw = _brute.topp_drop(ch, sc[ch], p)
        kept = idx[t] >= 0
        assert kept.any() and np.array_equal(idx[t][kept], full[t][kept])   # a subset, in place
        assert np.isclose(w[t][kept].sum(), 1.0, atol=1e-6) and np.all(w[t][~kept] == 0)
        f = sc[full[t]].astype(np.float64) / sc[full[t]].astype(np.float64).sum()
        if not kept.all():
            assert f[kept].sum() >= p - 1e-6                  # reaches p
            assert f[kept].sum() - f[kept].min() < p + 1e-6   # and no kept expert is spare
        if margins[t] > 1e-5:                                 # decisions far from the edge
            assert np.array_equal(idx[t], bi), t
            assert np.allclose(w[t], bw, rtol=1e-6, atol=1e-7)
            checked += 1
    assert checked > 150


def test_dispatch_drops_minus_one():
    ids = np.array([[0, -1, 5, 9], [-1, 5, -1, 7]], np.int32)
    off, sp, ps = oracle.dispatch(ids, 10)
    assert ps.tolist()[1] == -1 and ps.tolist()[4] == -1 and ps.tolist()[6] == -1
    assert off[-1] == 5
    flat = ids.reshape(-1)
    valid = [q for q in range(8) if flat[q] >= 0]
    assert sp[:5].tolist() == sorted(valid, key=lambda q: (flat[q], q))
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([[0, -2, 1, 2]], np.int32), 10)


def test_layer_topp_matches_brute_force_tiny():
    d = dataclasses.replace(k3gen.TINY, topp=0.6)
    dense = k3gen.gen_dense(d, 0)
    lay = k3gen.ExpertLayout(d)
    blobs = k3gen.gen_experts(d, 0, 0, d.n_experts)
    ex = oracle.ExpertSet(blobs, lay.blob_bytes, lay.offsets)
    x = k3gen.gen_x(d, 0, 8)
    r = oracle.layer(d, x, dense, ex, want_inner=True)
    assert (r["idx"] < 0).any()          # the rule dropped something
    B = lay.blob_bytes
    for t in range(x.shape[0]):
        b = _brute.layer_token(d, x[t], dense, lambda e: blobs[e * B:(e + 1) * B], lay.offsets)
        assert np.array_equal(r["idx"][t], b["idx"])
        for k in ("acc", "y"):
            ref = b[k].astype(np.float64)
            assert np.linalg.norm(r[k][t] - ref) / np.linalg.norm(ref) < 1e-6, (t, k)


# ---------------------------------------------------------------- int8-activation products
def test_q8_round_hand_cases():
    # amax 127 gives d = 1: q is v rounded to nearest, ties away from zero
    v = np.zeros(32, np.float32)
    v[:6] = [127.0, -2.5, 2.5, 0.49, -0.51, 3.75]
    q, d = oracle.q8_round(v)
    assert d == 1.0
    assert q[:6].tolist() == [127, -3, 3, 0, -1, 4] and not q[6:].any()
    # the largest magnitude maps to +-127 exactly; d = amax / 127 in fp32
    v = np.linspace(-0.8, 0.3, 32).astype(np.float32)
    q, d = oracle.q8_round(v)
    assert q[0] == -127 and d == np.float32(np.float32(0.8) / np.float32(127.0))
    assert np.all(np.abs(q.astype(np.float64) * d - v) <= d / 2 + 1e-9)
    # an all-zero group
    q, d = oracle.q8_round(np.zeros(32, np.float32))
    assert d == 0.0 and not q.any()


def test_matvec_q8_integer_dot_vs_dense_decode():
    # the integer form (doubled codes times q, then 2^(s-127) * d / 2) equals a dense fp64
    # product of the decoded weights with q * d
    rng = np.random.default_rng(11)
    rows, cols = 40, 96
    packed = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(118, 131, (rows, cols // 32), dtype=np.uint8)
    scales[3, 1] = 255
    q = rng.integers(-127, 128, cols).astype(np.int8)
    d = rng.uniform(1e-3, 2e-2, cols // 32).astype(np.float32)
    y = oracle.mxfp4_matvec_q8(q, d, packed, scales, cols, rows)
    xd = q.astype(np.float64) * np.repeat(d.astype(np.float64), 32)
    W = _brute.decode_mxfp4(packed, scales, 32)
    ref = W @ xd
    assert np.all(np.abs(y - ref) <= 2 ** -23 * np.abs(ref) + 1e-12)


def _tiny_layer_idot(seed, T):
    d = dataclasses.replace(k3gen.TINY, idot=1)
    dense = k3gen.gen_dense(d, seed)
    lay = k3gen.ExpertLayout(d)
    blobs = k3gen.gen_experts(d, seed, 0, d.n_experts)
    ex = oracle.ExpertSet(blobs, lay.blob_bytes, lay.offsets)
    return d, dense, lay, blobs, ex, k3gen.gen_x(d, seed, T)


def test_layer_idot_matches_brute_force_tiny():
    d, dense, lay, blobs, ex, x = _tiny_layer_idot(0, 8)
    r = oracle.layer(d, x, dense, ex, want_inner=True)
    B = lay.blob_bytes
    for t in range(x.shape[0]):
        b = _brute.layer_token(d, x[t], dense, lambda e: blobs[e * B:(e + 1) * B], lay.offsets)
        for k in ("acc", "y"):
            ref = b[k].astype(np.float64)
            assert np.linalg.norm(r[k][t] - ref) / np.linalg.norm(ref) < 1e-6, (t, k)


def test_layer_idot_is_an_approximation_of_the_exact_layer():
    d, dense, lay, blobs, ex, x = _tiny_layer_idot(1, 16)
    a = oracle.layer(d, x, dense, ex)["y"].astype(np.float64)
    e = oracle.layer(dataclasses.replace(d, idot=0), x, dense, ex)["y"].astype(np.float64)
    rel = np.linalg.norm(a - e, axis=1) / np.linalg.norm(e, axis=1)
    # int8 per 32 leaves about 2^-8 of each group's maximum: a change of about 1e-2
    assert np.all(rel > 1e-3) and np.all(rel < 5e-2), rel
