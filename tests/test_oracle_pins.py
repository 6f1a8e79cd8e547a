"""Pins of the fp64 CPU oracle against facts that do not come from the oracle itself.

Each test targets a plausible mistake: a dropped term, a wrong sign or index,
a transposed operand, a wrong softmax axis, a wrong iteration count or order,
eps in the wrong place, a wrong flatten order, a wrong scale order.

Independent routes used here: numpy matmul/einsum (library primitives),
closed forms, the textbook scaling-vector form of Sinkhorn-Knopp (Sinkhorn &
Knopp 1967: P = diag(u) K diag(v), u = 1/(K v), v = 1/(K^T u)), invariants
(permutation equivariance, column sums) and bit-level rounding facts.
"""
import math

import numpy as np
import pytest

import oracle
from mhc_inputs import (HC, MIX, bf16_bits_to_f32, f32_to_bf16_bits, layer_inputs, layer_inputs_f32s,
                        sinkhorn_logits, stress_logits)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _bf16_f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _round_bf16_np(v):
    """Test-side fp64 -> bf16 rounding (nearest-even on the float64 bit pattern).

    bf16 keeps 8 of float64's 53 significant bits, so 45 bits are dropped.
    Valid for normal values in binary32 range, which is all these tests use.
    """
    v = np.ascontiguousarray(v, dtype=np.float64)
    u = v.view(np.uint64)
    r = (u + np.uint64((1 << 44) - 1) + ((u >> np.uint64(45)) & np.uint64(1))) >> np.uint64(45)
    r64 = (r << np.uint64(45)).view(np.float64)
    return f32_to_bf16_bits(r64.astype(np.float32))


def _sk_scaling(logits, num_iters, eps):
    """Textbook Sinkhorn-Knopp on K = softmax_rows(L) + eps via scaling vectors."""
    L = np.asarray(logits, dtype=np.float64)
    K = np.exp(L - L.max(axis=-1, keepdims=True))
    K = K / K.sum(axis=-1, keepdims=True) + eps
    v = np.ones(L.shape[:-1])
    for _ in range(num_iters):
        u = 1.0 / np.einsum("...ij,...j->...i", K, v)
        v = 1.0 / np.einsum("...ij,...i->...j", K, u)
    return u[..., :, None] * K * v[..., None, :]


# ---------------------------------------------------------------- rounding

def test_bf16_rounding_bit_facts():
    r = lambda v: int(oracle.round_bf16(np.array([v]))[0])
    assert r(1.0) == 0x3F80
    assert r(-2.0) == 0xC000
    assert r(0.0) == 0x0000
    assert r(-0.0) == 0x8000
    # exact halfway cases go to the even neighbour
    assert r(1.0 + 2.0 ** -8) == 0x3F80
    assert r(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above halfway rounds up -- rounding through binary32 first would
    # lose the 2^-30 and tie back to even (0x3F80)
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert r(float("inf")) == 0x7F80
    assert r(3.5e38) == 0x7F80  # beyond the largest bf16 -> inf


def test_bf16_rounding_matches_independent_rounders():
    g = np.random.default_rng(11)
    v32 = (g.standard_normal(20000) * np.exp(g.uniform(-20, 20, 20000))).astype(np.float32)
    # for binary32-representable values, the generator's binary32 rounder is an independent check
    assert np.array_equal(oracle.round_bf16(v32.astype(np.float64)), f32_to_bf16_bits(v32))
    v64 = g.standard_normal(20000) * np.exp(g.uniform(-20, 20, 20000))
    assert np.array_equal(oracle.round_bf16(v64), _round_bf16_np(v64))


# ---------------------------------------------------------------- A1: RMS statistic

def test_rms_constant_closed_form():
    T, H, c, eps = 3, 37, 1.5, 1e-6
    res = np.full((T, HC, H), f32_to_bf16_bits(np.array([c], np.float32))[0], dtype=np.uint16)
    sq, rstd = oracle.rms(res, eps)
    assert np.allclose(sq, 4 * H * c * c, rtol=0, atol=1e-12)
    assert np.allclose(rstd, 1.0 / math.sqrt(c * c + eps), rtol=1e-15)


def test_rms_matches_numpy_and_k_is_4h():
    inp = layer_inputs(5, 48, cfg=101)
    sq, rstd = oracle.rms(inp.res, 1e-6)
    r = _bf16_f64(inp.res)
    assert np.allclose(sq, (r * r).sum(axis=(1, 2)), rtol=1e-14)
    assert np.allclose(rstd, 1.0 / np.sqrt((r * r).mean(axis=(1, 2)) + 1e-6), rtol=1e-14)


# ---------------------------------------------------------------- A2: projection

def test_project_matches_matmul_with_row_major_flatten():
    inp = layer_inputs(6, 40, cfg=102)
    dot = oracle.project(inp.res, inp.hc_fn)
    ref = _bf16_f64(inp.res).reshape(6, HC * 40) @ inp.hc_fn.astype(np.float64).T
    assert np.allclose(dot, ref, rtol=1e-12, atol=1e-12)


def test_project_one_hot_rows_pick_stream_i_element_h():
    T, H = 4, 16
    inp = layer_inputs(T, H, cfg=103)
    fn = np.zeros((MIX, HC * H), np.float32)
    picks = [(r, r % HC, (5 * r + 3) % H) for r in range(MIX)]
    for r, i, h in picks:
        fn[r, i * H + h] = 1.0
    dot = oracle.project(inp.res, fn)
    r64 = _bf16_f64(inp.res)
    for r, i, h in picks:
        assert np.array_equal(dot[:, r], r64[:, i, h])


# ---------------------------------------------------------------- A3: activations

def _sig(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def test_activation_zero_scale_gives_base_layout():
    g = np.random.default_rng(5)
    T = 3
    dot = g.standard_normal((T, MIX))
    rstd = g.uniform(0.5, 2, T)
    base = g.standard_normal(MIX).astype(np.float32)
    pre, post, L = oracle.mix_activation(dot, rstd, np.zeros(3, np.float32), base, 1e-6, 2.0)
    b = base.astype(np.float64)
    for t in range(T):
        assert np.allclose(pre[t], _sig(b[0:4]) + 1e-6, rtol=1e-15)
        assert np.allclose(post[t], 2.0 * _sig(b[4:8]), rtol=1e-15)
        assert np.array_equal(L[t], b[8:24].reshape(4, 4))


def test_activation_sigmoid_of_zero_is_half():
    pre, post, L = oracle.mix_activation(np.zeros((1, MIX)), np.ones(1), np.ones(3, np.float32),
                                         np.zeros(MIX, np.float32), 1e-6, 1.0)
    assert np.all(pre == 0.5 + 1e-6) and np.all(post == 0.5) and np.all(L == 0.0)


def test_activation_scale_order_pre_post_comb_and_rstd():
    T = 2
    dot = np.zeros((T, MIX))
    dot[:, 1] = 0.3   # a pre logit
    dot[:, 6] = -0.7  # a post logit
    dot[:, 8 + 4 * 2 + 1] = 0.9  # comb[2][1]
    rstd = np.array([2.0, 0.5])
    s = np.array([3.0, 5.0, 7.0], np.float32)
    pre, post, L = oracle.mix_activation(dot, rstd, s, np.zeros(MIX, np.float32), 1e-6, 1.0)
    for t in range(T):
        assert math.isclose(pre[t, 1], _sig(0.3 * rstd[t] * 3.0) + 1e-6, rel_tol=1e-15)
        assert math.isclose(post[t, 2], _sig(-0.7 * rstd[t] * 5.0), rel_tol=1e-15)
        assert math.isclose(L[t, 2, 1], 0.9 * rstd[t] * 7.0, rel_tol=1e-15)
        assert pre[t, 0] == 0.5 + 1e-6 and L[t, 1, 2] == 0.0


# ---------------------------------------------------------------- A4: Sinkhorn

def test_sinkhorn_constant_and_separable_give_quarter():
    lg = np.zeros((3, 4, 4))
    lg[1] = 5.0
    a = np.array([3.0, -2.0, 0.5, -7.0])
    b = np.array([-1.0, 4.0, 2.5, -3.5])
    lg[2] = a[:, None] + b[None, :]
    for it in (1, 2, 20):
        out = oracle.sinkhorn(lg, it, 1e-6)
        assert np.allclose(out, 0.25, atol=1e-15)


def test_sinkhorn_one_iteration_closed_form_pins_softmax_axis():
    # L = 8 at (0,1), 0 elsewhere.  K = softmax_rows(L) + eps has equal row sums,
    # so one (row, column) round gives P_ij = K_ij / sum_i K_ij.
    eps = 1e-6
    L = np.zeros((1, 4, 4))
    L[0, 0, 1] = 8.0
    Q = math.exp(8) / (math.exp(8) + 3)
    q = 1.0 / (math.exp(8) + 3)
    K = np.full((4, 4), 0.25 + eps)
    K[0] = [q + eps, Q + eps, q + eps, q + eps]
    P = K / K.sum(axis=0, keepdims=True)
    out = oracle.sinkhorn(L, 1, eps)[0]
    assert np.allclose(out, P, rtol=1e-14, atol=1e-16)
    # the column-axis softmax would give a different matrix
    Kc = np.full((4, 4), 0.25 + eps)
    Kc[:, 1] = [Q + eps, q + eps, q + eps, q + eps]
    assert not np.allclose(out, Kc / Kc.sum(axis=0, keepdims=True), atol=1e-3)


@pytest.mark.parametrize("iters", [1, 2, 3, 7, 20])
def test_sinkhorn_matches_textbook_scaling_form(iters):
    lg = sinkhorn_logits(2000, seed=3)
    out = oracle.sinkhorn(lg, iters, 1e-6)
    ref = _sk_scaling(lg, iters, 1e-6)
    assert np.allclose(out, ref, rtol=0, atol=1e-13)


def test_sinkhorn_iteration_count_matters():
    lg = sinkhorn_logits(500, seed=4)
    a = oracle.sinkhorn(lg, 19, 1e-6)
    b = oracle.sinkhorn(lg, 20, 1e-6)
    assert np.abs(a - b).max() > 1e-4  # adjacent counts are distinguishable at the 1e-5 tolerance


def test_sinkhorn_columns_sum_to_one_and_rows_converge():
    lg = sinkhorn_logits(4000, seed=5)
    out = oracle.sinkhorn(lg, 20, 1e-6)
    assert np.abs(out.sum(axis=-2) - 1).max() < 1e-14  # last step normalises columns
    assert np.all(out > 0)
    lg1 = np.random.default_rng(6).standard_normal((500, 4, 4))
    lim = oracle.sinkhorn(lg1, 2000, 1e-6)
    assert np.abs(lim.sum(axis=-1) - 1).max() < 1e-9
    assert np.abs(lim.sum(axis=-2) - 1).max() < 1e-14


def test_sinkhorn_permutation_equivariance():
    lg = sinkhorn_logits(300, seed=7).astype(np.float64)
    perm = np.array([2, 0, 3, 1])
    Pm = np.eye(4)[perm]
    out = oracle.sinkhorn(lg, 20, 1e-6)
    out_p = oracle.sinkhorn(Pm @ lg @ Pm.T, 20, 1e-6)
    assert np.allclose(out_p, Pm @ out @ Pm.T, atol=1e-14)


def test_sinkhorn_eps_added_once_after_softmax():
    # Softmax of [0, -1000, -1000, -1000] is one-hot; only the post-softmax eps keeps
    # the other entries positive, so the column of zeros fills with eps-sized mass.
    L = np.full((1, 4, 4), -1000.0)
    for i in range(4):
        L[0, i, 0] = 0.0
    out = oracle.sinkhorn(L, 5, 1e-6)[0]
    ref = _sk_scaling(L, 5, 1e-6)[0]
    assert np.allclose(out, ref, atol=1e-14)
    assert np.allclose(out.sum(axis=0), 1.0, atol=1e-14)
    assert np.all(out[:, 1:] > 0)


def test_sinkhorn_log_of_doubly_stochastic_is_fixed_point():
    d = 0.7 * np.eye(4) + 0.3 * np.roll(np.eye(4), 1, axis=1)
    d = 0.9 * d + 0.1 * 0.25
    out = oracle.sinkhorn(np.log(d)[None], 20, 1e-6)[0]
    assert np.abs(out - d).max() < 5e-6


def test_stress_logits_in_range():
    s = stress_logits()
    assert s.shape == (8, 4, 4) and np.abs(s).max() <= 8.0
    out = oracle.sinkhorn(s, 20, 1e-6)
    assert np.all(np.isfinite(out)) and np.abs(out.sum(axis=-2) - 1).max() < 1e-14


# ---------------------------------------------------------------- A5: collapse

def test_collapse_matches_einsum_and_one_hot():
    inp = layer_inputs(4, 33, cfg=104)
    g = np.random.default_rng(8)
    pre = g.uniform(0, 1, (4, HC))
    y = oracle.collapse(inp.res, pre)
    assert np.allclose(y, np.einsum("ti,tih->th", pre, _bf16_f64(inp.res)), rtol=1e-15, atol=1e-15)
    oh = np.zeros((4, HC))
    oh[:, 2] = 1.0
    assert np.array_equal(oracle.collapse(inp.res, oh), _bf16_f64(inp.res)[:, 2, :])


# ---------------------------------------------------------------- A6: post-map

def test_post_identity_comb_unit_post_is_res_plus_x_bit_exact():
    inp = layer_inputs(5, 64, cfg=105)
    T, H = 5, 64
    out = oracle.post(inp.x, inp.res, np.ones((T, HC)), np.broadcast_to(np.eye(HC), (T, HC, HC)))
    ref = _bf16_f64(inp.res) + _bf16_f64(inp.x)[:, None, :]
    assert np.array_equal(out, ref)
    assert np.array_equal(oracle.round_bf16(out), _round_bf16_np(ref))


def test_post_identity_comb_zero_post_is_res():
    inp = layer_inputs(3, 50, cfg=106)
    out = oracle.post(inp.x, inp.res, np.zeros((3, HC)), np.broadcast_to(np.eye(HC), (3, HC, HC)))
    assert np.array_equal(oracle.round_bf16(out), inp.res)


def test_post_permutation_comb_orientation():
    # comb[o][n] = 1 when n = perm[o]: old stream o moves to new stream perm[o]
    inp = layer_inputs(3, 20, cfg=107)
    perm = [1, 3, 0, 2]
    comb = np.zeros((3, HC, HC))
    for o, n in enumerate(perm):
        comb[:, o, n] = 1.0
    out = oracle.post(inp.x, inp.res, np.zeros((3, HC)), comb)
    r = _bf16_f64(inp.res)
    for o, n in enumerate(perm):
        assert np.array_equal(out[:, n], r[:, o])


def test_post_matches_einsum():
    inp = layer_inputs(4, 24, cfg=108)
    g = np.random.default_rng(9)
    post = g.uniform(0, 2, (4, HC))
    comb = g.uniform(0, 1, (4, HC, HC))
    out = oracle.post(inp.x, inp.res, post, comb)
    ref = _bf16_f64(inp.x)[:, None, :] * post[:, :, None] + np.einsum("toh,ton->tnh", _bf16_f64(inp.res), comb)
    assert np.allclose(out, ref, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- whole pre-map

def _pre_numpy(inp, rms_eps=1e-6, pre_eps=1e-6, sk_eps=1e-6, post_mult=1.0, iters=20):
    """Composition of library routines and closed forms, independent of the oracle's loops."""
    r = _bf16_f64(inp.res)
    T, _, H = r.shape
    flat = r.reshape(T, HC * H)
    rstd = 1.0 / np.sqrt((flat * flat).sum(axis=1) / (HC * H) + rms_eps)
    m = (flat @ inp.hc_fn.astype(np.float64).T) * rstd[:, None]
    s = inp.hc_scale.astype(np.float64)
    b = inp.hc_base.astype(np.float64)
    pre = _sig(m[:, 0:4] * s[0] + b[0:4]) + pre_eps
    post = _sig(m[:, 4:8] * s[1] + b[4:8]) * post_mult
    comb = _sk_scaling((m[:, 8:24] * s[2] + b[8:24]).reshape(T, 4, 4), iters, sk_eps)
    y = np.einsum("ti,tih->th", pre, r)
    return y, post, comb, pre


@pytest.mark.parametrize("post_mult", [1.0, 2.0])
def test_pre_matches_independent_composition(post_mult):
    inp = layer_inputs(16, 256, cfg=1)
    o = oracle.pre(inp.res, inp.hc_fn, inp.hc_scale, inp.hc_base, post_mult=post_mult)
    y, post, comb, pre = _pre_numpy(inp, post_mult=post_mult)
    assert np.allclose(o["pre"], pre, atol=1e-13)
    assert np.allclose(o["post"], post, atol=1e-13)
    assert np.allclose(o["comb"], comb, atol=1e-12)
    assert np.allclose(o["y"], y, atol=1e-12)


def test_pre_hc_permutation_equivariance():
    """Permuting streams, hc_fn column blocks, pre/post rows and comb indices alike
    leaves y unchanged, permutes post and conjugates comb."""
    T, H = 6, 40
    inp = layer_inputs(T, H, cfg=109)
    perm = np.array([3, 0, 2, 1])
    res_p = inp.res[:, perm, :]
    fn = inp.hc_fn.reshape(MIX, HC, H)[:, perm, :]
    rows = np.concatenate([perm, 4 + perm, [8 + 4 * perm[i] + perm[j] for i in range(4) for j in range(4)]])
    fn_p = fn[rows].reshape(MIX, HC * H)
    base_p = inp.hc_base[rows]
    a = oracle.pre(inp.res, inp.hc_fn, inp.hc_scale, inp.hc_base)
    b = oracle.pre(res_p, fn_p, inp.hc_scale, base_p)
    assert np.allclose(b["y"], a["y"], atol=1e-13)
    assert np.allclose(b["post"], a["post"][:, perm], atol=1e-15)
    assert np.allclose(b["pre"], a["pre"][:, perm], atol=1e-15)
    assert np.allclose(b["comb"], a["comb"][:, perm][:, :, perm], atol=1e-13)


def test_pre_zero_scale_collapse_selects_stream():
    T, H = 3, 30
    inp = layer_inputs(T, H, cfg=110, scale=(0.0, 0.0, 0.0))
    inp.hc_base[:4] = [30.0, -30.0, -30.0, -30.0]
    o = oracle.pre(inp.res, inp.hc_fn, inp.hc_scale, inp.hc_base)
    r = _bf16_f64(inp.res)
    assert np.allclose(o["y"], r[:, 0, :], atol=1e-5)
    assert np.allclose(o["pre"][:, 0], 1.0 + 1e-6, atol=1e-12)


def test_sinkhorn_subtracts_row_max_before_exp():
    # The FlashInfer mHC article (section 3.4) subtracts the row maximum before the
    # softmax; with logits near 1000 the un-shifted exp overflows to inf/nan.
    L = np.array([[[1000.0, 999.0, 0.0, 0.0], [0.0, 1000.0, 998.0, 0.0],
                   [0.0, 0.0, 1000.0, 0.0], [997.0, 0.0, 0.0, 1000.0]]])
    out = oracle.sinkhorn(L, 20, 1e-6)
    assert np.all(np.isfinite(out))
    assert np.allclose(out, _sk_scaling(L, 20, 1e-6), atol=1e-13)


# ---------------------------------------------------------------- pre-map from an external projection

def _dots_f32(inp):
    """fp32 dots from numpy's matmul on the row-major flatten (independent of the oracle)."""
    r = _bf16_f64(inp.res)
    T, _, H = r.shape
    return (r.reshape(T, HC * H) @ inp.hc_fn.astype(np.float64).T).astype(np.float32)


def test_pre_from_dots_matches_independent_composition():
    """dots computed outside + sum of squares computed inside == the whole pre-map (FI sections 3 and 4)."""
    inp = layer_inputs(12, 96, cfg=120)
    y, post, comb, pre = _pre_numpy(inp)
    o = oracle.pre_from_dots(_dots_f32(inp), inp.res, inp.hc_scale, inp.hc_base)
    # the only difference is the fp32 rounding of the dots (relative 2^-24 of |dot| <= ~1)
    assert np.abs(o["pre"] - pre).max() < 1e-7
    assert np.abs(o["post"] - post).max() < 1e-7
    assert np.abs(o["comb"] - comb).max() < 1e-6
    assert np.abs(o["y"] - y).max() < 1e-6


def test_pre_from_dots_split_partials_are_summed():
    inp = layer_inputs(9, 64, cfg=121)
    d = _dots_f32(inp)
    one = oracle.pre_from_dots(d, inp.res, inp.hc_scale, inp.hc_base)
    # four equal quarters sum back exactly (power-of-two scaling, fp64 accumulation)
    four = oracle.pre_from_dots(np.stack([d / 4] * 4), inp.res, inp.hc_scale, inp.hc_base)
    for key in ("y", "post", "comb", "pre"):
        assert np.array_equal(one[key], four[key]), key
    # an uneven partition agrees up to fp64 rounding
    g = np.random.default_rng(5)
    parts = g.standard_normal((3,) + d.shape).astype(np.float32)
    parts[2] = (d.astype(np.float64) - parts[0] - parts[1]).astype(np.float32)
    exact = parts.astype(np.float64).sum(axis=0).astype(np.float32)
    a = oracle.pre_from_dots(parts, inp.res, inp.hc_scale, inp.hc_base)
    b = oracle.pre_from_dots(exact, inp.res, inp.hc_scale, inp.hc_base)
    assert np.abs(a["comb"] - b["comb"]).max() < 1e-6 and np.abs(a["pre"] - b["pre"]).max() < 1e-7


def test_pre_from_dots_supplied_sum_of_squares_and_denominator():
    inp = layer_inputs(7, 32, cfg=122)
    d = _dots_f32(inp)
    r = _bf16_f64(inp.res)
    S = (r * r).sum(axis=(1, 2))
    inside = oracle.pre_from_dots(d, inp.res, inp.hc_scale, inp.hc_base)
    given = oracle.pre_from_dots(d, inp.res, inp.hc_scale, inp.hc_base, sqrsum=S.astype(np.float32))
    assert np.abs(inside["pre"] - given["pre"]).max() < 1e-7
    # S and k scaled together by 4: rstd, hence every output, is unchanged bit for bit
    s4 = oracle.pre_from_dots(np.stack([d, d * 0]), inp.res, inp.hc_scale, inp.hc_base,
                              sqrsum=np.stack([S * 4, S * 0]).astype(np.float32), k=4 * HC * 32)
    s1 = oracle.pre_from_dots(d, inp.res, inp.hc_scale, inp.hc_base, sqrsum=S.astype(np.float32))
    for key in ("y", "post", "comb", "pre"):
        assert np.array_equal(s1[key], s4[key]), key


def test_pre_from_dots_rms_denominator_closed_form():
    """S = 3k gives rstd = 1/sqrt(3 + eps): the pre weight is sigmoid(d * rstd * s0 + b) + pre_eps."""
    T, H = 2, 16
    res = np.zeros((T, HC, H), np.uint16)
    d = np.zeros((T, MIX), np.float32)
    d[:, 0] = [1.5, -2.0]
    k = 1000.0
    sq = np.full(T, 3 * k, np.float32)
    o = oracle.pre_from_dots(d, res, np.array([2.0, 1.0, 1.0], np.float32), np.zeros(MIX, np.float32),
                             sqrsum=sq, k=k, rms_eps=0.25, pre_eps=0.0)
    rstd = 1 / np.sqrt(3.25)
    expect = 1 / (1 + np.exp(-(d[:, 0].astype(np.float64) * rstd * 2.0)))
    assert np.allclose(o["pre"][:, 0], expect, rtol=0, atol=1e-15)
    assert np.allclose(o["pre"][:, 1:], 0.5, rtol=0, atol=0)


# ---------------------------------------------------------------- backward passes

def _fd_sinkhorn(L, G, iters, eps, h=1e-6):
    """Central finite differences of sum(G * sinkhorn(L)) with respect to L (the forward oracle only)."""
    out = np.empty_like(L)
    for idx in np.ndindex(*L.shape):
        a = L.copy()
        b = L.copy()
        a[idx] += h
        b[idx] -= h
        fa = (G * oracle.sinkhorn(a, iters, eps)).sum()
        fb = (G * oracle.sinkhorn(b, iters, eps)).sum()
        out[idx] = (fa - fb) / (2 * h)
    return out


@pytest.mark.parametrize("iters,eps,scale", [(1, 1e-6, 1.0), (3, 1e-3, 2.0), (20, 1e-6, 2.0), (20, 1e-6, 6.0)])
def test_sinkhorn_backward_matches_finite_differences(iters, eps, scale):
    g = np.random.default_rng(iters * 7 + int(scale))
    L = g.standard_normal((3, 4, 4)) * scale
    G = g.standard_normal((3, 4, 4))
    d = oracle.sinkhorn_backward(G, L, iters, eps)
    fd = _fd_sinkhorn(L, G, iters, eps)
    assert np.abs(d - fd).max() < 1e-6 * max(1.0, np.abs(fd).max())


def test_sinkhorn_backward_rows_sum_to_zero():
    """Adding a constant to a row of the logits leaves the output unchanged, so each row of
    d_logits sums to zero."""
    g = np.random.default_rng(3)
    L = g.standard_normal((50, 4, 4)) * 3
    G = g.standard_normal((50, 4, 4))
    d = oracle.sinkhorn_backward(G, L, 20, 1e-6)
    assert np.abs(d.sum(axis=-1)).max() < 1e-13


def test_post_backward_bilinear_identities():
    """out is bilinear in (x, res) and (post, comb): <G, out> = <d_x, x> + <d_res, res>
    = <d_post, post> + <d_comb, comb> (Euler's identity for each pair)."""
    inp = layer_inputs(5, 40, cfg=130)
    g = np.random.default_rng(8)
    post = g.uniform(0, 2, (5, HC))
    comb = g.uniform(0, 1, (5, HC, HC))
    G16 = f32_to_bf16_bits(g.standard_normal((5, HC, 40)).astype(np.float32))
    G = _bf16_f64(G16)
    out = oracle.post(inp.x, inp.res, post, comb)
    d_x, d_res, d_post, d_comb = oracle.post_backward(G16, inp.x, inp.res, post, comb)
    inner = (G * out).sum()
    assert abs(inner - ((d_x * _bf16_f64(inp.x)).sum() + (d_res * _bf16_f64(inp.res)).sum())) < 1e-10
    assert abs(inner - ((d_post * post).sum() + (d_comb * comb).sum())) < 1e-10


def test_post_backward_directional_derivatives_and_identity():
    inp = layer_inputs(3, 16, cfg=131)
    g = np.random.default_rng(9)
    post = g.uniform(0, 2, (3, HC))
    comb = g.uniform(0, 1, (3, HC, HC))
    G16 = f32_to_bf16_bits(g.standard_normal((3, HC, 16)).astype(np.float32))
    G = _bf16_f64(G16)
    base = (G * oracle.post(inp.x, inp.res, post, comb)).sum()
    _, _, d_post, d_comb = oracle.post_backward(G16, inp.x, inp.res, post, comb)
    # out is linear in post and comb: a unit step gives the derivative exactly
    p2 = post.copy()
    p2[1, 2] += 1.0
    assert abs(((G * oracle.post(inp.x, inp.res, p2, comb)).sum() - base) - d_post[1, 2]) < 1e-10
    c2 = comb.copy()
    c2[2, 0, 3] += 1.0
    assert abs(((G * oracle.post(inp.x, inp.res, post, c2)).sum() - base) - d_comb[2, 0, 3]) < 1e-10
    # identity comb, unit post: d_x = sum over new streams of G, d_res = G
    eye = np.broadcast_to(np.eye(HC), (3, HC, HC))
    d_x, d_res, _, _ = oracle.post_backward(G16, inp.x, inp.res, np.ones((3, HC)), eye)
    assert np.array_equal(d_res, G) and np.allclose(d_x, G.sum(axis=1), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- pre-map reverse mode
#
# The forward oracle is evaluated at inputs moved by +-d and +-2d along a random
# direction; base values and steps are dyadic, so every moved input is exactly
# representable in its dtype (bf16 streams, fp32 weights, scales, bases, dots).  The
# Richardson combination (4 D(d) - D(2d)) / 3 of the central differences leaves an
# O(d^4) truncation error.

def _pre_bwd_case(seed, T=3, H=8):
    g = np.random.default_rng(seed)
    res_v = g.integers(-15, 16, (T, HC, H)) / 32.0      # |v| < 1/2: v +- 2^-9 and v +- 2^-8 are bf16
    res = f32_to_bf16_bits(res_v.astype(np.float32))
    hc_fn = (g.integers(-128, 129, (MIX, HC * H)) / 256.0).astype(np.float32)
    hc_scale = np.array([0.75, 1.25, 1.5], np.float32)
    hc_base = (g.integers(-64, 65, MIX) / 256.0).astype(np.float32)
    dy = f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    d_post = g.standard_normal((T, HC))
    d_comb = g.standard_normal((T, HC, HC))
    return res, hc_fn, hc_scale, hc_base, dy, d_post, d_comb


def _pre_objective(out, dy, d_post, d_comb):
    return (_bf16_f64(dy) * out["y"]).sum() + (d_post * out["post"]).sum() + (d_comb * out["comb"]).sum()


def _richardson(J, step):
    d1 = (J(step) - J(-step)) / (2 * step)
    d2 = (J(2 * step) - J(-2 * step)) / (4 * step)
    return (4 * d1 - d2) / 3


@pytest.mark.parametrize("seed", [0, 1])
def test_pre_backward_matches_finite_differences(seed):
    res, hc_fn, hc_scale, hc_base, dy, d_post, d_comb = _pre_bwd_case(seed)
    kw = dict(rms_eps=1e-3, pre_eps=1e-6, sinkhorn_eps=1e-6, post_mult=2.0, num_iters=20)
    b = oracle.pre_backward(dy, d_post, d_comb, res, hc_fn, hc_scale, hc_base, **kw)
    g = np.random.default_rng(100 + seed)
    res_v = _bf16_f64(res)
    v_res = g.integers(-1, 2, res.shape).astype(np.float64)
    v_fn = g.integers(-1, 2, hc_fn.shape).astype(np.float64)
    v_sc = np.array([1.0, -1.0, 1.0])
    v_b = g.integers(-1, 2, MIX).astype(np.float64)

    def J(dres=0.0, dfn=0.0, dsc=0.0, db=0.0):
        r = f32_to_bf16_bits((res_v + dres * v_res).astype(np.float32))
        assert np.array_equal(_bf16_f64(r), res_v + dres * v_res)  # the moved streams are exact
        out = oracle.pre(r, (hc_fn + dfn * v_fn).astype(np.float32), (hc_scale + dsc * v_sc).astype(np.float32),
                         (hc_base + db * v_b).astype(np.float32), **kw)
        return _pre_objective(out, dy, d_post, d_comb)

    checks = [
        ((b["d_res"] * v_res).sum(), _richardson(lambda s: J(dres=s), 2.0 ** -9)),
        ((b["d_hc_fn"] * v_fn).sum(), _richardson(lambda s: J(dfn=s), 2.0 ** -12)),
        ((b["d_hc_scale"] * v_sc).sum(), _richardson(lambda s: J(dsc=s), 2.0 ** -10)),
        ((b["d_hc_base"] * v_b).sum(), _richardson(lambda s: J(db=s), 2.0 ** -10)),
    ]
    for analytic, fd in checks:
        assert abs(analytic - fd) < 1e-7 * max(1.0, abs(fd)), (analytic, fd)


@pytest.mark.parametrize("supplied", [False, True])
def test_pre_from_dots_backward_matches_finite_differences(supplied):
    res, _, hc_scale, hc_base, dy, d_post, d_comb = _pre_bwd_case(5)
    T, _, H = res.shape
    g = np.random.default_rng(6)
    dot = (g.integers(-512, 513, (T, MIX)) / 256.0).astype(np.float32)    # |d| <= 2, dyadic
    sq = (g.integers(80, 240, T) / 16.0).astype(np.float32) if supplied else None
    kw = dict(k=40.0, rms_eps=1e-3, pre_eps=1e-6, sinkhorn_eps=1e-6, post_mult=1.5, num_iters=20)
    b = oracle.pre_from_dots_backward(dy, d_post, d_comb, dot, res, hc_scale, hc_base, sqrsum=sq, **kw)
    res_v = _bf16_f64(res)
    v_res = g.integers(-1, 2, res.shape).astype(np.float64)
    v_dot = g.integers(-1, 2, dot.shape).astype(np.float64)
    v_sq = g.integers(-1, 2, T).astype(np.float64)
    v_sc = np.array([-1.0, 1.0, 1.0])
    v_b = g.integers(-1, 2, MIX).astype(np.float64)

    def J(dres=0.0, ddot=0.0, dsq=0.0, dsc=0.0, db=0.0):
        r = f32_to_bf16_bits((res_v + dres * v_res).astype(np.float32))
        assert np.array_equal(_bf16_f64(r), res_v + dres * v_res)
        s = None if sq is None else (sq + dsq * v_sq).astype(np.float32)
        out = oracle.pre_from_dots((dot + ddot * v_dot).astype(np.float32), r,
                                   (hc_scale + dsc * v_sc).astype(np.float32),
                                   (hc_base + db * v_b).astype(np.float32), sqrsum=s, **kw)
        return _pre_objective(out, dy, d_post, d_comb)

    checks = [
        ((b["d_res"] * v_res).sum(), _richardson(lambda s: J(dres=s), 2.0 ** -9)),
        ((b["d_dot"] * v_dot).sum(), _richardson(lambda s: J(ddot=s), 2.0 ** -10)),
        ((b["d_hc_scale"] * v_sc).sum(), _richardson(lambda s: J(dsc=s), 2.0 ** -10)),
        ((b["d_hc_base"] * v_b).sum(), _richardson(lambda s: J(db=s), 2.0 ** -10)),
    ]
    if supplied:
        checks.append(((b["d_sqrsum"] * v_sq).sum(), _richardson(lambda s: J(dsq=s), 2.0 ** -8)))
    else:
        assert b["d_sqrsum"] is None
    for analytic, fd in checks:
        assert abs(analytic - fd) < 1e-7 * max(1.0, abs(fd)), (analytic, fd)


def test_pre_backward_euler_homogeneity():
    """With rms_eps = 0 the mixes are invariant to scaling the streams, and y is linear in
    them, so d/dc J(c res) at c = 1 is <dy, y>: <d_res, res> = <dy, y> (projection, RMS and
    collapse terms together)."""
    res, hc_fn, hc_scale, hc_base, dy, d_post, d_comb = _pre_bwd_case(11, T=4, H=24)
    kw = dict(rms_eps=0.0, pre_eps=1e-6, sinkhorn_eps=1e-6, post_mult=1.0, num_iters=20)
    b = oracle.pre_backward(dy, d_post, d_comb, res, hc_fn, hc_scale, hc_base, **kw)
    y = oracle.pre(res, hc_fn, hc_scale, hc_base, **kw)["y"]
    lhs = (b["d_res"] * _bf16_f64(res)).sum()
    rhs = (_bf16_f64(dy) * y).sum()
    assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(rhs))


def test_pre_backward_scale_and_weight_rows_agree():
    """Scaling the weight rows of group g by c equals scaling hc_scale[g] by c, so
    sum over the group's rows of <d_hc_fn[r], hc_fn[r]> = d_hc_scale[g] * hc_scale[g]."""
    res, hc_fn, hc_scale, hc_base, dy, d_post, d_comb = _pre_bwd_case(12, T=5, H=16)
    b = oracle.pre_backward(dy, d_post, d_comb, res, hc_fn, hc_scale, hc_base)
    for grp, rows in enumerate((slice(0, 4), slice(4, 8), slice(8, 24))):
        lhs = (b["d_hc_fn"][rows] * hc_fn[rows].astype(np.float64)).sum()
        assert abs(lhs - b["d_hc_scale"][grp] * float(hc_scale[grp])) < 1e-12 * max(1.0, abs(lhs))


def test_pre_from_dots_backward_dot_and_square_scaling_invariance():
    """With rms_eps = 0 and the sum of squares supplied, (dots * c, S * c^2) leaves every
    mix unchanged: <d_dot, dot> + 2 <d_sqrsum, S> = 0."""
    res, _, hc_scale, hc_base, dy, d_post, d_comb = _pre_bwd_case(13, T=6, H=8)
    g = np.random.default_rng(14)
    dot = g.standard_normal((6, MIX)) * 3
    sq = g.uniform(5, 50, 6)
    b = oracle.pre_from_dots_backward(dy, d_post, d_comb, dot, res, hc_scale, hc_base, sqrsum=sq, k=32.0,
                                      rms_eps=0.0)
    total = (b["d_dot"] * dot).sum() + 2 * (b["d_sqrsum"] * sq).sum()
    assert abs(total) < 1e-12 * max(1.0, np.abs(b["d_dot"] * dot).sum())


def test_pre_backward_zero_scale_reduces_to_the_logit_level_op():
    """hc_scale = 0: the logits are hc_base alone, so the projection and the RMS statistic
    receive no gradient, d_res = pre dy, and d_hc_base carries the sigmoid derivatives and
    the Sinkhorn reverse mode of the logit-level pre-op."""
    res, hc_fn, _, hc_base, dy, d_post, d_comb = _pre_bwd_case(15, T=4, H=16)
    zero = np.zeros(3, np.float32)
    b = oracle.pre_backward(dy, d_post, d_comb, res, hc_fn, zero, hc_base, post_mult=2.0)
    assert np.array_equal(b["d_hc_fn"], np.zeros_like(b["d_hc_fn"]))
    pre = 1 / (1 + np.exp(-hc_base[:4].astype(np.float64))) + 1e-6
    dyv = _bf16_f64(dy)
    assert np.allclose(b["d_res"], pre[None, :, None] * dyv[:, None, :], rtol=0, atol=1e-15)
    s = 1 / (1 + np.exp(-hc_base.astype(np.float64)))
    d_pre = np.einsum("th,tih->ti", dyv, _bf16_f64(res))
    assert np.allclose(b["d_hc_base"][:4], (d_pre * (s[:4] * (1 - s[:4]))).sum(0), rtol=0, atol=1e-12)
    assert np.allclose(b["d_hc_base"][4:8], (d_post * 2.0 * s[4:8] * (1 - s[4:8])).sum(0), rtol=0, atol=1e-12)
    L = np.broadcast_to(hc_base[8:].astype(np.float64).reshape(HC, HC), (4, HC, HC))
    dL = oracle.sinkhorn_backward(d_comb, L, 20, 1e-6).sum(0).reshape(-1)
    assert np.allclose(b["d_hc_base"][8:], dL, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- model entry and exit

def test_expand_is_a_broadcast_and_head_mean_undoes_it():
    inp = layer_inputs(7, 33, cfg=140)
    s = oracle.expand(inp.x)
    assert np.array_equal(s, np.repeat(inp.x[:, None, :], HC, axis=1))
    assert np.array_equal(oracle.round_bf16(oracle.head_mean(s)), inp.x)


def test_head_mean_matches_numpy_mean():
    inp = layer_inputs(9, 40, cfg=141)
    assert np.allclose(oracle.head_mean(inp.res), _bf16_f64(inp.res).mean(axis=1), rtol=0, atol=1e-15)


def test_head_agrees_with_the_pre_groups_of_the_pre_map():
    """The weighted head is the pre-map's pre group alone: with the same 4 weight rows,
    scale, bases and eps, y and pre agree with the (pinned) whole pre-map."""
    inp = layer_inputs(6, 48, cfg=142, scale=(1.3, 0.7, 0.9))
    full = oracle.pre(inp.res, inp.hc_fn, inp.hc_scale, inp.hc_base, rms_eps=1e-5, pre_eps=3e-3)
    hd = oracle.head(inp.res, inp.hc_fn[:HC], inp.hc_scale[:1], inp.hc_base[:HC], norm_eps=1e-5, hc_eps=3e-3)
    assert np.allclose(hd["pre"], full["pre"], rtol=0, atol=1e-15)
    assert np.allclose(hd["y"], full["y"], rtol=0, atol=1e-13)


def test_head_zero_scale_and_stream_permutation():
    inp = layer_inputs(5, 24, cfg=143)
    b = np.array([0.5, -1.0, 2.0, 0.0], np.float32)
    hd = oracle.head(inp.res, inp.hc_fn[:HC], np.zeros(1, np.float32), b, hc_eps=1e-3)
    assert np.allclose(hd["pre"], 1 / (1 + np.exp(-b.astype(np.float64))) + 1e-3, rtol=0, atol=1e-15)
    perm = [2, 0, 3, 1]
    H = 24
    fn = inp.hc_fn[:HC].reshape(HC, HC, H)              # [row][stream][h]
    fn_p = fn[perm][:, perm].reshape(HC, HC * H)        # rows and stream blocks permuted alike
    a = oracle.head(inp.res, inp.hc_fn[:HC], np.ones(1, np.float32), b)
    p = oracle.head(inp.res[:, perm], fn_p, np.ones(1, np.float32), b[perm])
    assert np.allclose(p["y"], a["y"], rtol=0, atol=1e-12)
    assert np.allclose(p["pre"], a["pre"][:, perm], rtol=0, atol=1e-14)


# ---------------------------------------------------------------- fp32 residual streams

def test_f32_streams_holding_bf16_values_reduce_to_the_bf16_oracle():
    """fp32 streams whose values are bf16 values: every fp32-stream function equals its
    (pinned) bf16-stream counterpart bit for bit."""
    inp = layer_inputs(6, 40, cfg=150, scale=(0.8, 1.2, 1.1))
    wide = bf16_bits_to_f32(inp.res)
    a = oracle.pre(inp.res, inp.hc_fn, inp.hc_scale, inp.hc_base, post_mult=2.0)
    b = oracle.pre_f32s(wide, inp.hc_fn, inp.hc_scale, inp.hc_base, post_mult=2.0)
    for k in ("y", "post", "comb", "pre"):
        assert np.array_equal(a[k], b[k]), k
    g = np.random.default_rng(5)
    post = g.uniform(0, 2, (6, HC))
    comb = g.uniform(0, 1, (6, HC, HC))
    assert np.array_equal(oracle.post(inp.x, inp.res, post, comb), oracle.post_f32s(inp.x, wide, post, comb))
    assert np.array_equal(oracle.head_mean(inp.res), oracle.head_mean_f32s(wide))
    assert np.array_equal(oracle.rms(inp.res, 1e-6)[1], oracle.rms_f32s(wide, 1e-6)[1])
    assert np.array_equal(oracle.project(inp.res, inp.hc_fn), oracle.project_f32s(wide, inp.hc_fn))


def test_f32_streams_keep_their_low_bits():
    """Values below bf16 resolution reach the result: 1 + 2^-20 in every stream element
    gives sum squares 4H (1 + 2^-20)^2 exactly in fp64, and a collapse that sees them."""
    H = 16
    res = np.full((1, HC, H), 1.0 + 2.0 ** -20, np.float32)
    sq, rstd = oracle.rms_f32s(res, 0.0)
    assert sq[0] == 4 * H * (1.0 + 2.0 ** -20) ** 2
    assert rstd[0] == 1.0 / (1.0 + 2.0 ** -20)
    y = oracle.collapse_f32s(res, np.array([[0.25, 0.25, 0.25, 0.25]]))
    assert np.all(y == 1.0 + 2.0 ** -20)


def test_f32_stream_steps_match_numpy():
    inp = layer_inputs_f32s(5, 48, cfg=151)
    r = inp.res.astype(np.float64)
    T, _, H = r.shape
    flat = r.reshape(T, HC * H)
    sq, rstd = oracle.rms_f32s(inp.res, 1e-6)
    assert np.allclose(sq, (flat * flat).sum(axis=1), rtol=1e-14, atol=0)
    assert np.allclose(rstd, 1 / np.sqrt(sq / (HC * H) + 1e-6), rtol=1e-15, atol=0)
    assert np.allclose(oracle.project_f32s(inp.res, inp.hc_fn), flat @ inp.hc_fn.astype(np.float64).T,
                       rtol=1e-12, atol=1e-13)
    pre = np.random.default_rng(3).uniform(0, 1, (T, HC))
    assert np.allclose(oracle.collapse_f32s(inp.res, pre), np.einsum("ti,tih->th", pre, r), rtol=1e-14, atol=1e-14)
    g = np.random.default_rng(4)
    post = g.uniform(0, 2, (T, HC))
    comb = g.uniform(0, 1, (T, HC, HC))
    out = oracle.post_f32s(inp.x, inp.res, post, comb)
    ref = _bf16_f64(inp.x)[:, None, :] * post[:, :, None] + np.einsum("toh,ton->tnh", r, comb)
    assert np.allclose(out, ref, rtol=1e-14, atol=1e-14)
    assert np.allclose(oracle.head_mean_f32s(inp.res), r.mean(axis=1), rtol=0, atol=1e-15)


def test_f32_stream_post_orientation_and_identity():
    """Identity comb with post = 0 returns the streams exactly; a permutation comb sends
    old stream o to new stream perm[o]."""
    inp = layer_inputs_f32s(3, 20, cfg=152)
    eye = np.broadcast_to(np.eye(HC), (3, HC, HC))
    out = oracle.post_f32s(inp.x, inp.res, np.zeros((3, HC)), eye)
    assert np.array_equal(out, inp.res.astype(np.float64))
    perm = [1, 3, 0, 2]
    P = np.zeros((3, HC, HC))
    for o, n in enumerate(perm):
        P[:, o, n] = 1.0
    out = oracle.post_f32s(inp.x, inp.res, np.zeros((3, HC)), P)
    for o, n in enumerate(perm):
        assert np.array_equal(out[:, n], inp.res[:, o].astype(np.float64))


def test_f32_stream_pre_matches_independent_composition():
    inp = layer_inputs_f32s(8, 64, cfg=153, scale=(1.1, 0.9, 1.3))
    o = oracle.pre_f32s(inp.res, inp.hc_fn, inp.hc_scale, inp.hc_base, post_mult=2.0)
    r = inp.res.astype(np.float64)
    T, _, H = r.shape
    flat = r.reshape(T, HC * H)
    rstd = 1.0 / np.sqrt((flat * flat).sum(axis=1) / (HC * H) + 1e-6)
    m = (flat @ inp.hc_fn.astype(np.float64).T) * rstd[:, None]
    s, b = inp.hc_scale.astype(np.float64), inp.hc_base.astype(np.float64)
    pre = _sig(m[:, 0:4] * s[0] + b[0:4]) + 1e-6
    post = _sig(m[:, 4:8] * s[1] + b[4:8]) * 2.0
    comb = _sk_scaling((m[:, 8:24] * s[2] + b[8:24]).reshape(T, 4, 4), 20, 1e-6)
    assert np.allclose(o["pre"], pre, atol=1e-13)
    assert np.allclose(o["post"], post, atol=1e-13)
    assert np.allclose(o["comb"], comb, atol=1e-12)
    assert np.allclose(o["y"], np.einsum("ti,tih->th", pre, r), atol=1e-12)


def test_f32_stream_pre_is_scale_invariant_without_eps():
    """With rms_eps = 0 the mixes see res / rms(res) only: scaling the streams by 8 leaves
    pre, post and comb unchanged and scales y by 8."""
    inp = layer_inputs_f32s(4, 32, cfg=154)
    a = oracle.pre_f32s(inp.res, inp.hc_fn, inp.hc_scale, inp.hc_base, rms_eps=0.0)
    b = oracle.pre_f32s(inp.res * np.float32(8), inp.hc_fn, inp.hc_scale, inp.hc_base, rms_eps=0.0)
    for k in ("pre", "post", "comb"):
        assert np.allclose(a[k], b[k], rtol=0, atol=1e-14), k
    assert np.allclose(b["y"], 8 * a["y"], rtol=1e-14, atol=0)


def test_f32_stream_expand_widens_exactly():
    inp = layer_inputs(4, 24, cfg=155)
    s = oracle.expand_f32s(inp.x)
    assert s.dtype == np.float32
    assert np.array_equal(s, np.repeat(bf16_bits_to_f32(inp.x)[:, None, :], HC, axis=1))
    assert np.array_equal(oracle.round_bf16(oracle.head_mean_f32s(s)), inp.x)
