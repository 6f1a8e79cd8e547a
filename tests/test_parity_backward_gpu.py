"""GPU parity of the reverse-mode entry points against the fp64 CPU oracle.

Tolerances (derived from the fp32 arithmetic of the kernels):
  * Sinkhorn reverse mode: |err| <= 1e-5 * max|grad| of the matrix.  An fp32
    emulation of the same steps stays below 7e-7 * max|grad| up to 100 iterations.
  * d_x, d_res: the bf16 output tolerance 2^-7 |ref| + 1e-3 (one fp32 sum of four
    products, then one rounding to bf16).
  * d_post, d_comb: |err| <= 1e-5 * sum_h |a_h b_h| + 1e-6: a sum of H products
    in fp32 with at most a few dozen roundings on any path of the reduction tree
    (about 40 * 2^-24 = 2.4e-6 relative to sum |a b|).
  * pre-map reverse mode: each fp32 quantity within 1e-5 of its own magnitude, plus
    the worst case of its one long reduction, d_pre_i = sum_h dy res_i (2.5e-6 *
    sum_h |dy res_i|), carried through the chain (see _pre_bwd_tolerances).
"""
import numpy as np
import pytest

import oracle
from mhc_inputs import (HC, MIX, bf16_bits_to_f32, external_dots, layer_inputs, post_grad, post_inputs, pre_grads,
                        sinkhorn_grad, sinkhorn_logits)
from tests._helpers import assert_bf16_close, bits_of, f32_of, sample_tokens, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SK_RTOL = 1e-5
SUM_RTOL = 1e-5
SUM_ATOL = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connection_amd as mhc
    mhc.lib()
    yield


def _mhc():
    import mhc_hyper_connection_amd as mhc
    return mhc


def _assert_sk_close(got, ref, grad, what):
    n = grad.shape[0]
    err = np.abs(np.asarray(got, np.float64) - ref).reshape(n, -1).max(-1)
    tol = SK_RTOL * np.abs(grad).reshape(n, -1).max(-1)
    bad = ~(err <= tol)
    if bad.any():
        i = int(np.argmax(bad))
        raise AssertionError(f"{what}: {int(bad.sum())} of {n} matrices outside tolerance; first {i}: "
                             f"err {err[i]:.3e} tol {tol[i]:.3e}")


def _assert_sum_close(got, ref, scale, what):
    err = np.abs(np.asarray(got, np.float64) - ref)
    tol = SUM_RTOL * scale + SUM_ATOL
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first at {idx.tolist()}; "
                             f"max err/scale {(err / np.maximum(scale, 1e-30)).max():.3e}")


# ----------------------------------------------------------------------------- Sinkhorn reverse mode

@pytest.mark.parametrize("n,iters", [(1, 1), (3, 20), (4099, 1), (4099, 3), (4099, 20), (777, 100), (65, 255)])
def test_sinkhorn_backward_matches_oracle(n, iters):
    mhc = _mhc()
    lg = sinkhorn_logits(n, cfg=40 + iters)
    g = sinkhorn_grad(n, cfg=40 + iters)
    got = mhc.mhc_sinkhorn_backward(to_dev_f32(g), to_dev_f32(lg), num_iters=iters, eps=1e-6)
    torch.cuda.synchronize()
    ref = oracle.sinkhorn_backward(g.astype(np.float64), lg.astype(np.float64), iters, 1e-6)
    _assert_sk_close(f32_of(got), ref, g, f"sinkhorn backward n={n} iters={iters}")


def test_sinkhorn_backward_full_size_sampled():
    """2^20 matrices at 20 iterations: sampled matrices against the oracle, and the
    zero row sums of a row-softmax gradient on every matrix."""
    mhc = _mhc()
    n = 1 << 20
    lg = sinkhorn_logits(n)
    g = sinkhorn_grad(n)
    got = f32_of(mhc.mhc_sinkhorn_backward(to_dev_f32(g), to_dev_f32(lg), num_iters=20, eps=1e-6))
    pick = np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n),
                                     np.random.default_rng(5).integers(0, n, 20000)]))
    ref = oracle.sinkhorn_backward(g[pick].astype(np.float64), lg[pick].astype(np.float64), 20, 1e-6)
    _assert_sk_close(got[pick], ref, g[pick], "sinkhorn backward 2^20 sampled")
    rows = np.abs(got.astype(np.float64).sum(-1))
    assert rows.max() <= 1e-5 * np.abs(g).max(), rows.max()


def test_sinkhorn_backward_in_place_and_deterministic():
    mhc = _mhc()
    n = 1000
    lg = sinkhorn_logits(n, cfg=47)
    g = sinkhorn_grad(n, cfg=47)
    ref = f32_of(mhc.mhc_sinkhorn_backward(to_dev_f32(g), to_dev_f32(lg), num_iters=20))
    again = f32_of(mhc.mhc_sinkhorn_backward(to_dev_f32(g), to_dev_f32(lg), num_iters=20))
    assert np.array_equal(ref, again)
    gd = to_dev_f32(g)
    mhc.mhc_sinkhorn_backward(gd, to_dev_f32(lg), num_iters=20, d_logits=gd)
    ld = to_dev_f32(lg)
    mhc.mhc_sinkhorn_backward(to_dev_f32(g), ld, num_iters=20, d_logits=ld)
    torch.cuda.synchronize()
    assert np.array_equal(f32_of(gd), ref)
    assert np.array_equal(f32_of(ld), ref)
    empty = torch.empty(0, 4, 4, device="cuda")
    assert mhc.mhc_sinkhorn_backward(empty, empty).numel() == 0


# ----------------------------------------------------------------------------- post-map reverse mode

BWD_SHAPES = [(16, 256), (5, 64), (7, 127), (3, 1001), (9, 1536), (6, 2048), (37, 4096), (21, 7168), (4, 8192),
              (3, 16392), (1, 1), (2, 8), (3, 520), (300, 1000), (65, 2056)]


def _post_bwd_case(T, H, cfg):
    res, x, post, comb_logits = post_inputs(T, H, cfg=cfg)
    comb = oracle.sinkhorn(comb_logits, 20, 1e-6).astype(np.float32)
    d_out = post_grad(T, H, cfg=cfg)
    return d_out, x, res, post, comb


def _check_post_bwd(got, case, what, tokens=None):
    d_out, x, res, post, comb = case
    if tokens is not None:
        d_out, x, res, post, comb = d_out[tokens], x[tokens], res[tokens], post[tokens], comb[tokens]
        got = tuple(g[tokens] for g in got)
    d_x, d_res, d_post, d_comb = got
    r_x, r_res, r_post, r_comb = oracle.post_backward(d_out, x, res, post.astype(np.float64),
                                                      comb.astype(np.float64))
    assert_bf16_close(d_x, r_x, what + " d_x")
    assert_bf16_close(d_res, r_res, what + " d_res")
    g = np.abs(bf16_bits_to_f32(d_out).astype(np.float64))
    xa = np.abs(bf16_bits_to_f32(x).astype(np.float64))
    ra = np.abs(bf16_bits_to_f32(res).astype(np.float64))
    _assert_sum_close(d_post, r_post, np.einsum("tnh,th->tn", g, xa), what + " d_post")
    _assert_sum_close(d_comb, r_comb, np.einsum("toh,tnh->ton", ra, g), what + " d_comb")


def _run_post_bwd(case, **kw):
    mhc = _mhc()
    d_out, x, res, post, comb = case
    out = mhc.mhc_post_backward(to_dev_bf16(d_out), to_dev_bf16(x), to_dev_bf16(res), to_dev_f32(post),
                                to_dev_f32(comb), **kw)
    torch.cuda.synchronize()
    return bits_of(out[0]), bits_of(out[1]), f32_of(out[2]), f32_of(out[3])


@pytest.mark.parametrize("T,H", BWD_SHAPES)
def test_post_backward_matches_oracle(T, H):
    case = _post_bwd_case(T, H, cfg=300 + H % 89)
    _check_post_bwd(_run_post_bwd(case), case, f"post backward T={T} H={H}")


def test_post_backward_full_size_h7168_sampled():
    """T=8192, H=7168: sampled tokens (tile edges, ends, random) against the oracle."""
    T, H = 8192, 7168
    case = _post_bwd_case(T, H, cfg=3)
    got = _run_post_bwd(case)
    _check_post_bwd(got, case, "post backward 8192x7168", tokens=sample_tokens(T, 48))


def test_post_backward_in_place_and_post_shape():
    mhc = _mhc()
    T, H = 33, 4096
    case = _post_bwd_case(T, H, cfg=311)
    d_out, x, res, post, comb = case
    ref = _run_post_bwd(case)
    g = to_dev_bf16(d_out)
    d_x, d_res, d_post, d_comb = mhc.mhc_post_backward(g, to_dev_bf16(x), to_dev_bf16(res),
                                                       to_dev_f32(post).reshape(T, HC, 1), to_dev_f32(comb), d_res=g)
    torch.cuda.synchronize()
    assert d_res.data_ptr() == g.data_ptr()
    assert tuple(d_post.shape) == (T, HC, 1)
    assert np.array_equal(bits_of(d_x), ref[0])
    assert np.array_equal(bits_of(g), ref[1])
    assert np.array_equal(f32_of(d_post).reshape(T, HC), ref[2])
    assert np.array_equal(f32_of(d_comb), ref[3])


def test_post_backward_deterministic_and_empty():
    mhc = _mhc()
    case = _post_bwd_case(100, 7168, cfg=312)
    a = _run_post_bwd(case)
    b = _run_post_bwd(case)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    z = torch.empty(0, HC, 64, dtype=torch.bfloat16, device="cuda")
    out = mhc.mhc_post_backward(z, torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"), z,
                                torch.empty(0, HC, device="cuda"), torch.empty(0, HC, HC, device="cuda"))
    assert all(o.numel() == 0 for o in out)


# ----------------------------------------------------------------------------- pre-map reverse mode (external dots)

def _pre_bwd_case(T, H, splits, supplied, cfg):
    inp = layer_inputs(T, H, cfg=cfg, scale=(0.9, 1.1, 1.3))
    dm = external_dots(T, H, cfg=cfg, splits=splits)
    sq = None
    if supplied:
        full = (bf16_bits_to_f32(inp.res).astype(np.float64) ** 2).sum(axis=(1, 2))
        sq = np.repeat((full / splits)[None, :], splits, axis=0).astype(np.float32)
    dy, d_post, d_comb = pre_grads(T, H, cfg=cfg)
    return inp, dm, sq, dy, d_post, d_comb


def _pre_bwd_tolerances(inp, dm, sq, dy, d_post, d_comb, k, ref, post_mult=1.0):
    """Per-element tolerances for the outputs of the pre-map reverse mode (fp32 arithmetic).

    Besides 1e-5 of each value: the worst case of the d_pre reduction, and the sigmoid
    derivative sigma (1 - sigma) formed from an fp32 sigma, whose absolute error is a few
    ulp of 1 (bounded by 1e-6 here), times the gradient it multiplies."""
    res = bf16_bits_to_f32(inp.res).astype(np.float64)
    dyv = bf16_bits_to_f32(dy).astype(np.float64)
    d = dm.astype(np.float64).sum(axis=0)
    S = (res ** 2).sum(axis=(1, 2)) if sq is None else sq.astype(np.float64).sum(axis=0)
    rstd = 1 / np.sqrt(S / k + 1e-6)
    s = inp.hc_scale.astype(np.float64)
    sg = np.concatenate([np.full(4, s[0]), np.full(4, s[1]), np.full(16, s[2])])
    A = np.einsum("th,tih->ti", np.abs(dyv), np.abs(res))       # sum_h |dy res_i|
    rel = 1e-5
    tol_dot = rel * np.abs(ref["d_dot"])
    tol_dot[:, :4] += (2.5e-6 * 0.25 + 1e-6) * rstd[:, None] * abs(s[0]) * A
    tol_dot[:, 4:8] += 1e-6 * rstd[:, None] * abs(s[1]) * abs(post_mult) * np.abs(d_post) + 1e-7
    tol_dot[:, 8:] += rel * abs(s[2]) * rstd[:, None] * np.abs(d_comb).reshape(-1, 16).max(axis=1)[:, None]
    tol_dS = rstd ** 2 / (2 * k) * ((rel * np.abs(ref["d_dot"]) + tol_dot) * np.abs(d)).sum(axis=1)
    tol_dz = tol_dot / (np.abs(sg)[None, :] * rstd[:, None])
    dz = ref["d_dot"] / (sg[None, :] * rstd[:, None])
    m = d * rstd[:, None]
    tol_base = (tol_dz + rel * np.abs(dz)).sum(axis=0)
    tz = (tol_dz * np.abs(m) + rel * np.abs(dz * m))
    tol_scale = np.array([tz[:, :4].sum(), tz[:, 4:8].sum(), tz[:, 8:].sum()])
    extra_res = (2 * tol_dS)[:, None, None] * np.abs(res) if sq is None else 0.0
    return dict(d_dot=tol_dot, d_sqrsum=rel * np.abs(ref["d_sqrsum"] if ref["d_sqrsum"] is not None else 0) + tol_dS,
                d_hc_base=tol_base, d_hc_scale=tol_scale, d_res_extra=extra_res)


def _assert_within(got, ref, tol, what):
    err = np.abs(np.asarray(got, np.float64) - ref)
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first at {idx.tolist()}; "
                             f"max err/tol {(err / np.maximum(tol, 1e-30)).max():.3e}")


def _run_pre_bwd(case, k=None, **kw):
    mhc = _mhc()
    inp, dm, sq, dy, d_post, d_comb = case
    T, _, H = inp.res.shape
    dmd = to_dev_f32(dm if dm.shape[0] > 1 else dm[0])
    out = mhc.mhc_pre_from_dots_backward(to_dev_bf16(dy), to_dev_f32(d_post), to_dev_f32(d_comb), dmd,
                                         to_dev_bf16(inp.res), to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base),
                                         sqrsum=None if sq is None else to_dev_f32(sq), k=k, **kw)
    torch.cuda.synchronize()
    return dict(d_res=bits_of(out["d_res"]), d_dot=f32_of(out["d_dot"]),
                d_sqrsum=None if out["d_sqrsum"] is None else f32_of(out["d_sqrsum"]),
                d_hc_scale=f32_of(out["d_hc_scale"]), d_hc_base=f32_of(out["d_hc_base"]))


def _check_pre_bwd(got, case, what, k=None, tokens=None):
    inp, dm, sq, dy, d_post, d_comb = case
    T, _, H = inp.res.shape
    kk = float(4 * H) if k is None else k
    ref = oracle.pre_from_dots_backward(dy, d_post, d_comb, dm.astype(np.float64).sum(axis=0), inp.res,
                                        inp.hc_scale, inp.hc_base,
                                        sqrsum=None if sq is None else sq.astype(np.float64).sum(axis=0), k=kk)
    tol = _pre_bwd_tolerances(inp, dm, sq, dy, d_post, d_comb, kk, ref)
    _assert_within(got["d_hc_base"], ref["d_hc_base"], tol["d_hc_base"], what + " d_hc_base")
    _assert_within(got["d_hc_scale"], ref["d_hc_scale"], tol["d_hc_scale"], what + " d_hc_scale")
    sel = slice(None) if tokens is None else tokens
    _assert_within(got["d_dot"][sel], ref["d_dot"][sel], tol["d_dot"][sel], what + " d_dot")
    if sq is not None:
        _assert_within(got["d_sqrsum"][sel], ref["d_sqrsum"][sel], tol["d_sqrsum"][sel], what + " d_sqrsum")
    gres = bf16_bits_to_f32(got["d_res"][sel]).astype(np.float64)
    rres = ref["d_res"][sel]
    extra = tol["d_res_extra"][sel] if sq is None else 0.0
    _assert_within(gres, rres, 2.0 ** -7 * np.abs(rres) + 1e-3 + extra, what + " d_res")


PRE_BWD_SHAPES = [(16, 256, 1, False), (5, 64, 1, True), (7, 127, 1, False), (3, 1001, 2, True),
                  (37, 4096, 1, False), (21, 7168, 3, False), (9, 16392, 1, False), (1, 1, 1, False),
                  (300, 1000, 1, True), (65, 2056, 4, False), (70, 96, 2, True)]


@pytest.mark.parametrize("T,H,splits,supplied", PRE_BWD_SHAPES)
def test_pre_from_dots_backward_matches_oracle(T, H, splits, supplied):
    case = _pre_bwd_case(T, H, splits, supplied, cfg=400 + H % 83)
    _check_pre_bwd(_run_pre_bwd(case), case, f"pre backward T={T} H={H} S={splits} sq={supplied}")


@pytest.mark.parametrize("iters", [1, 3, 100])
def test_pre_from_dots_backward_iterations_and_k(iters):
    case = _pre_bwd_case(33, 512, 1, True, cfg=420 + iters)
    got = _run_pre_bwd(case, k=700.0, num_iters=iters)
    inp, dm, sq, dy, d_post, d_comb = case
    ref = oracle.pre_from_dots_backward(dy, d_post, d_comb, dm[0].astype(np.float64), inp.res, inp.hc_scale,
                                        inp.hc_base, sqrsum=sq[0].astype(np.float64), k=700.0, num_iters=iters)
    tol = _pre_bwd_tolerances(inp, dm, sq, dy, d_post, d_comb, 700.0, ref)
    _assert_within(got["d_dot"], ref["d_dot"], tol["d_dot"], f"d_dot iters={iters}")
    _assert_within(got["d_hc_base"], ref["d_hc_base"], tol["d_hc_base"], f"d_hc_base iters={iters}")


def test_pre_from_dots_backward_full_size_h7168_sampled():
    """T=8192, H=7168: the token sums against the oracle over every token; the per-token
    outputs on sampled tokens."""
    case = _pre_bwd_case(8192, 7168, 1, False, cfg=3)
    got = _run_pre_bwd(case)
    _check_pre_bwd(got, case, "pre backward 8192x7168", tokens=sample_tokens(8192, 48))


def test_pre_from_dots_backward_in_place_deterministic_and_empty():
    mhc = _mhc()
    case = _pre_bwd_case(40, 7168, 1, False, cfg=430)
    a = _run_pre_bwd(case)
    b = _run_pre_bwd(case)
    for key in a:
        if a[key] is not None:
            assert np.array_equal(a[key], b[key]), key
    inp, dm, sq, dy, d_post, d_comb = case
    r = to_dev_bf16(inp.res)
    out = mhc.mhc_pre_from_dots_backward(to_dev_bf16(dy), to_dev_f32(d_post), to_dev_f32(d_comb), to_dev_f32(dm[0]),
                                         r, to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base), d_res=r)
    torch.cuda.synchronize()
    assert out["d_res"].data_ptr() == r.data_ptr()
    assert np.array_equal(bits_of(r), a["d_res"])
    z = torch.empty(0, HC, 64, dtype=torch.bfloat16, device="cuda")
    e = mhc.mhc_pre_from_dots_backward(torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"),
                                       torch.empty(0, HC, device="cuda"), torch.empty(0, HC, HC, device="cuda"),
                                       torch.empty(0, MIX, device="cuda"), z, to_dev_f32(inp.hc_scale),
                                       to_dev_f32(inp.hc_base))
    torch.cuda.synchronize()
    assert not f32_of(e["d_hc_base"]).any() and not f32_of(e["d_hc_scale"]).any()


# ----------------------------------------------------------------------------- whole pre-map reverse mode

def _full_pre_bwd_check(inp, dy, d_post, d_comb, got, what, tokens=None):
    """got: dict of host arrays from mhc_pre_fused_backward.  The oracle's reverse mode on the
    (sampled) tokens; d_hc_fn, d_hc_scale and d_hc_base need every token, so `tokens` may only
    be given for the per-token outputs when the sums are checked separately."""
    T, _, H = inp.res.shape
    K = HC * H
    kw = dict()
    fwd = oracle.pre(inp.res, inp.hc_fn, inp.hc_scale, inp.hc_base)
    dm = fwd["dot"][None].astype(np.float64)
    ref_fd = oracle.pre_from_dots_backward(dy, d_post, d_comb, fwd["dot"], inp.res, inp.hc_scale, inp.hc_base,
                                           k=float(K))
    tol = _pre_bwd_tolerances(inp, dm, None, dy, d_post, d_comb, float(K), ref_fd)
    ref = oracle.pre_backward(dy, d_post, d_comb, inp.res, inp.hc_fn, inp.hc_scale, inp.hc_base)
    W = np.abs(inp.hc_fn.astype(np.float64))
    dd_err = tol["d_dot"] + 2.0 ** -15 * np.abs(ref_fd["d_dot"])          # d_dot and its hi/lo halves
    resv = np.abs(bf16_bits_to_f32(inp.res).astype(np.float64)).reshape(T, K)
    tol_fn = dd_err.T @ resv + 1e-5 * (np.abs(ref_fd["d_dot"]).T @ resv) + 1e-6
    _assert_within(got["d_hc_fn"], ref["d_hc_fn"], tol_fn, what + " d_hc_fn")
    _assert_within(got["d_hc_base"], ref["d_hc_base"], tol["d_hc_base"], what + " d_hc_base")
    _assert_within(got["d_hc_scale"], ref["d_hc_scale"], tol["d_hc_scale"], what + " d_hc_scale")
    sel = slice(None) if tokens is None else tokens
    proj_tol = (dd_err[sel] @ W).reshape(-1, HC, H) + 2.0 ** -15 * (np.abs(ref_fd["d_dot"][sel]) @ W).reshape(-1, HC, H)
    rres = ref["d_res"][sel]
    gres = bf16_bits_to_f32(got["d_res"][sel]).astype(np.float64)
    _assert_within(gres, rres, 2.0 ** -7 * np.abs(rres) + 1e-3 + tol["d_res_extra"][sel] + proj_tol, what + " d_res")


def _run_full_pre_bwd(inp, dy, d_post, d_comb, **kw):
    mhc = _mhc()
    out = mhc.mhc_pre_fused_backward(to_dev_bf16(dy), to_dev_f32(d_post), to_dev_f32(d_comb), to_dev_bf16(inp.res),
                                     to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base), **kw)
    torch.cuda.synchronize()
    return dict(d_res=bits_of(out["d_res"]), d_hc_fn=f32_of(out["d_hc_fn"]), d_hc_scale=f32_of(out["d_hc_scale"]),
                d_hc_base=f32_of(out["d_hc_base"]))


@pytest.mark.parametrize("T,H", [(16, 256), (5, 64), (33, 1000), (70, 96), (130, 4096), (21, 7168), (300, 1024),
                                 (1, 8), (65, 2056)])
def test_pre_fused_backward_matches_oracle(T, H):
    inp = layer_inputs(T, H, cfg=800 + H % 79, scale=(0.9, 1.1, 1.3))
    dy, d_post, d_comb = pre_grads(T, H, cfg=800 + H % 79)
    got = _run_full_pre_bwd(inp, dy, d_post, d_comb)
    _full_pre_bwd_check(inp, dy, d_post, d_comb, got, f"pre_fused backward T={T} H={H}")


def test_pre_fused_backward_many_tokens_h4096():
    """T=2048, H=4096: several token ranges per column block, the d_hc_fn sums over all of them."""
    inp = layer_inputs(2048, 4096, cfg=820)
    dy, d_post, d_comb = pre_grads(2048, 4096, cfg=820)
    got = _run_full_pre_bwd(inp, dy, d_post, d_comb)
    _full_pre_bwd_check(inp, dy, d_post, d_comb, got, "pre_fused backward 2048x4096")


def test_pre_fused_backward_in_place_deterministic_and_empty():
    mhc = _mhc()
    inp = layer_inputs(40, 1024, cfg=830)
    dy, d_post, d_comb = pre_grads(40, 1024, cfg=830)
    a = _run_full_pre_bwd(inp, dy, d_post, d_comb)
    b = _run_full_pre_bwd(inp, dy, d_post, d_comb)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    r = to_dev_bf16(inp.res)
    out = mhc.mhc_pre_fused_backward(to_dev_bf16(dy), to_dev_f32(d_post), to_dev_f32(d_comb), r,
                                     to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base), d_res=r)
    torch.cuda.synchronize()
    assert out["d_res"].data_ptr() == r.data_ptr() and np.array_equal(bits_of(r), a["d_res"])
    assert np.array_equal(f32_of(out["d_hc_fn"]), a["d_hc_fn"])
    z = torch.empty(0, HC, 64, dtype=torch.bfloat16, device="cuda")
    e = mhc.mhc_pre_fused_backward(torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"),
                                   torch.empty(0, HC, device="cuda"), torch.empty(0, HC, HC, device="cuda"), z,
                                   torch.ones(MIX, HC * 64, device="cuda"), to_dev_f32(inp.hc_scale),
                                   to_dev_f32(inp.hc_base))
    torch.cuda.synchronize()
    assert not f32_of(e["d_hc_fn"]).any() and not f32_of(e["d_hc_base"]).any() and not f32_of(e["d_hc_scale"]).any()
