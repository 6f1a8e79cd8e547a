"""GPU parity of the reverse-mode entry points against the fp64 CPU oracle.

Tolerances (derived from the fp32 arithmetic of the kernels):
  * Sinkhorn reverse mode: |err| <= 1e-5 * max|grad| of the matrix.  An fp32
    emulation of the same steps stays below 7e-7 * max|grad| up to 100 iterations.
  * d_x, d_res: the bf16 output tolerance 2^-7 |ref| + 1e-3 (one fp32 sum of four
    products, then one rounding to bf16).
  * d_post, d_comb: |err| <= 1e-5 * sum_h |a_h b_h| + 1e-6: a sum of H products
    in fp32 with at most a few dozen roundings on any path of the reduction tree
    (about 40 * 2^-24 = 2.4e-6 relative to sum |a b|).
"""
import numpy as np
import pytest

import oracle
from mhc_inputs import (HC, bf16_bits_to_f32, post_grad, post_inputs, sinkhorn_grad, sinkhorn_logits)
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
