"""GPU parity at the size limits: the token chunking of the projection's partial sums
(a batch whose partial sums pass 2^31 bytes is processed in chunks: in the pre-map, in
the reverse's recompute and in the post-map fused with the next projection) and the
largest accepted hidden size.
Sampled tokens against the fp64 oracle, with the tolerances of the other parity tests."""
import numpy as np
import pytest

import oracle
from mhc_inputs import HC, MIX, bf16_bits_to_f32, device_normal_bf16, device_normal_f32, normal_f32, post_inputs
from tests._helpers import assert_bf16_close, assert_f32_close, bits_of, f32_of, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PRE_MAX_H = 1 << 21


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


def _bits_rows(t, rows):
    return bits_of(t[torch.as_tensor(rows, device=t.device)])


def _check_pre(res_rows, hc_fn, hc_scale, hc_base, y, post, comb, what):
    ref = oracle.pre(res_rows, hc_fn, hc_scale, hc_base)
    assert_f32_close(post, ref["post"], what + " post")
    assert_f32_close(comb, ref["comb"], what + " comb")
    assert_bf16_close(y, ref["y"], what + " y")


def test_pre_token_chunking():
    """H = 8: one 128-wide slice, 6400 bytes of partial sums per 64-token tile, so the
    first chunk ends after floor(2^31 / 6400) tiles; T runs 3000 tokens into a second,
    ragged chunk."""
    mhc = _mhc()
    H = 8
    chunk = (2 ** 31 // (1 * 100 * 64)) * 64
    T = chunk + 3000
    res = device_normal_bf16(0, 600, "res", (T, HC, H))
    hc_fn = normal_f32(0, 600, "hc_fn", (MIX, HC * H), 0.02)
    hc_scale = np.ones(3, np.float32)
    hc_base = normal_f32(0, 600, "hc_base", (MIX,), 0.1)
    y, post, comb = mhc.mhc_pre_fused(res, to_dev_f32(hc_fn), to_dev_f32(hc_scale), to_dev_f32(hc_base))
    torch.cuda.synchronize()
    rows = sorted({0, 1, 63, 64, chunk - 65, chunk - 64, chunk - 1, chunk, chunk + 1, chunk + 63, chunk + 64,
                   chunk + 2999, T // 2, 12345678})
    _check_pre(_bits_rows(res, rows), hc_fn, hc_scale, hc_base, _bits_rows(y, rows),
               f32_of(post[torch.as_tensor(rows, device="cuda")]), f32_of(comb[torch.as_tensor(rows, device="cuda")]),
               f"pre chunked T={T}")


def test_pre_fused_backward_token_chunking():
    """The reverse's recompute keeps 29 fields per record (the 25 of the forward and the
    four <dy, res_i>): at H = 8 that is 7424 bytes per 64-token tile, so the recompute and
    the per-token reverse run in chunks of floor(2^31 / 7424) tiles, and T runs 3000
    tokens into a second, ragged chunk.  A token's d_res depends on its own inputs only,
    so sampled rows are checked against the oracle run on those rows alone (the sums
    over tokens are covered by the smaller parity tests)."""
    mhc = _mhc()
    H = 8
    chunk = (2 ** 31 // (1 * 29 * 64 * 4)) * 64
    T = chunk + 3000
    res = device_normal_bf16(0, 620, "res", (T, HC, H))
    dy = device_normal_bf16(0, 620, "dy", (T, H))
    d_post = device_normal_f32(0, 620, "d_post", (T, HC))
    d_comb = device_normal_f32(0, 620, "d_comb", (T, HC, HC))
    hc_fn = normal_f32(0, 620, "hc_fn", (MIX, HC * H), 0.02)
    hc_scale = np.ones(3, np.float32)
    hc_base = normal_f32(0, 620, "hc_base", (MIX,), 0.1)
    out = mhc.mhc_pre_fused_backward(dy, d_post, d_comb, res, to_dev_f32(hc_fn), to_dev_f32(hc_scale),
                                     to_dev_f32(hc_base))
    torch.cuda.synchronize()
    rows = sorted({0, 1, 31, 32, 63, 64, chunk - 65, chunk - 33, chunk - 1, chunk, chunk + 1, chunk + 31, chunk + 32,
                   chunk + 2999, T // 2, 12345678})
    idx = torch.as_tensor(rows, device="cuda")
    ref = oracle.pre_backward(_bits_rows(dy, rows), f32_of(d_post[idx]), f32_of(d_comb[idx]), _bits_rows(res, rows),
                              hc_fn, hc_scale, hc_base)
    assert_bf16_close(_bits_rows(out["d_res"], rows), ref["d_res"], f"pre_fused backward chunked T={T} d_res")


def _check_post_project(x_rows, res_rows, post_rows, comb_rows, fn, out_rows, dm_rows, sq_rows, what):
    """out against the oracle's post-map; the dots and sum of squares against the fp64
    projection of the kernel's own out (within 1e-5 of the sum of |term|)."""
    assert_bf16_close(out_rows, oracle.post(x_rows, res_rows, post_rows.astype(np.float64),
                                            comb_rows.astype(np.float64)), what + " out")
    n = out_rows.shape[0]
    o = bf16_bits_to_f32(out_rows).astype(np.float64).reshape(n, -1)
    w = fn.astype(np.float64)
    err = np.abs(dm_rows.astype(np.float64) - o @ w.T)
    assert (err <= 1e-5 * (np.abs(o) @ np.abs(w).T) + 1e-9).all(), what + " dot_mix"
    rsq = (o * o).sum(axis=1)
    assert (np.abs(sq_rows.astype(np.float64) - rsq) <= 1e-5 * rsq + 1e-9).all(), what + " sqrsum"


def test_post_project_token_chunking():
    """The post-map fused with the next projection writes the pre-map's 25-field records:
    at H = 8 the first chunk ends after floor(2^31 / 6400) tiles, and T runs 3000 tokens
    into a second, ragged chunk.  Then the next pre-map from those dots."""
    mhc = _mhc()
    H = 8
    chunk = (2 ** 31 // (1 * 100 * 64)) * 64
    T = chunk + 3000
    x = device_normal_bf16(0, 630, "x", (T, H))
    res = device_normal_bf16(0, 630, "res", (T, HC, H))
    post = device_normal_f32(0, 630, "post", (T, HC))
    comb = device_normal_f32(0, 630, "comb_logits", (T, HC, HC))
    hc_fn = normal_f32(0, 630, "hc_fn", (MIX, HC * H), 0.02)
    hc_scale = np.ones(3, np.float32)
    hc_base = normal_f32(0, 630, "hc_base", (MIX,), 0.1)
    out, dm, sq = mhc.mhc_post_project(x, res, post, comb, to_dev_f32(hc_fn))
    torch.cuda.synchronize()
    rows = sorted({0, 1, 31, 32, 63, 64, chunk - 65, chunk - 64, chunk - 33, chunk - 1, chunk, chunk + 1, chunk + 63,
                   chunk + 64, chunk + 2999, T // 2, 12345678})
    idx = torch.as_tensor(rows, device="cuda")
    res_rows = _bits_rows(res, rows)
    out_rows = _bits_rows(out, rows)
    _check_post_project(_bits_rows(x, rows), res_rows, f32_of(post[idx]), f32_of(comb[idx]), hc_fn, out_rows,
                        f32_of(dm[idx]), f32_of(sq[idx]), f"post_project chunked T={T}")
    y, npost, ncomb = mhc.mhc_pre_from_dots(dm, out, to_dev_f32(hc_scale), to_dev_f32(hc_base), sqrsum=sq)
    torch.cuda.synchronize()
    _check_pre(out_rows, hc_fn, hc_scale, hc_base, _bits_rows(y, rows), f32_of(npost[idx]), f32_of(ncomb[idx]),
               f"pre from post_project chunked T={T}")


@pytest.mark.parametrize("fn", ["pre_fused", "pre_from_dots", "post", "post_project"])
def test_largest_hidden_size(fn):
    """H = 2^21, the pre-map's limit (its 64-token tiles are addressed with 32-bit byte
    offsets), with a ragged T of 3."""
    mhc = _mhc()
    T, H = 3, PRE_MAX_H
    res = device_normal_bf16(0, 610, "res", (T, HC, H))
    rows = list(range(T))
    if fn == "pre_fused":
        hc_fn = normal_f32(0, 610, "hc_fn", (MIX, HC * H), 0.02)
        hc_scale = np.ones(3, np.float32)
        hc_base = normal_f32(0, 610, "hc_base", (MIX,), 0.1)
        y, post, comb = mhc.mhc_pre_fused(res, to_dev_f32(hc_fn), to_dev_f32(hc_scale), to_dev_f32(hc_base))
        torch.cuda.synchronize()
        _check_pre(bits_of(res), hc_fn, hc_scale, hc_base, bits_of(y), f32_of(post), f32_of(comb), "pre H=2^21")
    elif fn == "pre_from_dots":
        dm = normal_f32(0, 610, "logits", (T, MIX), 5.0)
        hc_scale = np.ones(3, np.float32)
        hc_base = normal_f32(0, 610, "hc_base", (MIX,), 0.1)
        y, post, comb = mhc.mhc_pre_from_dots(to_dev_f32(dm), res, to_dev_f32(hc_scale), to_dev_f32(hc_base))
        torch.cuda.synchronize()
        ref = oracle.pre_from_dots(dm, bits_of(res), hc_scale, hc_base)
        assert_f32_close(f32_of(post), ref["post"], "pre_from_dots H=2^21 post")
        assert_f32_close(f32_of(comb), ref["comb"], "pre_from_dots H=2^21 comb")
        assert_bf16_close(bits_of(y), ref["y"], "pre_from_dots H=2^21 y")
    elif fn == "post_project":
        x = device_normal_bf16(0, 610, "x", (T, H))
        g = np.random.default_rng(611)
        post = g.uniform(0, 2, (T, HC)).astype(np.float32)
        comb = oracle.sinkhorn(g.standard_normal((T, HC, HC)), 20, 1e-6).astype(np.float32)
        hc_fn = normal_f32(0, 610, "hc_fn", (MIX, HC * H), 0.02)
        hc_scale = np.ones(3, np.float32)
        hc_base = normal_f32(0, 610, "hc_base", (MIX,), 0.1)
        out, dm, sq = mhc.mhc_post_project(x, res, to_dev_f32(post), to_dev_f32(comb), to_dev_f32(hc_fn))
        torch.cuda.synchronize()
        ob = bits_of(out)
        _check_post_project(bits_of(x), bits_of(res), post, comb, hc_fn, ob, f32_of(dm), f32_of(sq),
                            "post_project H=2^21")
        y, npost, ncomb = mhc.mhc_pre_from_dots(dm, out, to_dev_f32(hc_scale), to_dev_f32(hc_base), sqrsum=sq)
        torch.cuda.synchronize()
        _check_pre(ob, hc_fn, hc_scale, hc_base, bits_of(y), f32_of(npost), f32_of(ncomb),
                   "pre from post_project H=2^21")
    else:
        x = device_normal_bf16(0, 610, "x", (T, H))
        g = np.random.default_rng(610)
        post = g.uniform(0, 2, (T, HC)).astype(np.float32)
        comb = oracle.sinkhorn(g.standard_normal((T, HC, HC)), 20, 1e-6).astype(np.float32)
        out = mhc.mhc_post(x, res, to_dev_f32(post), to_dev_f32(comb))
        torch.cuda.synchronize()
        ref = oracle.post(bits_of(x), bits_of(res), post.astype(np.float64), comb.astype(np.float64))
        assert_bf16_close(bits_of(out), ref, "post H=2^21")
