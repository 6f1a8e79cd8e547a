"""GPU parity across the launch chunks of the token-parallel kernels.

A call on more tokens (or Sinkhorn matrices) than one launch may cover is split into
launches over token chunks (mhc_launch_plan reports the split: 2^24 tokens per launch for
the one-wave-per-token kernels at small H, about 2^23 for the 256-thread ones).  Each case
runs T a few tokens past the first chunk, at H = 8 to keep memory at a few GB, and checks
the tokens on both sides of every chunk edge and at the end: the forward entry points
against the fp64 oracle, the reverse ones bit for bit against a call on the sampled
tokens alone (a size whose parity with the oracle the other reverse-mode tests cover;
every output checked here depends on its own token only)."""
import numpy as np
import pytest

import oracle
from mhc_inputs import HC, MIX, device_normal_bf16, device_normal_f32, normal_f32
from tests._helpers import assert_bf16_close, assert_f32_close, bits_of, f32_of, to_dev_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

H = 8
TAIL = 37


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connection_amd as mhc
    mhc.lib()
    yield
    torch.cuda.empty_cache()


def _mhc():
    import mhc_hyper_connection_amd as mhc
    return mhc


def _plan(entry, vec8=True):
    """(T, rows): T runs TAIL tokens past the first chunk edge; rows straddle every edge."""
    p = _mhc().launch_plan(entry, 1 << 30, H, vec8)
    per = p["tokens_per_launch"]
    T = per + TAIL
    assert _mhc().launch_plan(entry, T, H, vec8)["launches"] == 2
    rows = sorted({0, 1, per - 2, per - 1, per, per + 1, T - 1})
    print(f"chunk case {entry}: T={T} edge={per}", flush=True)
    return T, rows


def _at(t, rows):
    return t[torch.as_tensor(rows, device=t.device)]


def test_post_chunks():
    mhc = _mhc()
    T, rows = _plan("post")
    x = device_normal_bf16(0, 900, "x", (T, H))
    res = device_normal_bf16(0, 900, "res", (T, HC, H))
    post = device_normal_f32(0, 900, "post", (T, HC))
    comb = device_normal_f32(0, 900, "comb_logits", (T, HC, HC), std=0.5)
    out = mhc.mhc_post(x, res, post, comb)
    torch.cuda.synchronize()
    ref = oracle.post(bits_of(_at(x, rows)), bits_of(_at(res, rows)), f32_of(_at(post, rows)).astype(np.float64),
                      f32_of(_at(comb, rows)).astype(np.float64))
    assert_bf16_close(bits_of(_at(out, rows)), ref, f"post T={T}")


def test_expand_and_head_mean_chunks():
    mhc = _mhc()
    T, rows = _plan("expand")
    assert _plan("head_mean")[0] == T
    hidden = device_normal_bf16(0, 901, "x", (T, H))
    streams = mhc.mhc_expand(hidden)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(_at(streams, rows)), oracle.expand(bits_of(_at(hidden, rows))))
    del streams
    res = device_normal_bf16(0, 901, "res", (T, HC, H))
    y = mhc.mhc_head_mean(res)
    torch.cuda.synchronize()
    assert_bf16_close(bits_of(_at(y, rows)), oracle.head_mean(bits_of(_at(res, rows))), f"head_mean T={T}")


def _pre_inputs(T, cfg):
    res = device_normal_bf16(0, cfg, "res", (T, HC, H))
    hc_scale = np.array([0.9, 1.1, 1.3], np.float32)
    hc_base = normal_f32(0, cfg, "hc_base", (MIX,), 0.1)
    return res, hc_scale, hc_base


def test_pre_from_dots_collapse_chunks():
    """One split with the sum of squares supplied, 16-byte rows: the collapse kernel's chunks."""
    mhc = _mhc()
    T, rows = _plan("collapse")
    res, hc_scale, hc_base = _pre_inputs(T, 902)
    dm = device_normal_f32(0, 902, "dots", (T, MIX), std=3.0)
    sq = (device_normal_f32(0, 902, "logits", (T,), std=0.2).abs() + 1.0) * (HC * H)
    y, post, comb, pre = mhc.mhc_pre_from_dots(dm, res, to_dev_f32(hc_scale), to_dev_f32(hc_base), sqrsum=sq,
                                               return_pre=True)
    torch.cuda.synchronize()
    ref = oracle.pre_from_dots(f32_of(_at(dm, rows)), bits_of(_at(res, rows)), hc_scale, hc_base,
                               sqrsum=f32_of(_at(sq, rows)))
    assert_f32_close(f32_of(_at(post, rows)), ref["post"], "collapse chunks post")
    assert_f32_close(f32_of(_at(comb, rows)), ref["comb"], "collapse chunks comb")
    assert_f32_close(f32_of(_at(pre, rows)), ref["pre"], "collapse chunks pre")
    assert_bf16_close(bits_of(_at(y, rows)), ref["y"], "collapse chunks y")


def test_pre_from_dots_two_splits_chunks():
    """Two splits, the sum of squares computed from the streams: the per-token kernel's chunks
    (its split arrays keep the whole call's token stride)."""
    mhc = _mhc()
    T, rows = _plan("pre_from_dots")
    res, hc_scale, hc_base = _pre_inputs(T, 903)
    dm = device_normal_f32(0, 903, "dots", (2, T, MIX), std=2.0)
    y, post, comb = mhc.mhc_pre_from_dots(dm, res, to_dev_f32(hc_scale), to_dev_f32(hc_base))
    torch.cuda.synchronize()
    idx = torch.as_tensor(rows, device="cuda")
    ref = oracle.pre_from_dots(f32_of(dm[:, idx]), bits_of(_at(res, rows)), hc_scale, hc_base)
    assert_f32_close(f32_of(_at(post, rows)), ref["post"], "dots chunks post")
    assert_f32_close(f32_of(_at(comb, rows)), ref["comb"], "dots chunks comb")
    assert_bf16_close(bits_of(_at(y, rows)), ref["y"], "dots chunks y")


def test_sinkhorn_chunks():
    mhc = _mhc()
    n, rows = _plan("sinkhorn")
    logits = device_normal_f32(0, 904, "logits", (n, HC, HC), std=2.0)
    out = mhc.mhc_sinkhorn(logits)
    torch.cuda.synchronize()
    ref = oracle.sinkhorn(f32_of(_at(logits, rows)).astype(np.float64), 20, 1e-6)
    assert_f32_close(f32_of(_at(out, rows)), ref, f"sinkhorn n={n}")


def test_sinkhorn_backward_chunks():
    mhc = _mhc()
    n, rows = _plan("sinkhorn_backward")
    logits = device_normal_f32(0, 905, "logits", (n, HC, HC), std=2.0)
    grad = device_normal_f32(0, 905, "grad", (n, HC, HC))
    d = mhc.mhc_sinkhorn_backward(grad, logits)
    torch.cuda.synchronize()
    small = mhc.mhc_sinkhorn_backward(_at(grad, rows).contiguous(), _at(logits, rows).contiguous())
    torch.cuda.synchronize()
    assert np.array_equal(f32_of(_at(d, rows)), f32_of(small))


def test_post_backward_chunks():
    mhc = _mhc()
    T, rows = _plan("post_backward")
    d_out = device_normal_bf16(0, 906, "d_out", (T, HC, H))
    x = device_normal_bf16(0, 906, "x", (T, H))
    res = device_normal_bf16(0, 906, "res", (T, HC, H))
    post = device_normal_f32(0, 906, "post", (T, HC))
    comb = device_normal_f32(0, 906, "comb_logits", (T, HC, HC), std=0.5)
    big = mhc.mhc_post_backward(d_out, x, res, post, comb)
    torch.cuda.synchronize()
    big = [(bits_of(_at(g, rows)) if g.dtype == torch.bfloat16 else f32_of(_at(g, rows))) for g in big]
    small = mhc.mhc_post_backward(*[_at(t, rows).contiguous() for t in (d_out, x, res, post, comb)])
    torch.cuda.synchronize()
    small = [(bits_of(g) if g.dtype == torch.bfloat16 else f32_of(g)) for g in small]
    for a, b, name in zip(big, small, ("d_x", "d_res", "d_post", "d_comb")):
        assert np.array_equal(a, b), name


def test_pre_from_dots_backward_chunks():
    mhc = _mhc()
    T, rows = _plan("pre_from_dots_backward")
    res, hc_scale, hc_base = _pre_inputs(T, 907)
    dm = device_normal_f32(0, 907, "dots", (2, T, MIX), std=2.0)
    dy = device_normal_bf16(0, 907, "dy", (T, H))
    d_post = device_normal_f32(0, 907, "d_post", (T, HC))
    d_comb = device_normal_f32(0, 907, "d_comb", (T, HC, HC))
    sc, base = to_dev_f32(hc_scale), to_dev_f32(hc_base)
    big = mhc.mhc_pre_from_dots_backward(dy, d_post, d_comb, dm, res, sc, base)
    torch.cuda.synchronize()
    idx = torch.as_tensor(rows, device="cuda")
    got = {k: bits_of(big["d_res"][idx]) if k == "d_res" else f32_of(big[k][idx]) for k in ("d_res", "d_dot")}
    del big
    small = mhc.mhc_pre_from_dots_backward(_at(dy, rows).contiguous(), _at(d_post, rows).contiguous(),
                                           _at(d_comb, rows).contiguous(), dm[:, idx].contiguous(),
                                           _at(res, rows).contiguous(), sc, base)
    torch.cuda.synchronize()
    assert np.array_equal(got["d_res"], bits_of(small["d_res"]))
    assert np.array_equal(got["d_dot"], f32_of(small["d_dot"]))


def test_f32_stream_post_expand_head_mean_chunks():
    """The fp32-stream post-map, model entry and unweighted head across a chunk edge."""
    from tests._helpers import assert_f32_chain_close, post_f32s_scale
    mhc = _mhc()
    T, rows = _plan("post_f32")
    assert _plan("expand_f32")[0] == T and _plan("head_mean_f32")[0] == T
    x = device_normal_bf16(0, 908, "x", (T, H))
    res = device_normal_f32(0, 908, "res", (T, HC, H))
    post = device_normal_f32(0, 908, "post", (T, HC))
    comb = device_normal_f32(0, 908, "comb_logits", (T, HC, HC), std=0.5)
    out = mhc.mhc_post_f32(x, res, post, comb)
    torch.cuda.synchronize()
    xr, rr, pr, cr = bits_of(_at(x, rows)), f32_of(_at(res, rows)), f32_of(_at(post, rows)), f32_of(_at(comb, rows))
    ref = oracle.post_f32s(xr, rr, pr.astype(np.float64), cr.astype(np.float64))
    assert_f32_chain_close(f32_of(_at(out, rows)), ref, post_f32s_scale(xr, rr, pr, cr), f"post f32 T={T}")
    del out, post, comb
    y = mhc.mhc_head_mean_f32(res)
    torch.cuda.synchronize()
    assert_bf16_close(bits_of(_at(y, rows)), oracle.head_mean_f32s(rr), f"head_mean f32 T={T}")
    del res, y
    streams = mhc.mhc_expand_f32(x)
    torch.cuda.synchronize()
    assert np.array_equal(f32_of(_at(streams, rows)), oracle.expand_f32s(xr))
