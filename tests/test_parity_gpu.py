"""GPU parity: libmhc (through its C ABI via the thin binding) against the fp64 CPU oracle.

Every case compares element by element on seeded inputs; full-size workloads
compare sampled tokens (tokens are independent, so the oracle runs only on
those rows) plus properties that hold at any size.
"""
import numpy as np
import pytest

import oracle
from mhc_inputs import (HC, bf16_bits_to_f32, layer_inputs, named_layer, post_inputs, sinkhorn_logits,
                        SINKHORN_N)
from tests._helpers import (assert_bf16_close, assert_f32_close, bits_of, check_pre_all_tokens, f32_of, sample_tokens,
                            to_dev_bf16, to_dev_f32)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


# ----------------------------------------------------------------------------- post-map

POST_SHAPES = [(16, 256), (5, 64), (7, 127), (3, 1001), (9, 1536), (6, 2048), (37, 4096), (21, 7168),
               (4, 8192), (3, 16392), (3000, 1000), (1, 1), (2, 8), (3, 520)]


def _post_case(T, H, cfg=2):
    res, x, post, comb_logits = post_inputs(T, H, cfg=cfg)
    comb = oracle.sinkhorn(comb_logits, 20, 1e-6).astype(np.float32)
    return res, x, post, comb


@pytest.mark.parametrize("T,H", POST_SHAPES)
def test_post_matches_oracle(T, H):
    mhc = _mhc()
    res, x, post, comb = _post_case(T, H, cfg=200 + H % 97)
    out = mhc.mhc_post(to_dev_bf16(x), to_dev_bf16(res), to_dev_f32(post), to_dev_f32(comb))
    torch.cuda.synchronize()
    ref = oracle.post(x, res, post.astype(np.float64), comb.astype(np.float64))
    assert_bf16_close(bits_of(out), ref, f"post T={T} H={H}")


def test_post_full_size_h4096():
    """The post-map workload T=4096, H=4096, every element."""
    mhc = _mhc()
    res, x, post, comb = _post_case(4096, 4096, cfg=2)
    out = mhc.mhc_post(to_dev_bf16(x), to_dev_bf16(res), to_dev_f32(post), to_dev_f32(comb))
    torch.cuda.synchronize()
    ref = oracle.post(x, res, post.astype(np.float64), comb.astype(np.float64))
    assert_bf16_close(bits_of(out), ref, "post 4096x4096")


def test_post_post_shape_t41_accepted():
    mhc = _mhc()
    res, x, post, comb = _post_case(6, 64, cfg=210)
    a = mhc.mhc_post(to_dev_bf16(x), to_dev_bf16(res), to_dev_f32(post), to_dev_f32(comb))
    b = mhc.mhc_post(to_dev_bf16(x), to_dev_bf16(res), to_dev_f32(post).reshape(6, 4, 1), to_dev_f32(comb))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("H", [256, 127])
def test_post_identity_bit_exact(H):
    """comb = I, post = 1 gives bf16(res + x) with one rounding; post = 0 gives res."""
    mhc = _mhc()
    T = 64
    res, x, _, _ = _post_case(T, H, cfg=220)
    eye = np.broadcast_to(np.eye(HC, dtype=np.float32), (T, HC, HC)).copy()
    out1 = mhc.mhc_post(to_dev_bf16(x), to_dev_bf16(res), to_dev_f32(np.ones((T, HC))), to_dev_f32(eye))
    out0 = mhc.mhc_post(to_dev_bf16(x), to_dev_bf16(res), to_dev_f32(np.zeros((T, HC))), to_dev_f32(eye))
    torch.cuda.synchronize()
    s = bf16_bits_to_f32(res).astype(np.float64) + bf16_bits_to_f32(x).astype(np.float64)[:, None, :]
    exact32 = s.astype(np.float32).astype(np.float64) == s  # the fp32 accumulator holds the sum exactly
    assert exact32.mean() > 0.999
    got = bits_of(out1)
    assert np.array_equal(got[exact32], oracle.round_bf16(s)[exact32])
    assert_bf16_close(got, s, "identity post")
    assert np.array_equal(bits_of(out0), res)


def test_post_permutation_orientation():
    mhc = _mhc()
    T, H = 8, 512
    res, x, _, _ = _post_case(T, H, cfg=221)
    perm = [2, 0, 3, 1]
    comb = np.zeros((T, HC, HC), np.float32)
    for o, n in enumerate(perm):
        comb[:, o, n] = 1.0
    out = bits_of(mhc.mhc_post(to_dev_bf16(x), to_dev_bf16(res), to_dev_f32(np.zeros((T, HC))), to_dev_f32(comb)))
    for o, n in enumerate(perm):
        assert np.array_equal(out[:, n], res[:, o])


@pytest.mark.parametrize("H", [4096, 1001])
def test_post_in_place_alias(H):
    """out == res: the new streams overwrite the old ones."""
    mhc = _mhc()
    T = 33
    res, x, post, comb = _post_case(T, H, cfg=222)
    r = to_dev_bf16(res)
    out = mhc.mhc_post(to_dev_bf16(x), r, to_dev_f32(post), to_dev_f32(comb), out=r)
    torch.cuda.synchronize()
    assert out.data_ptr() == r.data_ptr()
    ref = oracle.post(x, res, post.astype(np.float64), comb.astype(np.float64))
    assert_bf16_close(bits_of(r), ref, "post in place")


def test_post_deterministic_and_empty():
    mhc = _mhc()
    res, x, post, comb = _post_case(100, 1000, cfg=223)
    args = (to_dev_bf16(x), to_dev_bf16(res), to_dev_f32(post), to_dev_f32(comb))
    a, b = mhc.mhc_post(*args), mhc.mhc_post(*args)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    e = mhc.mhc_post(torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"),
                     torch.empty(0, 4, 64, dtype=torch.bfloat16, device="cuda"),
                     torch.empty(0, 4, device="cuda"), torch.empty(0, 4, 4, device="cuda"))
    assert e.shape == (0, 4, 64)


# ----------------------------------------------------------------------------- Sinkhorn

@pytest.mark.parametrize("iters", [1, 2, 3, 20])
def test_sinkhorn_full_size(iters):
    """2^20 matrices of clamp(N(0,2), +-8) logits with stress matrices; every element."""
    mhc = _mhc()
    lg = sinkhorn_logits(SINKHORN_N, seed=0)
    out = f32_of(mhc.mhc_sinkhorn(to_dev_f32(lg), num_iters=iters, eps=1e-6))
    ref = oracle.sinkhorn(lg.astype(np.float64), iters, 1e-6)
    assert_f32_close(out, ref, f"sinkhorn iters={iters}")
    assert np.abs(out.sum(axis=-2) - 1.0).max() <= 1e-5  # columns are normalised last


def test_sinkhorn_row_sums_report_and_tiny_case_converges():
    mhc = _mhc()
    lg = sinkhorn_logits(SINKHORN_N, seed=0)
    out = f32_of(mhc.mhc_sinkhorn(to_dev_f32(lg), num_iters=20, eps=1e-6))
    frac = float((np.abs(out.sum(axis=-1) - 1).max(axis=-1) > 1e-5).mean())
    print(f"\nrow-sum |err| > 1e-5 after 20 iterations: {frac:.4f} of matrices")
    # the tiny layer's comb logits converge within 20 iterations in every row
    inp = named_layer("tiny")
    y, post, comb = mhc.mhc_pre_fused(to_dev_bf16(inp.res), to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale),
                                      to_dev_f32(inp.hc_base))
    c = f32_of(comb)
    assert np.abs(c.sum(axis=-1) - 1).max() <= 1e-5 and np.abs(c.sum(axis=-2) - 1).max() <= 1e-5


def test_sinkhorn_in_place_and_unaligned():
    mhc = _mhc()
    lg = sinkhorn_logits(1000, seed=9)
    ref = oracle.sinkhorn(lg.astype(np.float64), 20, 1e-6)
    d = to_dev_f32(lg)
    mhc.mhc_sinkhorn(d, out=d)
    assert_f32_close(f32_of(d), ref, "sinkhorn in place")
    # a view starting 4 bytes into a buffer takes the scalar-load path
    buf = torch.zeros(1000 * 16 + 1, device="cuda")
    buf[1:] = to_dev_f32(lg).reshape(-1)
    view = buf[1:].view(1000, 4, 4)
    out = torch.empty(1000 * 16 + 1, device="cuda")[1:].view(1000, 4, 4)
    mhc.mhc_sinkhorn(view, out=out)
    assert_f32_close(f32_of(out), ref, "sinkhorn unaligned")


# ----------------------------------------------------------------------------- pre-map

def _run_pre(inp, **kw):
    mhc = _mhc()
    p = dict(inp.params)
    p.update(kw)
    y, post, comb, pre = mhc.mhc_pre_fused(
        to_dev_bf16(inp.res), to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base),
        rms_eps=p["rms_eps"], pre_eps=p["pre_eps"], sinkhorn_eps=p["sinkhorn_eps"], post_mult=p["post_mult"],
        num_iters=p["num_iters"], return_pre=True)
    torch.cuda.synchronize()
    return bits_of(y), f32_of(post), f32_of(comb), f32_of(pre), p


def _check_pre(inp, got, tokens=None, what=""):
    y, post, comb, pre, p = got
    res = inp.res if tokens is None else inp.res[tokens]
    ref = oracle.pre(res, inp.hc_fn, inp.hc_scale, inp.hc_base, rms_eps=p["rms_eps"], pre_eps=p["pre_eps"],
                     sinkhorn_eps=p["sinkhorn_eps"], post_mult=p["post_mult"], num_iters=p["num_iters"])
    sel = (lambda a: a) if tokens is None else (lambda a: a[tokens])
    assert_f32_close(sel(pre), ref["pre"], f"{what} pre")
    assert_f32_close(sel(post), ref["post"], f"{what} post")
    assert_f32_close(sel(comb), ref["comb"], f"{what} comb")
    assert_bf16_close(sel(y), ref["y"], f"{what} y")
    return ref


# (T, H): tile edges (T = 1, 63..65, 129), ragged H (H % 32 != 0, H % 8 != 0), one slice
# (H <= 128), many slices, and H above the fused kernel's range (split-K fallback path).
PRE_SHAPES = [(16, 256), (1, 64), (3, 8), (100, 512), (65, 7168), (32, 7168), (40, 127), (24, 1001),
              (129, 1536), (7, 16392), (70, 96), (63, 200), (130, 4104), (3, 65544), (2, 65537),
              # many 64-token tiles per workgroup (odd and even counts), H % 32 != 0
              (1100, 2048), (600, 7000), (1537, 4104), (1030, 7168), (700, 8)]


@pytest.mark.parametrize("T,H", PRE_SHAPES)
def test_pre_matches_oracle(T, H):
    inp = layer_inputs(T, H, cfg=300 + (T * 7 + H) % 89)
    _check_pre(inp, _run_pre(inp), what=f"pre T={T} H={H}")


def test_pre_tiny_layer_all_outputs():
    inp = named_layer("tiny")
    _check_pre(inp, _run_pre(inp), what="tiny")


@pytest.mark.parametrize("kw", [dict(post_mult=2.0), dict(num_iters=1), dict(num_iters=3),
                                dict(rms_eps=1e-2, pre_eps=0.0, sinkhorn_eps=1e-3)])
def test_pre_parameters(kw):
    inp = layer_inputs(48, 384, cfg=330)
    _check_pre(inp, _run_pre(inp, **kw), what=f"pre {kw}")


def test_pre_scale_vectors_and_base():
    inp = layer_inputs(20, 640, cfg=331, scale=(0.5, 2.0, 3.0), base_std=1.0)
    _check_pre(inp, _run_pre(inp), what="pre scales")


def test_pre_ragged_h1000_full():
    inp = named_layer("ragged_h1000")
    _check_pre(inp, _run_pre(inp), what="pre 3000x1000")


def test_pre_decode_h7168_full():
    inp = named_layer("decode_h7168")
    _check_pre(inp, _run_pre(inp), what="pre 32x7168")


def test_pre_full_size_h7168_all_tokens():
    """T=8192, H=7168 (the measured layer, in the launch the benchmark times): every token of
    y, post, comb and pre against the oracle."""
    inp = named_layer("layer_h7168")
    y, post, comb, pre, _ = _run_pre(inp)
    check_pre_all_tokens(inp, (y, post, comb, pre), "pre 8192x7168")
    assert np.abs(comb.sum(axis=-2) - 1).max() <= 1e-5
    assert np.all(pre > 0) and np.all(pre <= 1 + 2e-6) and np.all(post >= 0) and np.all(post <= 1)


def test_pre_zero_scale_selects_stream():
    inp = layer_inputs(12, 256, cfg=332, scale=(0.0, 0.0, 0.0))
    inp.hc_base[:4] = [30.0, -30.0, -30.0, -30.0]
    y, post, comb, pre, p = _run_pre(inp)
    assert_bf16_close(y, bf16_bits_to_f32(inp.res[:, 0, :]).astype(np.float64) * (1 + 1e-6), "y selects stream 0")
    assert np.allclose(comb, oracle.sinkhorn(inp.hc_base[8:].reshape(1, 4, 4).astype(np.float64), 20, 1e-6),
                       atol=1e-5)


def test_pre_deterministic():
    inp = layer_inputs(1100, 2048, cfg=333)
    a, b = _run_pre(inp), _run_pre(inp)
    for u, v in zip(a[:4], b[:4]):
        assert np.array_equal(u, v)


def test_pre_empty():
    mhc = _mhc()
    y, post, comb = mhc.mhc_pre_fused(torch.empty(0, 4, 64, dtype=torch.bfloat16, device="cuda"),
                                      torch.zeros(24, 256, device="cuda"), torch.ones(3, device="cuda"),
                                      torch.zeros(24, device="cuda"))
    assert y.shape == (0, 64) and post.shape == (0, 4) and comb.shape == (0, 4, 4)


# ----------------------------------------------------------------------------- pre-map from external dots

def _dots_inputs(inp, splits, cfg):
    """fp32 dot partials: the exact fp64 projection, split into `splits` random parts (last part closes it)."""
    d = oracle.project(inp.res, inp.hc_fn)
    g = np.random.default_rng(cfg)
    if splits == 1:
        return d.astype(np.float32)[None]
    parts = (g.standard_normal((splits - 1,) + d.shape) * 0.5).astype(np.float32)
    last = (d - parts.astype(np.float64).sum(axis=0)).astype(np.float32)
    return np.concatenate([parts, last[None]], axis=0)


def _run_dots(inp, dm, sq=None, k=None, **kw):
    mhc = _mhc()
    p = dict(inp.params)
    p.update(kw)
    y, post, comb, pre = mhc.mhc_pre_from_dots(
        to_dev_f32(dm), to_dev_bf16(inp.res), to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base),
        sqrsum=None if sq is None else to_dev_f32(sq), k=k, rms_eps=p["rms_eps"], pre_eps=p["pre_eps"],
        sinkhorn_eps=p["sinkhorn_eps"], post_mult=p["post_mult"], num_iters=p["num_iters"], return_pre=True)
    torch.cuda.synchronize()
    ref = oracle.pre_from_dots(dm, inp.res, inp.hc_scale, inp.hc_base, sqrsum=sq, k=k, rms_eps=p["rms_eps"],
                               pre_eps=p["pre_eps"], sinkhorn_eps=p["sinkhorn_eps"], post_mult=p["post_mult"],
                               num_iters=p["num_iters"])
    return (bits_of(y), f32_of(post), f32_of(comb), f32_of(pre)), ref


def _check_dots(got, ref, what, tokens=None):
    y, post, comb, pre = got
    sel = (lambda a: a) if tokens is None else (lambda a: a[tokens])
    assert_f32_close(sel(pre), sel(ref["pre"]), f"{what} pre")
    assert_f32_close(sel(post), sel(ref["post"]), f"{what} post")
    assert_f32_close(sel(comb), sel(ref["comb"]), f"{what} comb")
    assert_bf16_close(sel(y), sel(ref["y"]), f"{what} y")


# (T, H, splits): register path for 1, 2, 4 and 8 chunks per thread (H <= 2048, 4096, 8192, 16384), the
# two-pass path (H % 8 != 0, H > 16384), one and several splits
DOTS_SHAPES = [(16, 256, 1), (5, 8, 2), (33, 2048, 4), (9, 4096, 1), (7, 7168, 16), (3, 16384, 2),
               (4, 16392, 1), (6, 127, 3), (5, 1001, 1), (2, 65537, 2), (70, 96, 8)]


@pytest.mark.parametrize("T,H,splits", DOTS_SHAPES)
def test_pre_from_dots_computed_sum_of_squares(T, H, splits):
    inp = layer_inputs(T, H, cfg=400 + (T * 13 + H) % 71)
    dm = _dots_inputs(inp, splits, cfg=T + H)
    got, ref = _run_dots(inp, dm)
    _check_dots(got, ref, f"dots T={T} H={H} S={splits}")


@pytest.mark.parametrize("splits", [1, 4])
def test_pre_from_dots_supplied_sum_of_squares_and_k(splits):
    inp = layer_inputs(40, 1536, cfg=430)
    dm = _dots_inputs(inp, splits, cfg=splits)
    r = bf16_bits_to_f32(inp.res).astype(np.float64)
    S = (r * r).sum(axis=(1, 2))
    sq = np.stack([S / splits] * splits).astype(np.float32)
    got, ref = _run_dots(inp, dm, sq=sq, k=2.0 * 4 * 1536, post_mult=2.0, num_iters=3)
    _check_dots(got, ref, f"dots supplied S={splits}")


# one split with the sum of squares supplied: the collapse-kernel path when H % 8 == 0
# (any H, including past the register path's 16384), the workgroup-per-token path otherwise
ONE_SPLIT_SHAPES = [(16, 256), (5, 8), (33, 2048), (7, 7168), (3, 16384), (4, 16392), (6, 127), (2, 65544),
                    (70, 96), (1, 1000), (130, 520)]


@pytest.mark.parametrize("T,H", ONE_SPLIT_SHAPES)
def test_pre_from_dots_one_split_supplied_sum_of_squares(T, H):
    inp = layer_inputs(T, H, cfg=440 + (T * 11 + H) % 67)
    dm = _dots_inputs(inp, 1, cfg=T * 3 + H)
    r = bf16_bits_to_f32(inp.res).astype(np.float64)
    sq = (r * r).sum(axis=(1, 2)).astype(np.float32)[None]
    got, ref = _run_dots(inp, dm, sq=sq)
    _check_dots(got, ref, f"one split T={T} H={H}")
    got, ref = _run_dots(inp, dm, sq=sq, k=3.0 * H, post_mult=1.5, num_iters=7, pre_eps=1e-3)
    _check_dots(got, ref, f"one split, parameters T={T} H={H}")


def test_pre_from_dots_full_size_h7168_sampled():
    """T=8192, H=7168 with one split and the sum of squares computed here (the measured launch)."""
    mhc = _mhc()
    inp = named_layer("layer_h7168")
    toks = sample_tokens(inp.T, 32, seed=3)
    d = np.zeros((inp.T, 24), np.float32)
    d[toks] = oracle.project(inp.res[toks], inp.hc_fn).astype(np.float32)
    y, post, comb, pre = mhc.mhc_pre_from_dots(to_dev_f32(d), to_dev_bf16(inp.res), to_dev_f32(inp.hc_scale),
                                               to_dev_f32(inp.hc_base), return_pre=True)
    torch.cuda.synchronize()
    ref = oracle.pre_from_dots(d[toks], inp.res[toks], inp.hc_scale, inp.hc_base)
    _check_dots((bits_of(y)[toks], f32_of(post)[toks], f32_of(comb)[toks], f32_of(pre)[toks]), ref,
                "dots 8192x7168")
    assert np.abs(f32_of(comb).sum(axis=-2) - 1).max() <= 1e-5


def test_pre_from_dots_agrees_with_pre_fused():
    """The external-projection path fed the projection of res gives the fused pre-map's outputs."""
    mhc = _mhc()
    inp = layer_inputs(64, 1024, cfg=431)
    res = to_dev_bf16(inp.res)
    fn, sc, base = to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base)
    a = mhc.mhc_pre_fused(res, fn, sc, base, return_pre=True)
    dm = torch.from_numpy(oracle.project(inp.res, inp.hc_fn).astype(np.float32)).cuda()
    b = mhc.mhc_pre_from_dots(dm, res, sc, base, return_pre=True)
    torch.cuda.synchronize()
    for u, v, name in zip(a[1:], b[1:], ("post", "comb", "pre")):
        assert np.abs(f32_of(u).astype(np.float64) - f32_of(v)).max() <= 2e-5, name


def test_pre_from_dots_deterministic_and_empty():
    mhc = _mhc()
    inp = layer_inputs(50, 2048, cfg=432)
    dm = _dots_inputs(inp, 2, cfg=1)
    a, _ = _run_dots(inp, dm)
    b, _ = _run_dots(inp, dm)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    y, post, comb = mhc.mhc_pre_from_dots(torch.zeros(0, 24, device="cuda"),
                                          torch.empty(0, 4, 64, dtype=torch.bfloat16, device="cuda"),
                                          torch.ones(3, device="cuda"), torch.zeros(24, device="cuda"))
    assert y.shape == (0, 64)


# ----------------------------------------------------------------------------- whole layer

def test_layer_pre_then_post_full_size_all_tokens():
    """T=8192, H=7168 pre-map then post-map with x as the sublayer output: every token of y
    and out against the oracle (out from the oracle's own post and comb)."""
    mhc = _mhc()
    inp = named_layer("layer_h7168")
    res_d = to_dev_bf16(inp.res)
    y, post, comb = mhc.mhc_pre_fused(res_d, to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale),
                                      to_dev_f32(inp.hc_base))
    out = mhc.mhc_post(to_dev_bf16(inp.x), res_d, post, comb)
    torch.cuda.synchronize()
    check_pre_all_tokens(inp, (bits_of(y), f32_of(post), f32_of(comb), None), "layer", x=inp.x, out=bits_of(out))
