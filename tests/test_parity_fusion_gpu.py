"""GPU parity of the cross-sublayer fusion: the post-map that also projects its output for
the next sublayer's pre-map (libmhc's mhc_post_project, through the thin binding).

What is checked, on the same seeded inputs:
- out against the fp64 oracle post-map (and bit for bit against mhc_post, which has the
  same arithmetic);
- the 24 dots and the sum of squares against the fp64 projection of out, within the fp32
  accumulation bound;
- the chained pre-map (mhc_pre_from_dots fed those dots, res = out) against the oracle's
  whole pre-map of out with the next weights, within the stated tolerances.
"""
import numpy as np
import pytest

import oracle
from mhc_inputs import HC, MIX, bf16_bits_to_f32, layer_inputs, named_layer, normal_f32, uniform_f32
from tests._helpers import (assert_bf16_close, assert_f32_close, bits_of, f32_of, sample_tokens, to_dev_bf16,
                            to_dev_f32)

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


def _mixes(T, cfg):
    """post ~ U(0, 2) and the Sinkhorn projection of N(0, 1) comb logits (fp32)."""
    post = uniform_f32(0, cfg, "post", (T, HC), 0.0, 2.0)
    comb = oracle.sinkhorn(normal_f32(0, cfg, "comb_logits", (T, HC, HC), 1.0), 20, 1e-6).astype(np.float32)
    return post, comb


def _check_dots(dm, sq, out_bits, fn, what):
    """dm [T, 24] and sq [T] from the kernel against the fp64 projection and sum of squares
    of out_bits [T, 4, H].  The products are exact (bf16 x bf16 in fp32), so the error is
    that of fp32 partial sums: a few dozen roundings per 128-wide slice and one per slice
    in the sum over slices, each below the sum of |term|."""
    T, _, H = out_bits.shape
    o = bf16_bits_to_f32(out_bits).astype(np.float64).reshape(T, HC * H)
    w = fn.astype(np.float64)
    rd = o @ w.T
    mags = np.abs(o) @ np.abs(w).T
    rsq = (o * o).sum(axis=1)
    assert dm.shape == rd.shape and sq.shape == rsq.shape, (what, dm.shape, sq.shape)
    err = np.abs(dm.astype(np.float64) - rd)
    bad = ~(err <= 1e-5 * mags + 1e-9)
    assert not bad.any(), f"{what} dot_mix: {int(bad.sum())} outside; first {np.argwhere(bad)[:3].tolist()}"
    err = np.abs(sq.astype(np.float64) - rsq)
    bad = ~(err <= 1e-5 * rsq + 1e-9)
    assert not bad.any(), f"{what} sqrsum: {int(bad.sum())} outside; first {np.argwhere(bad)[:3].tolist()}"


def _chain_check(mhc, inp, dm_d, sq_d, out_d, out_bits, what, tokens=None):
    """mhc_pre_from_dots on the dots against the oracle's pre-map of out (next weights)."""
    y, post, comb, pre = mhc.mhc_pre_from_dots(dm_d, out_d, to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base),
                                               sqrsum=sq_d, return_pre=True)
    torch.cuda.synchronize()
    sel = slice(None) if tokens is None else tokens
    ref = oracle.pre(out_bits[sel], inp.hc_fn, inp.hc_scale, inp.hc_base)
    assert_f32_close(f32_of(pre)[sel], ref["pre"], f"{what} next pre")
    assert_f32_close(f32_of(post)[sel], ref["post"], f"{what} next post")
    assert_f32_close(f32_of(comb)[sel], ref["comb"], f"{what} next comb")
    assert_bf16_close(bits_of(y)[sel], ref["y"], f"{what} next y")


def _run(mhc, inp, post, comb, **kw):
    fn_d = to_dev_f32(inp.hc_fn)
    out, dm, sq = mhc.mhc_post_project(to_dev_bf16(inp.x), to_dev_bf16(inp.res), to_dev_f32(post),
                                       to_dev_f32(comb), fn_d, **kw)
    torch.cuda.synchronize()
    return out, dm, sq


# (T, H): ragged token counts against the 32-token steps and 64-token ranges; H with a
# narrower last slice (1000, 96, 8, 2056), one slice (64, 128) and the wide shapes
FUSION_SHAPES = [(16, 256), (5, 64), (33, 1000), (70, 96), (130, 2056), (21, 7168), (300, 1024), (1, 8),
                 (65, 4096), (97, 128), (2, 16384)]


@pytest.mark.parametrize("T,H", FUSION_SHAPES)
def test_post_project_matches_oracle(T, H):
    mhc = _mhc()
    cfg = 700 + (T * 7 + H) % 89
    inp = layer_inputs(T, H, cfg=cfg)
    post, comb = _mixes(T, cfg)
    out, dm, sq = _run(mhc, inp, post, comb)
    assert dm.shape == (T, MIX) and sq.shape == (T,)
    ref_out = oracle.post(inp.x, inp.res, post.astype(np.float64), comb.astype(np.float64))
    ob = bits_of(out)
    assert_bf16_close(ob, ref_out, f"fused out T={T} H={H}")
    plain = mhc.mhc_post(to_dev_bf16(inp.x), to_dev_bf16(inp.res), to_dev_f32(post), to_dev_f32(comb))
    torch.cuda.synchronize()
    assert np.array_equal(ob, bits_of(plain)), "fused out differs from mhc_post"
    _check_dots(f32_of(dm), f32_of(sq), ob, inp.hc_fn, f"T={T} H={H}")
    _chain_check(mhc, inp, dm, sq, out, ob, f"T={T} H={H}")


def test_post_project_in_place_and_supplied_buffers():
    """out = res (the residual updated in place), caller-supplied partials and workspace."""
    mhc = _mhc()
    T, H = 77, 1536
    inp = layer_inputs(T, H, cfg=790)
    post, comb = _mixes(T, 790)
    res_d = to_dev_bf16(inp.res)
    dm = torch.full((T, MIX), float("nan"), device="cuda")
    sq = torch.full((T,), float("nan"), device="cuda")
    ws = torch.full((mhc.mhc_post_project_workspace_bytes(T, H),), 0xFF, dtype=torch.uint8, device="cuda")
    out, dm2, sq2 = mhc.mhc_post_project(to_dev_bf16(inp.x), res_d, to_dev_f32(post), to_dev_f32(comb),
                                         to_dev_f32(inp.hc_fn), out=res_d, dot_mix=dm, sqrsum=sq, workspace=ws)
    torch.cuda.synchronize()
    assert out.data_ptr() == res_d.data_ptr() and dm2.data_ptr() == dm.data_ptr() and sq2.data_ptr() == sq.data_ptr()
    ob = bits_of(res_d)
    assert_bf16_close(ob, oracle.post(inp.x, inp.res, post.astype(np.float64), comb.astype(np.float64)),
                      "in-place out")
    _check_dots(f32_of(dm), f32_of(sq), ob, inp.hc_fn, "in place")


def test_post_project_deterministic_and_empty():
    mhc = _mhc()
    inp = layer_inputs(150, 2048, cfg=791)
    post, comb = _mixes(150, 791)
    a = _run(mhc, inp, post, comb)
    b = _run(mhc, inp, post, comb)
    for u, v in zip(a, b):
        assert np.array_equal(bits_of(u) if u.dtype == torch.bfloat16 else f32_of(u),
                              bits_of(v) if v.dtype == torch.bfloat16 else f32_of(v))
    e = torch.empty(0, HC, 64, dtype=torch.bfloat16, device="cuda")
    out, dm, sq = mhc.mhc_post_project(torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"), e,
                                       torch.empty(0, HC, device="cuda"), torch.empty(0, HC, HC, device="cuda"),
                                       torch.zeros(MIX, HC * 64, device="cuda"))
    torch.cuda.synchronize()
    assert out.shape == (0, HC, 64) and dm.shape == (0, MIX) and sq.shape == (0,)


def test_post_project_full_size_h7168_sampled():
    """T=8192, H=7168: out bit for bit against mhc_post over every token, and sampled tokens
    against the oracle (out, the dots and sum of squares, the chained next pre-map)."""
    mhc = _mhc()
    inp = named_layer("layer_h7168")
    T, H = inp.T, inp.H
    post, comb = _mixes(T, 792)
    out, dm, sq = _run(mhc, inp, post, comb)
    plain = mhc.mhc_post(to_dev_bf16(inp.x), to_dev_bf16(inp.res), to_dev_f32(post), to_dev_f32(comb))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16)), "fused out differs from mhc_post"
    del plain
    toks = sample_tokens(T, 24, seed=11)
    ob = bits_of(out[torch.from_numpy(toks).cuda()])
    assert_bf16_close(ob, oracle.post(inp.x[toks], inp.res[toks], post[toks].astype(np.float64),
                                      comb[toks].astype(np.float64)), "8192x7168 out")
    _check_dots(f32_of(dm)[toks], f32_of(sq)[toks], ob, inp.hc_fn, "8192x7168")
    y, npost, ncomb, npre = mhc.mhc_pre_from_dots(dm, out, to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base),
                                                  sqrsum=sq, return_pre=True)
    torch.cuda.synchronize()
    ref = oracle.pre(ob, inp.hc_fn, inp.hc_scale, inp.hc_base)
    assert_f32_close(f32_of(npre)[toks], ref["pre"], "8192x7168 next pre")
    assert_f32_close(f32_of(npost)[toks], ref["post"], "8192x7168 next post")
    assert_f32_close(f32_of(ncomb)[toks], ref["comb"], "8192x7168 next comb")
    assert_bf16_close(bits_of(y)[toks], ref["y"], "8192x7168 next y")
