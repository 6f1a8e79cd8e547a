"""GPU parity of the fp32-residual-stream entry points (mhc_pre_fused_f32, mhc_post_f32,
mhc_expand_f32, mhc_head_mean_f32) against the fp64 oracle's fp32-stream functions.

Streams are full fp32 values (N(0,1) draws, almost none of them bf16 values), so a kernel
that rounded them through bf16 anywhere would fail the mix tolerance.  Tolerances: mixes
(pre, post, comb) within 1e-5, bf16 rows (y) within 2^-7 |ref| + 1e-3 of the unrounded
fp64 value, fp32 streams out of the post-map within 2^-21 of the sum of the absolute terms
(an fp32 chain of five roundings), expand exact."""
import numpy as np
import pytest

import oracle
from mhc_inputs import HC, layer_inputs_f32s, normal_bf16, normal_f32, uniform_f32
from tests._helpers import (assert_bf16_close, assert_f32_chain_close, bits_of, check_pre_all_tokens, f32_of,
                            post_f32s_scale, to_dev_bf16, to_dev_f32)

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


def _run_pre(inp, res=None, **kw):
    mhc = _mhc()
    p = dict(inp.params)
    p.update(kw)
    res = to_dev_f32(inp.res) if res is None else res
    y, post, comb, pre = mhc.mhc_pre_fused_f32(
        res, to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base), rms_eps=p["rms_eps"],
        pre_eps=p["pre_eps"], sinkhorn_eps=p["sinkhorn_eps"], post_mult=p["post_mult"], num_iters=p["num_iters"],
        return_pre=True)
    torch.cuda.synchronize()
    return bits_of(y), f32_of(post), f32_of(comb), f32_of(pre)


def _misaligned_f32(a: np.ndarray):
    """A device copy of `a` that starts 4 bytes past a 16-byte boundary (the scalar path)."""
    flat = torch.empty(a.size + 1, dtype=torch.float32, device="cuda")
    view = flat[1:].view(a.shape)
    view.copy_(to_dev_f32(a))
    assert view.data_ptr() % 16 == 4
    return view


# (T, H): tiny, ragged T around the 64-token tile, H off the 4-, 32- and 128-wide blocks
# (H % 4 != 0 takes the scalar path), and the model's widths
PRE_SHAPES = [(1, 1), (2, 3), (5, 8), (16, 256), (33, 1000), (64, 1024), (65, 2048), (200, 4096), (130, 7168),
              (64, 7169), (100, 5003), (129, 130), (700, 2056)]


@pytest.mark.parametrize("T,H", PRE_SHAPES)
def test_pre_f32_matches_oracle_every_token(T, H):
    inp = layer_inputs_f32s(T, H, cfg=800 + (T * 7 + H) % 89)
    check_pre_all_tokens(inp, _run_pre(inp), f"pre f32 T={T} H={H}")


@pytest.mark.parametrize("kw", [dict(post_mult=2.0), dict(num_iters=1), dict(num_iters=3),
                                dict(rms_eps=1e-2, pre_eps=1e-3, sinkhorn_eps=1e-3), dict(pre_eps=0.0)])
def test_pre_f32_parameters(kw):
    inp = layer_inputs_f32s(96, 1536, cfg=840)
    check_pre_all_tokens(inp, _run_pre(inp, **kw), f"pre f32 {kw}", params=kw)


def test_pre_f32_scales_and_large_stream_values():
    """Scale vectors, base std 1 and streams of std 100 (the RMS normalisation absorbs it)."""
    inp = layer_inputs_f32s(80, 2048, cfg=841, scale=(0.5, 2.0, 3.0), base_std=1.0)
    inp.res = inp.res * np.float32(100.0)
    check_pre_all_tokens(inp, _run_pre(inp), "pre f32 scales")


def test_pre_f32_scalar_path_equals_vector_path():
    """A misaligned copy of the streams takes the scalar loads: same products in the same
    order, so the outputs are bit-identical to the vector path's."""
    inp = layer_inputs_f32s(70, 1024, cfg=842)
    a = _run_pre(inp)
    b = _run_pre(inp, res=_misaligned_f32(inp.res))
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_pre_f32_full_size_h7168_all_tokens():
    """T = 8192, H = 7168 (the headline shape) over fp32 streams: every token."""
    inp = layer_inputs_f32s(8192, 7168, cfg=843)
    check_pre_all_tokens(inp, _run_pre(inp), "pre f32 T=8192 H=7168")


def test_pre_f32_garbage_workspace_and_determinism():
    mhc = _mhc()
    inp = layer_inputs_f32s(300, 4096, cfg=844)
    need = mhc.mhc_pre_fused_workspace_bytes(300, 4096)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    res = to_dev_f32(inp.res)
    outs = []
    for _ in range(2):
        y, post, comb = mhc.mhc_pre_fused_f32(res, to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale),
                                              to_dev_f32(inp.hc_base), workspace=ws)
        torch.cuda.synchronize()
        outs.append((bits_of(y), f32_of(post), f32_of(comb)))
    for u, v in zip(*outs):
        assert np.array_equal(u, v)
    check_pre_all_tokens(inp, outs[0] + (None,), "pre f32 garbage workspace")


# ---------------------------------------------------------------- post-map

def _post_case(T, H, cfg):
    res = normal_f32(0, cfg, "res", (T, HC, H), 1.0)
    x = normal_bf16(0, cfg, "x", (T, H))
    post = uniform_f32(0, cfg, "post", (T, HC), 0.0, 2.0)
    comb = oracle.sinkhorn(normal_f32(0, cfg, "comb_logits", (T, HC, HC), 1.0).astype(np.float64), 20,
                           1e-6).astype(np.float32)
    return x, res, post, comb


def _check_post(out, case, what):
    x, res, post, comb = case
    ref = oracle.post_f32s(x, res, post.astype(np.float64), comb.astype(np.float64))
    assert_f32_chain_close(out, ref, post_f32s_scale(x, res, post, comb), what)


@pytest.mark.parametrize("T,H", [(1, 1), (3, 5), (16, 256), (37, 1000), (64, 4096), (9, 7168), (21, 7170)])
def test_post_f32_matches_oracle(T, H):
    case = _post_case(T, H, cfg=850 + H % 71)
    x, res, post, comb = case
    out = _mhc().mhc_post_f32(to_dev_bf16(x), to_dev_f32(res), to_dev_f32(post), to_dev_f32(comb))
    torch.cuda.synchronize()
    _check_post(f32_of(out), case, f"post f32 T={T} H={H}")


def test_post_f32_in_place_scalar_path_and_identity():
    mhc = _mhc()
    case = _post_case(48, 2048, cfg=860)
    x, res, post, comb = case
    a = mhc.mhc_post_f32(to_dev_bf16(x), to_dev_f32(res), to_dev_f32(post), to_dev_f32(comb))
    r = to_dev_f32(res)
    b = mhc.mhc_post_f32(to_dev_bf16(x), r, to_dev_f32(post), to_dev_f32(comb), out=r)
    rm = _misaligned_f32(res)
    c = mhc.mhc_post_f32(to_dev_bf16(x), rm, to_dev_f32(post), to_dev_f32(comb), out=rm)
    torch.cuda.synchronize()
    assert b.data_ptr() == r.data_ptr()
    assert np.array_equal(f32_of(a), f32_of(b))
    assert np.array_equal(f32_of(a), f32_of(c))
    _check_post(f32_of(a), case, "post f32 in place")
    eye = np.broadcast_to(np.eye(HC, dtype=np.float32), (48, HC, HC)).copy()
    d = mhc.mhc_post_f32(to_dev_bf16(x), to_dev_f32(res), torch.zeros(48, HC, device="cuda"), to_dev_f32(eye))
    torch.cuda.synchronize()
    assert np.array_equal(f32_of(d), res)


def test_post_f32_full_size_h7168_all_tokens():
    """T = 8192, H = 7168: every token, the oracle over token chunks on threads."""
    from concurrent.futures import ThreadPoolExecutor

    from tests._helpers import oracle_threads
    mhc = _mhc()
    T, H = 8192, 7168
    case = _post_case(T, H, cfg=861)
    x, res, post, comb = case
    out = f32_of(mhc.mhc_post_f32(to_dev_bf16(x), to_dev_f32(res), to_dev_f32(post), to_dev_f32(comb)))

    def one(t0):
        sl = slice(t0, min(T, t0 + 256))
        _check_post(out[sl], (x[sl], res[sl], post[sl], comb[sl]), f"post f32 T=8192 H=7168 [{t0}:]")

    with ThreadPoolExecutor(oracle_threads()) as ex:
        list(ex.map(one, range(0, T, 256)))


# ---------------------------------------------------------------- model entry and exit

@pytest.mark.parametrize("T,H", [(1, 1), (7, 33), (16, 256), (50, 7168), (3, 1002)])
def test_expand_and_head_mean_f32(T, H):
    mhc = _mhc()
    inp = layer_inputs_f32s(T, H, cfg=870 + H % 13)
    s = mhc.mhc_expand_f32(to_dev_bf16(inp.x))
    torch.cuda.synchronize()
    assert np.array_equal(f32_of(s), oracle.expand_f32s(inp.x))
    y = mhc.mhc_head_mean_f32(to_dev_f32(inp.res))
    torch.cuda.synchronize()
    assert_bf16_close(bits_of(y), oracle.head_mean_f32s(inp.res), f"head_mean f32 T={T} H={H}")
    assert np.array_equal(bits_of(mhc.mhc_head_mean_f32(s)), inp.x)  # the mean of 4 copies is the row


def test_layer_expand_pre_post_f32_all_tokens():
    """Model entry onto fp32 streams, then one sublayer: pre-map, the sublayer output x, and
    the post-map writing the new fp32 streams in place; every token."""
    mhc = _mhc()
    T, H = 1024, 4096
    inp = layer_inputs_f32s(T, H, cfg=880)
    hidden = layer_inputs_f32s(T, H, cfg=881).x
    streams = mhc.mhc_expand_f32(to_dev_bf16(hidden))
    torch.cuda.synchronize()
    inp.res = f32_of(streams)
    assert np.array_equal(inp.res, oracle.expand_f32s(hidden))
    y, post, comb, pre = mhc.mhc_pre_fused_f32(streams, to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale),
                                               to_dev_f32(inp.hc_base), return_pre=True)
    out = mhc.mhc_post_f32(to_dev_bf16(inp.x), streams, post, comb, out=streams)
    torch.cuda.synchronize()
    check_pre_all_tokens(inp, (bits_of(y), f32_of(post), f32_of(comb), f32_of(pre)), "layer f32",
                         x=inp.x, out=f32_of(out))
