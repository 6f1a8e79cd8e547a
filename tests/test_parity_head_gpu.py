"""GPU parity of the model entry and exit ops and of the bf16-weight pre-map against the
fp64 CPU oracle (same tolerances as the pre-map: fp32 mixes within 1e-5, bf16 outputs
within 2^-7 |ref| + 1e-3; the stream broadcast is bit-exact)."""
import numpy as np
import pytest

import oracle
from mhc_inputs import HC, bf16_bits_to_f32, f32_to_bf16_bits, layer_inputs
from tests._helpers import (assert_bf16_close, assert_f32_close, bits_of, f32_of, sample_tokens, to_dev_bf16,
                            to_dev_f32)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SHAPES = [(16, 256), (5, 64), (7, 127), (3, 1001), (37, 4096), (21, 7168), (3, 16392), (1, 1), (70, 96),
          (300, 1000), (65, 2056)]


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


@pytest.mark.parametrize("T,H", SHAPES + [(8192, 7168)])
def test_expand_bit_exact(T, H):
    inp = layer_inputs(T, H, cfg=500 + H % 71) if T * H <= 8192 * 7168 // 4 else None
    x = inp.x if inp is not None else f32_to_bf16_bits(np.random.default_rng(5).standard_normal((T, H),
                                                                                                dtype=np.float32))
    got = bits_of(_mhc().mhc_expand(to_dev_bf16(x)))
    assert np.array_equal(got, oracle.expand(x))


@pytest.mark.parametrize("T,H", SHAPES)
def test_head_mean_matches_oracle(T, H):
    inp = layer_inputs(T, H, cfg=510 + H % 71)
    got = bits_of(_mhc().mhc_head_mean(to_dev_bf16(inp.res)))
    ref = oracle.head_mean(inp.res)
    assert_bf16_close(got, ref, f"head mean T={T} H={H}")
    s = bf16_bits_to_f32(inp.res).astype(np.float64).sum(axis=1)
    exact = s.astype(np.float32).astype(np.float64) == s      # the fp32 sum holds it exactly
    assert np.array_equal(got[exact], oracle.round_bf16(ref)[exact])


def _head_case(T, H, cfg):
    inp = layer_inputs(T, H, cfg=cfg)
    return inp.res, inp.hc_fn[:HC].copy(), np.array([1.3], np.float32), inp.hc_base[:HC].copy()


@pytest.mark.parametrize("T,H", SHAPES)
def test_head_matches_oracle(T, H):
    res, fn, sc, base = _head_case(T, H, 520 + H % 71)
    y, pre = _mhc().mhc_head(to_dev_bf16(res), to_dev_f32(fn), to_dev_f32(sc), to_dev_f32(base), 1e-6, 1e-3,
                             return_pre=True)
    torch.cuda.synchronize()
    ref = oracle.head(res, fn, sc, base, 1e-6, 1e-3)
    assert_f32_close(f32_of(pre), ref["pre"], f"head pre T={T} H={H}")
    assert_bf16_close(bits_of(y), ref["y"], f"head y T={T} H={H}")


def test_head_full_size_h7168_sampled():
    T, H = 8192, 7168
    res, fn, sc, base = _head_case(T, H, 3)
    y, pre = _mhc().mhc_head(to_dev_bf16(res), to_dev_f32(fn), to_dev_f32(sc), to_dev_f32(base), return_pre=True)
    torch.cuda.synchronize()
    tok = sample_tokens(T, 48)
    ref = oracle.head(res[tok], fn, sc, base)
    assert_f32_close(f32_of(pre)[tok], ref["pre"], "head pre 8192x7168")
    assert_bf16_close(bits_of(y)[tok], ref["y"], "head y 8192x7168")


def _pre_bf16_check(inp, tokens=None):
    mhc = _mhc()
    fn16 = f32_to_bf16_bits(inp.hc_fn)
    y, post, comb, pre = mhc.mhc_pre_fused_bf16(to_dev_bf16(inp.res), to_dev_bf16(fn16), to_dev_f32(inp.hc_scale),
                                                to_dev_f32(inp.hc_base), return_pre=True)
    torch.cuda.synchronize()
    sel = slice(None) if tokens is None else tokens
    ref = oracle.pre(inp.res[sel], bf16_bits_to_f32(fn16), inp.hc_scale, inp.hc_base)
    what = f"pre bf16 weights T={inp.T} H={inp.H}"
    assert_f32_close(f32_of(pre)[sel], ref["pre"], what + " pre")
    assert_f32_close(f32_of(post)[sel], ref["post"], what + " post")
    assert_f32_close(f32_of(comb)[sel], ref["comb"], what + " comb")
    assert_bf16_close(bits_of(y)[sel], ref["y"], what + " y")


@pytest.mark.parametrize("T,H", [(16, 256), (7, 127), (300, 1000), (21, 7168), (65, 2056)])
def test_pre_fused_bf16_weights_matches_oracle(T, H):
    _pre_bf16_check(layer_inputs(T, H, cfg=530 + H % 71))


def test_pre_fused_bf16_weights_full_size_sampled():
    _pre_bf16_check(layer_inputs(8192, 7168, cfg=3), tokens=sample_tokens(8192, 48))


def test_expand_then_head_mean_round_trip_and_empty():
    mhc = _mhc()
    inp = layer_inputs(33, 4096, cfg=540)
    x = to_dev_bf16(inp.x)
    assert torch.equal(mhc.mhc_head_mean(mhc.mhc_expand(x)).view(torch.int16), x.view(torch.int16))
    e = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    assert mhc.mhc_expand(e).numel() == 0
    assert mhc.mhc_head_mean(torch.empty(0, HC, 64, dtype=torch.bfloat16, device="cuda")).numel() == 0
