"""GPU parity of the pre-map's one-read form (a group of 32 workgroups per XCD splitting K,
16-token steps held in LDS, partial sums exchanged through L2).  The library takes this form
for 16-byte rows with 1024 < H <= 8192 and T >= 1024; these shapes span every slice width
(2 to 8 waves per workgroup), ragged token counts (a short last step, groups with one step
fewer than others) and H off the 32-wide blocks.  Every token is compared with the fp64
oracle at the stated tolerances (fp32 mixes 1e-5, bf16 outputs 2^-7 |ref| + 1e-3).

The exchange records carry tags naming the call and the step, so a workspace holding
another call's records (or garbage) must not change a result: the stale-workspace and
graph-replay cases check that."""
import numpy as np
import pytest

import oracle
from mhc_inputs import HC, bf16_bits_to_f32, f32_to_bf16_bits, layer_inputs
from tests._helpers import (assert_bf16_close, assert_f32_close, bits_of, check_pre_all_tokens, f32_of, to_dev_bf16,
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


def _run(inp, workspace=None, **kw):
    mhc = _mhc()
    p = dict(inp.params)
    p.update(kw)
    y, post, comb, pre = mhc.mhc_pre_fused(
        to_dev_bf16(inp.res), to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base),
        rms_eps=p["rms_eps"], pre_eps=p["pre_eps"], sinkhorn_eps=p["sinkhorn_eps"], post_mult=p["post_mult"],
        num_iters=p["num_iters"], return_pre=True, workspace=workspace)
    torch.cuda.synchronize()
    return bits_of(y), f32_of(post), f32_of(comb), f32_of(pre)


# (T, H): waves per workgroup W = ceil(ceil(H / 32) / 32) from 2 to 8; T = 1024 (8 steps per
# group), and ragged T (a short last step; groups 0..k with one step more than the rest)
COOP_SHAPES = [(1024, 2048), (1037, 1056), (1100, 2080), (1031, 4096), (1500, 4104), (1029, 6144),
               (1041, 7168), (1027, 7200), (1033, 8192), (2047, 5000), (1024, 7168)]


@pytest.mark.parametrize("T,H", COOP_SHAPES)
def test_coop_matches_oracle_every_token(T, H):
    inp = layer_inputs(T, H, cfg=600 + (T * 3 + H) % 97)
    check_pre_all_tokens(inp, _run(inp), f"coop T={T} H={H}")


@pytest.mark.parametrize("kw", [dict(post_mult=2.0), dict(num_iters=1), dict(num_iters=3),
                                dict(rms_eps=1e-2, pre_eps=1e-3, sinkhorn_eps=1e-3)])
def test_coop_parameters(kw):
    inp = layer_inputs(1040, 4096, cfg=640)
    check_pre_all_tokens(inp, _run(inp, **kw), f"coop {kw}", params=kw)


def test_coop_scale_vectors_and_base():
    inp = layer_inputs(1030, 3072, cfg=641, scale=(0.5, 2.0, 3.0), base_std=1.0)
    check_pre_all_tokens(inp, _run(inp), "coop scales")


def test_coop_bf16_weights():
    """mhc_pre_fused_bf16 on the one-read form: bf16 weights widen exactly to fp32."""
    mhc = _mhc()
    inp = layer_inputs(1100, 7168, cfg=642)
    fn_bits = f32_to_bf16_bits(inp.hc_fn)
    y, post, comb, pre = mhc.mhc_pre_fused_bf16(to_dev_bf16(inp.res), to_dev_bf16(fn_bits),
                                                to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base),
                                                return_pre=True)
    torch.cuda.synchronize()
    inp.hc_fn = bf16_bits_to_f32(fn_bits)
    check_pre_all_tokens(inp, (bits_of(y), f32_of(post), f32_of(comb), f32_of(pre)), "coop bf16 weights")


def test_coop_weighted_head():
    """mhc_head (the pre group alone) on the one-read form."""
    mhc = _mhc()
    inp = layer_inputs(1030, 4096, cfg=643)
    fn, sc, base = inp.hc_fn[:HC].copy(), np.array([1.3], np.float32), inp.hc_base[:HC].copy()
    y, pre = mhc.mhc_head(to_dev_bf16(inp.res), to_dev_f32(fn), to_dev_f32(sc), to_dev_f32(base), return_pre=True)
    torch.cuda.synchronize()
    ref = oracle.head(inp.res, fn, sc, base)
    assert_f32_close(f32_of(pre), ref["pre"], "coop head pre")
    assert_bf16_close(bits_of(y), ref["y"], "coop head y")


def test_coop_stale_and_garbage_workspace():
    """One workspace through a garbage fill (0xFF), a call on other inputs, and a call at
    another H (another record layout): every result still matches its own oracle."""
    mhc = _mhc()
    T, H = 1100, 4096
    need = max(mhc.mhc_pre_fused_workspace_bytes(T, H), mhc.mhc_pre_fused_workspace_bytes(T, 7168))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    a = layer_inputs(T, H, cfg=650)
    check_pre_all_tokens(a, _run(a, workspace=ws), "garbage workspace")
    b = layer_inputs(T, H, cfg=651)
    check_pre_all_tokens(b, _run(b, workspace=ws), "workspace after another call")
    c = layer_inputs(T, 7168, cfg=652)
    _run(c, workspace=ws)
    d = layer_inputs(T, H, cfg=653)
    check_pre_all_tokens(d, _run(d, workspace=ws), "workspace after another H")


def test_coop_deterministic():
    inp = layer_inputs(2000, 7168, cfg=654)
    a, b = _run(inp), _run(inp)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_coop_graph_replays_with_new_inputs():
    """A captured pre-map replayed on new stream contents each time: every replay equals an eager
    call on the same contents bit for bit (the tags differ per replay, so records left by the
    previous replay are never taken for this one's)."""
    mhc = _mhc()
    T, H = 1031, 4096
    inp = layer_inputs(T, H, cfg=660)
    res = to_dev_bf16(inp.res)
    fn, sc, base = to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base)
    ws = torch.empty(mhc.mhc_pre_fused_workspace_bytes(T, H), dtype=torch.uint8, device="cuda")
    y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    post = torch.empty(T, 4, device="cuda")
    comb = torch.empty(T, 4, 4, device="cuda")

    def step():
        mhc.mhc_pre_fused(res, fn, sc, base, y=y, post=post, comb=comb, workspace=ws)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        nxt = layer_inputs(T, H, cfg=661 + rep)
        res.copy_(to_dev_bf16(nxt.res))
        for t in (y, post, comb):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (bits_of(y), f32_of(post), f32_of(comb))
        ey, epost, ecomb = mhc.mhc_pre_fused(res, fn, sc, base)
        torch.cuda.synchronize()
        for u, v, name in zip(got, (bits_of(ey), f32_of(epost), f32_of(ecomb)), ("y", "post", "comb")):
            assert np.array_equal(u, v), f"replay {rep} {name}"
        inp.res = nxt.res
        check_pre_all_tokens(inp, got + (None,), f"replay {rep}")


def test_coop_missing_records_give_nan_not_a_hang():
    """The exchange's failure path, forced from the host: with a tag skew every record looks
    missing, so after the (here 2) reloads every step's outputs are NaN and the call still
    returns; with the hooks reset the same call is correct again."""
    mhc = _mhc()
    inp = layer_inputs(1100, 2048, cfg=670)
    try:
        mhc.set_exchange_test_hooks(max_retry=2, tag_skew=0x5A5A5A5A)
        y, post, comb, pre = _run(inp)
    finally:
        mhc.set_exchange_test_hooks()
    assert np.isnan(bf16_bits_to_f32(y)).all()
    assert np.isnan(post).all() and np.isnan(comb).all() and np.isnan(pre).all()
    check_pre_all_tokens(inp, _run(inp), "coop after the hooks are reset")


def test_post_pre_missing_records_keep_out_and_give_nan():
    """The same for mhc_post_pre_fused: the post-map's out does not depend on the exchange
    and stays exact; the pre-map's outputs are NaN."""
    mhc = _mhc()
    inp = layer_inputs(1100, 2048, cfg=671)
    x = to_dev_bf16(inp.x)
    res = to_dev_bf16(inp.res)
    post = torch.rand(1100, HC, device="cuda")
    comb = torch.full((1100, HC, HC), 0.25, device="cuda")
    fn, sc, base = to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base)
    try:
        mhc.set_exchange_test_hooks(max_retry=2, tag_skew=1)
        out, y, pn, cn = mhc.mhc_post_pre_fused(x, res, post, comb, fn, sc, base)
        torch.cuda.synchronize()
    finally:
        mhc.set_exchange_test_hooks()
    ref = mhc.mhc_post(x, res, post, comb)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out), bits_of(ref))
    assert np.isnan(bf16_bits_to_f32(bits_of(y))).all()
    assert np.isnan(f32_of(pn)).all() and np.isnan(f32_of(cn)).all()
