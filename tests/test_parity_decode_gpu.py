"""GPU parity of the pre-map's small-batch form: one launch for 1 <= T <= 192 (16-byte rows,
H <= 8192), a group of 32 workgroups per XCD splitting K over the group's ceil(T / 8)
tokens, the partial sums exchanged through the XCD's L2, the weights read as given.

The shapes span one to 24 tokens per group (one to six projection passes), groups left
without tokens (T < 8 and ragged T), slices that H leaves partly or wholly empty (H not a
multiple of 256, H below 256) and the widest slice (H = 8192).  Every token is compared with
the fp64 oracle at the stated tolerances (fp32 mixes 1e-5, bf16 outputs 2^-7 |ref| + 1e-3).
The exchange records carry tags naming the call and the group, so a workspace holding other
records (or garbage) must not change a result, and the weight split that
mhc_pre_split_weights stored in front of the records must survive these calls."""
import numpy as np
import pytest

import oracle
from mhc_inputs import HC, bf16_bits_to_f32, f32_to_bf16_bits, layer_inputs
from tests._helpers import assert_bf16_close, assert_f32_close, bits_of, check_pre_all_tokens, f32_of, to_dev_bf16, to_dev_f32

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


# (T, H): tokens per group ceil(T / 8) from 1 to 24; slice width 8 ceil(H / 256) from 8 to 256
DECODE_SHAPES = [(1, 7168), (2, 4096), (3, 7168), (7, 2048), (8, 7168), (9, 1024), (16, 4096), (17, 7200),
                 (24, 8192), (31, 2056), (32, 7168), (33, 6144), (40, 7168), (57, 3000), (63, 8192), (64, 7168),
                 (32, 8), (5, 64), (64, 248), (12, 520), (65, 7168), (100, 4096), (128, 7168), (131, 1000),
                 (150, 2056), (185, 7200), (192, 8192), (192, 7168), (192, 8)]


@pytest.mark.parametrize("T,H", DECODE_SHAPES)
def test_decode_matches_oracle_every_token(T, H):
    inp = layer_inputs(T, H, cfg=700 + (T * 7 + H) % 89)
    check_pre_all_tokens(inp, _run(inp), f"decode T={T} H={H}")


@pytest.mark.parametrize("kw", [dict(post_mult=2.0), dict(num_iters=1), dict(num_iters=3),
                                dict(rms_eps=1e-2, pre_eps=1e-3, sinkhorn_eps=1e-3)])
def test_decode_parameters(kw):
    inp = layer_inputs(32, 4096, cfg=740)
    check_pre_all_tokens(inp, _run(inp, **kw), f"decode {kw}", params=kw)


def test_decode_scale_vectors_and_base():
    inp = layer_inputs(29, 3072, cfg=741, scale=(0.5, 2.0, 3.0), base_std=1.0)
    check_pre_all_tokens(inp, _run(inp), "decode scales")


@pytest.mark.parametrize("T", [1, 32, 64, 192])
def test_decode_bf16_weights(T):
    """mhc_pre_fused_bf16 on the small-batch form: bf16 weights widen exactly to fp32."""
    mhc = _mhc()
    inp = layer_inputs(T, 7168, cfg=742 + T)
    fn_bits = f32_to_bf16_bits(inp.hc_fn)
    y, post, comb, pre = mhc.mhc_pre_fused_bf16(to_dev_bf16(inp.res), to_dev_bf16(fn_bits),
                                                to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base),
                                                return_pre=True)
    torch.cuda.synchronize()
    inp.hc_fn = bf16_bits_to_f32(fn_bits)
    check_pre_all_tokens(inp, (bits_of(y), f32_of(post), f32_of(comb), f32_of(pre)), f"decode bf16 weights T={T}")


@pytest.mark.parametrize("T,H", [(32, 7168), (5, 4096), (64, 1000 + 24), (160, 7168)])
def test_decode_weighted_head(T, H):
    """mhc_head (the pre group alone, 4 weight rows) on the small-batch form."""
    mhc = _mhc()
    inp = layer_inputs(T, H, cfg=743)
    fn, sc, base = inp.hc_fn[:HC].copy(), np.array([1.3], np.float32), inp.hc_base[:HC].copy()
    y, pre = mhc.mhc_head(to_dev_bf16(inp.res), to_dev_f32(fn), to_dev_f32(sc), to_dev_f32(base), return_pre=True)
    torch.cuda.synchronize()
    ref = oracle.head(inp.res, fn, sc, base)
    assert_f32_close(f32_of(pre), ref["pre"], "decode head pre")
    assert_bf16_close(bits_of(y), ref["y"], "decode head y")


def test_decode_stale_and_garbage_workspace():
    """One workspace through a garbage fill (0xFF), a call on other inputs, a call at
    another T (another record layout) and a one-read call: every result still matches its
    own oracle."""
    mhc = _mhc()
    H = 4096
    need = max(mhc.mhc_pre_fused_workspace_bytes(T, H) for T in (32, 64, 192, 1100))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    a = layer_inputs(32, H, cfg=750)
    check_pre_all_tokens(a, _run(a, workspace=ws), "garbage workspace")
    b = layer_inputs(32, H, cfg=751)
    check_pre_all_tokens(b, _run(b, workspace=ws), "workspace after another call")
    _run(layer_inputs(192, H, cfg=752), workspace=ws)
    c = layer_inputs(32, H, cfg=753)
    check_pre_all_tokens(c, _run(c, workspace=ws), "workspace after another T")
    _run(layer_inputs(1100, H, cfg=754), workspace=ws)
    d = layer_inputs(9, H, cfg=755)
    check_pre_all_tokens(d, _run(d, workspace=ws), "workspace after a one-read call")


def test_decode_keeps_the_stored_split():
    """Small-batch calls between a weight split and a two-pass presplit call on the same
    workspace leave the split intact: the two-pass call still equals mhc_pre_fused."""
    mhc = _mhc()
    H = 2048
    big = layer_inputs(300, H, cfg=756)
    small = layer_inputs(32, H, cfg=757)
    fn, sc, base = to_dev_f32(big.hc_fn), to_dev_f32(big.hc_scale), to_dev_f32(big.hc_base)
    ws = torch.empty(max(mhc.mhc_pre_fused_workspace_bytes(T, H) for T in (32, 300)), dtype=torch.uint8,
                     device="cuda")
    mhc.mhc_pre_split_weights(fn, ws)
    for _ in range(2):
        mhc.mhc_pre_fused_presplit(to_dev_bf16(small.res), fn, sc, base, workspace=ws)
    got = mhc.mhc_pre_fused_presplit(to_dev_bf16(big.res), fn, sc, base, workspace=ws, return_pre=True)
    ref = mhc.mhc_pre_fused(to_dev_bf16(big.res), fn, sc, base, return_pre=True)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)


def test_decode_deterministic():
    inp = layer_inputs(64, 7168, cfg=758)
    a, b = _run(inp), _run(inp)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_decode_graph_replays_with_new_inputs():
    """A captured small-batch pre-map replayed on new stream contents each time: every replay
    equals an eager call on the same contents bit for bit (the tags differ per replay, so
    records left by the previous replay are never taken for this one's)."""
    mhc = _mhc()
    T, H = 32, 7168
    inp = layer_inputs(T, H, cfg=760)
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
        nxt = layer_inputs(T, H, cfg=761 + rep)
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


def test_decode_missing_records_give_nan_not_a_hang():
    """The exchange's failure path, forced from the host: with a tag skew every record looks
    missing, so after the (here 2) reloads every output is NaN and the call still returns;
    with the hooks reset the same call is correct again."""
    mhc = _mhc()
    inp = layer_inputs(32, 2048, cfg=770)
    try:
        mhc.set_exchange_test_hooks(max_retry=2, tag_skew=0x5A5A5A5A)
        y, post, comb, pre = _run(inp)
    finally:
        mhc.set_exchange_test_hooks()
    assert np.isnan(bf16_bits_to_f32(y)).all()
    assert np.isnan(post).all() and np.isnan(comb).all() and np.isnan(pre).all()
    check_pre_all_tokens(inp, _run(inp), "decode after the hooks are reset")


def test_post_pre_small_batch_missing_records_keep_out_and_give_nan():
    """mhc_post_pre_fused in the small-batch form with every record made to look missing:
    the post-map's out does not depend on the exchange and stays exact, the pre-map's
    outputs are NaN, and the call returns."""
    mhc = _mhc()
    T, H = 32, 2048
    inp = layer_inputs(T, H, cfg=771)
    x, res = to_dev_bf16(inp.x), to_dev_bf16(inp.res)
    post = torch.rand(T, HC, device="cuda")
    comb = torch.full((T, HC, HC), 0.25, device="cuda")
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
    assert torch.isnan(pn).all() and torch.isnan(cn).all()
