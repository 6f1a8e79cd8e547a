"""GPU parity of mhc_post_pre_fused: the post-map of one sublayer and the next pre-map in
one call.

`out` must equal mhc_post's result bit for bit (the same products in the same order), and
every token of y, post_next, comb_next and pre_next must match the fp64 oracle's pre-map
over that `out` with the next weights, at the pre-map's tolerances (fp32 mixes 1e-5, bf16
rows 2^-7 |ref| + 1e-3).  The one-pass form runs for 16-byte rows with T >= 1024 and
1024 < H <= 8192; the shapes span its slice widths (2 to 8 waves per workgroup), ragged
token counts and H off the 32-wide blocks.  The small-batch form (16-byte rows, T <= 192,
H <= 8192) is one launch too: the post-map on each workgroup's tile, then the pre-map on
it.  The other shapes take the post-map and then the pre-map."""
import numpy as np
import pytest

import oracle
from mhc_inputs import HC, layer_inputs, normal_bf16, normal_f32, uniform_f32
from tests._helpers import assert_bf16_close, bits_of, check_pre_all_tokens, f32_of, to_dev_bf16, to_dev_f32

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


def _case(T, H, cfg):
    """Post-map inputs (x, old streams, post U(0,2), comb = Sinkhorn of N(0,1) logits) and
    the next pre-map's weights."""
    nxt = layer_inputs(T, H, cfg=cfg)
    x = normal_bf16(0, cfg + 1, "x", (T, H))
    res = normal_bf16(0, cfg + 1, "res", (T, HC, H))
    post = uniform_f32(0, cfg + 1, "post", (T, HC), 0.0, 2.0)
    comb = oracle.sinkhorn(normal_f32(0, cfg + 1, "comb_logits", (T, HC, HC), 1.0).astype(np.float64), 20,
                           1e-6).astype(np.float32)
    return nxt, x, res, post, comb


def _run(nxt, x, res, post, comb, res_dev=None, in_place=False, workspace=None, **kw):
    mhc = _mhc()
    p = dict(nxt.params)
    p.update(kw)
    r = to_dev_bf16(res) if res_dev is None else res_dev
    out, y, pn, cn, pr = mhc.mhc_post_pre_fused(
        to_dev_bf16(x), r, to_dev_f32(post), to_dev_f32(comb), to_dev_f32(nxt.hc_fn), to_dev_f32(nxt.hc_scale),
        to_dev_f32(nxt.hc_base), rms_eps=p["rms_eps"], pre_eps=p["pre_eps"], sinkhorn_eps=p["sinkhorn_eps"],
        post_mult=p["post_mult"], num_iters=p["num_iters"], out=r if in_place else None, return_pre=True,
        workspace=workspace)
    torch.cuda.synchronize()
    if in_place:
        assert out.data_ptr() == r.data_ptr()
    return bits_of(out), (bits_of(y), f32_of(pn), f32_of(cn), f32_of(pr))


def _post_ref(x, res, post, comb):
    out = _mhc().mhc_post(to_dev_bf16(x), to_dev_bf16(res), to_dev_f32(post), to_dev_f32(comb))
    torch.cuda.synchronize()
    return bits_of(out)


def _check(T, H, cfg, what, **kw):
    nxt, x, res, post, comb = _case(T, H, cfg)
    print(f"post_pre {what}: T={T} H={H}", flush=True)
    out, got = _run(nxt, x, res, post, comb, **kw)
    assert np.array_equal(out, _post_ref(x, res, post, comb)), f"{what}: out differs from mhc_post"
    assert_bf16_close(out, oracle.post(x, res, post.astype(np.float64), comb.astype(np.float64)), f"{what} out")
    nxt.res = out
    check_pre_all_tokens(nxt, got, f"post_pre {what} T={T} H={H}", params=kw or None)
    return out, got


# (T, H): one pass (waves per workgroup 2..8, ragged T, H off the 32-wide blocks)
ONE_PASS = [(1024, 2048), (1037, 1056), (1100, 2080), (1031, 4096), (1500, 4104), (1029, 6144), (1041, 7168),
            (1027, 7200), (1033, 8192), (2047, 5000)]
# post-map then pre-map: H outside both one-launch ranges, rows not 16-byte multiples, or
# between the small-batch and one-pass token counts
TWO_PASS = [(300, 1000), (900, 4096), (64, 7169), (1030, 1024), (1030, 8200), (193, 7168), (32, 8200)]
# the small-batch form with the post-map in front (one to 24 tokens per group)
SMALL = [(1, 8), (16, 256), (1, 7168), (5, 4096), (32, 7168), (33, 2056), (64, 8192), (17, 7200), (97, 1000),
         (128, 7168), (192, 4096)]


@pytest.mark.parametrize("T,H", ONE_PASS)
def test_post_pre_one_pass_every_token(T, H):
    _check(T, H, 950 + (T + H) % 37, "one pass")


@pytest.mark.parametrize("T,H", TWO_PASS)
def test_post_pre_two_pass_every_token(T, H):
    _check(T, H, 990 + (T + H) % 31, "two pass")


@pytest.mark.parametrize("T,H", SMALL)
def test_post_pre_small_batch_every_token(T, H):
    _check(T, H, 1040 + (T + H) % 29, "small batch")


def test_post_pre_small_batch_in_place_and_against_two_calls():
    """The small-batch form in place equals it out of place, and both equal mhc_post then
    mhc_pre_fused (the same kernel's pre-map on the same streams) bit for bit."""
    mhc = _mhc()
    nxt, x, res, post, comb = _case(32, 7168, 1041)
    a = _run(nxt, x, res, post, comb)
    b = _run(nxt, x, res, post, comb, in_place=True)
    assert np.array_equal(a[0], b[0])
    for u, v in zip(a[1], b[1]):
        assert np.array_equal(u, v)
    o2 = mhc.mhc_post(to_dev_bf16(x), to_dev_bf16(res), to_dev_f32(post), to_dev_f32(comb))
    y2, p2, c2, r2 = mhc.mhc_pre_fused(o2, to_dev_f32(nxt.hc_fn), to_dev_f32(nxt.hc_scale),
                                       to_dev_f32(nxt.hc_base), return_pre=True)
    torch.cuda.synchronize()
    assert np.array_equal(a[0], bits_of(o2))
    for g, r, name in zip(a[1], (bits_of(y2), f32_of(p2), f32_of(c2), f32_of(r2)), ("y", "post", "comb", "pre")):
        assert np.array_equal(g, r), name


@pytest.mark.parametrize("kw", [dict(post_mult=2.0), dict(num_iters=3), dict(rms_eps=1e-2, pre_eps=0.0)])
def test_post_pre_parameters(kw):
    _check(1100, 3072, 1020, f"params {kw}", **kw)


def test_post_pre_in_place_equals_out_of_place():
    nxt, x, res, post, comb = _case(1100, 7168, 1021)
    a = _run(nxt, x, res, post, comb)
    b = _run(nxt, x, res, post, comb, in_place=True)
    assert np.array_equal(a[0], b[0])
    for u, v in zip(a[1], b[1]):
        assert np.array_equal(u, v)


def test_post_pre_deterministic_with_garbage_workspace():
    mhc = _mhc()
    nxt, x, res, post, comb = _case(1500, 4096, 1022)
    ws = torch.full((mhc.mhc_pre_fused_workspace_bytes(1500, 4096),), 0xFF, dtype=torch.uint8, device="cuda")
    a = _run(nxt, x, res, post, comb, workspace=ws)
    b = _run(nxt, x, res, post, comb, workspace=ws)
    assert np.array_equal(a[0], b[0])
    for u, v in zip(a[1], b[1]):
        assert np.array_equal(u, v)


def test_post_pre_full_size_h7168_every_token():
    """T = 8192, H = 7168: the one-pass form at the layer's size, every token."""
    _check(8192, 7168, 1023, "full size")


def test_post_pre_matches_post_then_pre_fused():
    """Against the two calls it replaces, at a size where mhc_pre_fused also takes its
    one-read form: every output bit for bit (the same streams in LDS, the same products
    and reduction orders)."""
    mhc = _mhc()
    nxt, x, res, post, comb = _case(2048, 7168, 1024)
    out, got = _run(nxt, x, res, post, comb)
    o2 = mhc.mhc_post(to_dev_bf16(x), to_dev_bf16(res), to_dev_f32(post), to_dev_f32(comb))
    y2, p2, c2, r2 = mhc.mhc_pre_fused(o2, to_dev_f32(nxt.hc_fn), to_dev_f32(nxt.hc_scale),
                                       to_dev_f32(nxt.hc_base), return_pre=True)
    torch.cuda.synchronize()
    assert np.array_equal(out, bits_of(o2))
    for g, r, name in zip(got, (bits_of(y2), f32_of(p2), f32_of(c2), f32_of(r2)), ("y", "post", "comb", "pre")):
        assert np.array_equal(g, r), name


def test_post_pre_empty():
    mhc = _mhc()
    z = torch.zeros(0, HC, 64, dtype=torch.bfloat16, device="cuda")
    out, y, pn, cn = mhc.mhc_post_pre_fused(torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda"), z,
                                            torch.zeros(0, HC, device="cuda"), torch.zeros(0, HC, HC, device="cuda"),
                                            torch.zeros(24, 256, device="cuda"), torch.ones(3, device="cuda"),
                                            torch.zeros(24, device="cuda"))
    assert out.shape == (0, HC, 64) and y.shape == (0, 64)


def test_post_pre_graph_replays_with_new_inputs():
    """A captured call replayed on new inputs each time, in place: every replay equals an
    eager call on the same inputs bit for bit (the exchange tags differ per replay)."""
    mhc = _mhc()
    T, H = 1031, 4096
    nxt, x, res, post, comb = _case(T, H, 1030)
    xd, rd, pd, cd = to_dev_bf16(x), to_dev_bf16(res), to_dev_f32(post), to_dev_f32(comb)
    fn, sc, base = to_dev_f32(nxt.hc_fn), to_dev_f32(nxt.hc_scale), to_dev_f32(nxt.hc_base)
    ws = torch.empty(mhc.mhc_pre_fused_workspace_bytes(T, H), dtype=torch.uint8, device="cuda")
    y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    pn = torch.empty(T, HC, device="cuda")
    cn = torch.empty(T, HC, HC, device="cuda")

    def step():
        mhc.mhc_post_pre_fused(xd, rd, pd, cd, fn, sc, base, out=rd, y=y, post_next=pn, comb_next=cn, workspace=ws)

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
        _, x2, r2, p2, c2 = _case(T, H, 1031 + rep)
        xd.copy_(to_dev_bf16(x2))
        rd.copy_(to_dev_bf16(r2))
        pd.copy_(to_dev_f32(p2))
        cd.copy_(to_dev_f32(c2))
        for t in (y, pn, cn):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (bits_of(rd), bits_of(y), f32_of(pn), f32_of(cn))
        eo, ey, ep, ec = mhc.mhc_post_pre_fused(to_dev_bf16(x2), to_dev_bf16(r2), to_dev_f32(p2), to_dev_f32(c2), fn,
                                                sc, base)
        torch.cuda.synchronize()
        for u, v, name in zip(got, (bits_of(eo), bits_of(ey), f32_of(ep), f32_of(ec)), ("out", "y", "post", "comb")):
            assert np.array_equal(u, v), f"replay {rep}: {name}"
