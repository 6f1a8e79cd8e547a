"""mhc_pre_fused_noalloc (the pre-map on the library's static scratch, for callers that cannot
allocate device memory) against mhc_pre_fused on a workspace of its own, through the C ABI.

Calls come in a row on one stream, each smaller than the one before, so every call after the
first finds the scratch holding the previous call's contents: the one-read form at the
headline size, then at a smaller H (another record layout), then the two-pass form.  Each
result must equal mhc_pre_fused's bit for bit; the smallest is also checked against the fp64
oracle at the stated tolerances."""
import ctypes

import numpy as np
import pytest

from mhc_inputs import layer_inputs
from tests._helpers import bits_of, check_pre_all_tokens, f32_of, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connection_amd as mhc
    mhc.lib()
    yield


def _both(inp):
    import mhc_hyper_connection_amd as mhc
    res = to_dev_bf16(inp.res)
    fn, sc, base = to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base)
    p = inp.params
    kw = dict(rms_eps=p["rms_eps"], pre_eps=p["pre_eps"], sinkhorn_eps=p["sinkhorn_eps"], post_mult=p["post_mult"],
              num_iters=p["num_iters"], return_pre=True)
    got = mhc.mhc_pre_fused_noalloc(res, fn, sc, base, **kw)
    torch.cuda.synchronize()
    ref = mhc.mhc_pre_fused(res, fn, sc, base, **kw)
    torch.cuda.synchronize()
    return [(bits_of(g) if g.dtype == torch.bfloat16 else f32_of(g)) for g in got], \
           [(bits_of(r) if r.dtype == torch.bfloat16 else f32_of(r)) for r in ref]


def test_noalloc_matches_pre_fused_on_calls_in_a_row():
    shapes = [(8192, 7168), (1100, 4096), (300, 1000)]
    for k, (T, H) in enumerate(shapes):
        print(f"noalloc call {k}: T={T} H={H}", flush=True)
        inp = layer_inputs(T, H, cfg=700 + k)
        got, ref = _both(inp)
        for g, r, name in zip(got, ref, ("y", "post", "comb", "pre")):
            assert np.array_equal(g, r), f"call {k} (T={T}, H={H}): {name} differs from mhc_pre_fused"
        if k == len(shapes) - 1:
            check_pre_all_tokens(inp, tuple(got), f"noalloc T={T} H={H}")


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    """A two-pass shape whose workspace exceeds the scratch: MHC_ERROR_WORKSPACE, outputs untouched."""
    import mhc_hyper_connection_amd as mhc
    T, H = 2000, 16384
    assert mhc.mhc_pre_fused_workspace_bytes(T, H) > mhc.MHC_PRE_FUSED_NOALLOC_MAX_BYTES
    res = torch.zeros(T, 4, H, dtype=torch.bfloat16, device="cuda")
    fn = torch.zeros(24, 4 * H, device="cuda")
    sc = torch.ones(3, device="cuda")
    base = torch.zeros(24, device="cuda")
    y = torch.full((T, H), 7.0, dtype=torch.bfloat16, device="cuda")
    post = torch.full((T, 4), 7.0, device="cuda")
    comb = torch.full((T, 4, 4), 7.0, device="cuda")
    st = mhc.lib().mhc_pre_fused_noalloc(
        ctypes.c_void_p(res.data_ptr()), ctypes.c_void_p(fn.data_ptr()), ctypes.c_void_p(sc.data_ptr()),
        ctypes.c_void_p(base.data_ptr()), T, H, 1e-6, 1e-6, 1e-6, 1.0, 20, ctypes.c_void_p(y.data_ptr()),
        ctypes.c_void_p(post.data_ptr()), ctypes.c_void_p(comb.data_ptr()), None,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == mhc.MHC_ERROR_WORKSPACE
    assert bool((y == 7.0).all()) and bool((post == 7.0).all()) and bool((comb == 7.0).all())
