"""GPU parity of the pre-map with its weight split done ahead of the calls
(mhc_pre_split_weights + mhc_pre_fused_presplit) against mhc_pre_fused, and of the
two-pass form's collapse that sums the slices' records itself (T <= 64 per chunk), which
batches of at most 64 tokens take when the one-launch small-batch form does not apply
(rows not 16-byte, or H > 8192).

mhc_pre_fused_presplit must equal mhc_pre_fused bit for bit on a workspace holding the
split of the same weights, over calls in a row and after a plain mhc_pre_fused call on the
same workspace; the batches at and around the small-batch bound are also checked against
the fp64 oracle on every token."""
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


def _mhc():
    import mhc_hyper_connection_amd as mhc
    return mhc


def _host(out):
    return [bits_of(o) if o.dtype == torch.bfloat16 else f32_of(o) for o in out]


@pytest.mark.parametrize("T,H", [(1, 7168), (32, 7168), (63, 4096), (64, 4096), (65, 4096), (300, 1000),
                                 (64, 8), (1100, 4096), (33, 1000), (32, 8200)])
def test_presplit_equals_pre_fused(T, H):
    mhc = _mhc()
    inp = layer_inputs(T, H, cfg=910 + H % 37)
    res, fn = to_dev_bf16(inp.res), to_dev_f32(inp.hc_fn)
    sc, base = to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base)
    ws = torch.empty(mhc.mhc_pre_fused_workspace_bytes(T, H), dtype=torch.uint8, device="cuda")
    ref = _host(mhc.mhc_pre_fused(res, fn, sc, base, return_pre=True))
    mhc.mhc_pre_split_weights(fn, ws)
    for k in range(3):  # calls in a row; the second after a plain call on the same workspace
        if k == 1:
            mhc.mhc_pre_fused(res, fn, sc, base, workspace=ws)
        got = _host(mhc.mhc_pre_fused_presplit(res, fn, sc, base, workspace=ws, return_pre=True))
        torch.cuda.synchronize()
        for g, r, name in zip(got, ref, ("y", "post", "comb", "pre")):
            assert np.array_equal(g, r), f"call {k}: {name}"
    if T <= 300:
        check_pre_all_tokens(inp, tuple(ref), f"pre T={T} H={H}")


def test_presplit_uses_the_stored_split():
    """The two-pass form (here T = 300: above the small-batch form, below the one-read
    form) reads the stored split, not hc_fn: a split of other weights gives the results of
    those weights (the documented contract for a stale split)."""
    mhc = _mhc()
    T, H = 300, 2048
    a, b = layer_inputs(T, H, cfg=930), layer_inputs(T, H, cfg=931)
    res = to_dev_bf16(a.res)
    sc, base = to_dev_f32(a.hc_scale), to_dev_f32(a.hc_base)
    fa, fb = to_dev_f32(a.hc_fn), to_dev_f32(b.hc_fn)
    ws = torch.empty(mhc.mhc_pre_fused_workspace_bytes(T, H), dtype=torch.uint8, device="cuda")
    mhc.mhc_pre_split_weights(fb, ws)
    got = _host(mhc.mhc_pre_fused_presplit(res, fa, sc, base, workspace=ws))
    ref = _host(mhc.mhc_pre_fused(res, fb, sc, base))
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)
