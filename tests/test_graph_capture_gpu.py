"""The entry points under HIP graph capture: one mHC layer step (pre-map, post-map) and
the Sinkhorn, and the reverse-mode entry points, each captured once and replayed several
times, with eager work and synchronisations in between; every replay must equal the
eager result bit for bit.
The library launches only kernels on the caller's stream (no allocation, no memset,
no host synchronisation), so the step captures as it runs."""
import numpy as np
import pytest

from mhc_inputs import external_dots, layer_inputs, post_grad, pre_grads, sinkhorn_grad, sinkhorn_logits
from tests._helpers import to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connection_amd as mhc
    mhc.lib()
    yield


@pytest.mark.parametrize("T,H", [(32, 7168), (300, 1000), (1030, 4096)])
def test_layer_step_graph_replays_match_eager(T, H):
    import mhc_hyper_connection_amd as mhc
    inp = layer_inputs(T, H, cfg=700 + H % 13)
    res, x = to_dev_bf16(inp.res), to_dev_bf16(inp.x)
    fn, sc, base = to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base)
    ws = torch.empty(mhc.mhc_pre_fused_workspace_bytes(T, H), dtype=torch.uint8, device="cuda")
    y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    post = torch.empty(T, 4, device="cuda")
    comb = torch.empty(T, 4, 4, device="cuda")
    out = torch.empty_like(res)
    lg = to_dev_f32(sinkhorn_logits(4096, cfg=701))
    sk = torch.empty_like(lg)

    def step():
        mhc.mhc_pre_fused(res, fn, sc, base, y=y, post=post, comb=comb, workspace=ws)
        mhc.mhc_post(x, res, post, comb, out=out)
        mhc.mhc_sinkhorn(lg, out=sk)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (y, post, comb, out, sk)]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for t in (y, post, comb, out, sk):
            t.zero_()                     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip((y, post, comb, out, sk), eager):
            a = got.view(torch.int16) if got.dtype == torch.bfloat16 else got
            b = ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref
            assert torch.equal(a, b), f"replay {rep}"


def _replays_match(step, outputs_eager, reps=3):
    """Capture `step` (after a warm-up on the capture stream), then replay it `reps` times,
    zeroing its outputs eagerly before each replay; every replay must equal the eager
    outputs bit for bit."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for rep in range(reps):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j, (got, ref) in enumerate(zip(outs, outputs_eager)):
            a = got.view(torch.int16) if got.dtype == torch.bfloat16 else got
            b = ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref
            assert torch.equal(a, b), f"replay {rep}, output {j}"


@pytest.mark.parametrize("T,H", [(40, 1000), (300, 4096)])
def test_reverse_mode_graph_replays_match_eager(T, H):
    """mhc_pre_fused_backward, mhc_pre_from_dots_backward, mhc_post_backward and
    mhc_sinkhorn_backward in one captured step (workspaces and gradient buffers given;
    the small outputs the bindings allocate come from the graph's pool)."""
    import mhc_hyper_connection_amd as mhc
    inp = layer_inputs(T, H, cfg=710 + H % 11)
    dy, d_post, d_comb = pre_grads(T, H, cfg=711)
    res, x = to_dev_bf16(inp.res), to_dev_bf16(inp.x)
    fn, sc, base = to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base)
    dyd, dpd, dcd = to_dev_bf16(dy), to_dev_f32(d_post), to_dev_f32(d_comb)
    dots = to_dev_f32(external_dots(T, H, cfg=714)[0])
    d_out = to_dev_bf16(post_grad(T, H, cfg=712))
    _, post, comb = mhc.mhc_pre_fused(res, fn, sc, base)
    sl = to_dev_f32(sinkhorn_logits(4096, cfg=713))
    sg = to_dev_f32(sinkhorn_grad(4096, cfg=713))
    ws_f = torch.empty(mhc.mhc_pre_fused_backward_workspace_bytes(T, H), dtype=torch.uint8, device="cuda")
    ws_d = torch.empty(mhc.mhc_pre_backward_workspace_bytes(T), dtype=torch.uint8, device="cuda")
    dres1, dres2, dres3 = torch.empty_like(res), torch.empty_like(res), torch.empty_like(res)
    dx = torch.empty_like(x)
    dpost3, dcomb3 = torch.empty_like(post), torch.empty_like(comb)
    skd = torch.empty_like(sl)

    def step():
        r1 = mhc.mhc_pre_fused_backward(dyd, dpd, dcd, res, fn, sc, base, d_res=dres1, workspace=ws_f)
        r2 = mhc.mhc_pre_from_dots_backward(dyd, dpd, dcd, dots, res, sc, base, d_res=dres2, workspace=ws_d)
        mhc.mhc_post_backward(d_out, x, res, post, comb, d_x=dx, d_res=dres3, d_post=dpost3, d_comb=dcomb3)
        mhc.mhc_sinkhorn_backward(sg, sl, d_logits=skd)
        return [dres1, r1["d_hc_fn"], r1["d_hc_scale"], r1["d_hc_base"], dres2, r2["d_dot"], r2["d_hc_scale"],
                r2["d_hc_base"], dx, dres3, dpost3, dcomb3, skd]

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    _replays_match(step, eager)


@pytest.mark.parametrize("T,H", [(32, 7168), (300, 1000)])
def test_fused_sublayer_graph_replays_match_eager(T, H):
    """The steady-state sublayer step under capture: mhc_post_project (the post-map and
    the next projection), then mhc_pre_from_dots on its dots and sum of squares."""
    import mhc_hyper_connection_amd as mhc
    inp = layer_inputs(T, H, cfg=720 + H % 7)
    res, x = to_dev_bf16(inp.res), to_dev_bf16(inp.x)
    fn, sc, base = to_dev_f32(inp.hc_fn), to_dev_f32(inp.hc_scale), to_dev_f32(inp.hc_base)
    _, post0, comb0 = mhc.mhc_pre_fused(res, fn, sc, base)
    ws = torch.empty(mhc.mhc_post_project_workspace_bytes(T, H), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(res)
    dm = torch.empty(T, 24, device="cuda")
    sq = torch.empty(T, device="cuda")
    y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    post = torch.empty(T, 4, device="cuda")
    comb = torch.empty(T, 4, 4, device="cuda")
    pre = torch.empty(T, 4, device="cuda")

    def step():
        mhc.mhc_post_project(x, res, post0, comb0, fn, out=out, dot_mix=dm, sqrsum=sq, workspace=ws)
        mhc.mhc_pre_from_dots(dm, out, sc, base, sqrsum=sq, y=y, post=post, comb=comb, pre=pre, return_pre=True)
        return [out, dm, sq, y, post, comb, pre]

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    _replays_match(step, eager)
