"""The entry points under HIP graph capture: one mHC layer step (pre-map, post-map) and
the Sinkhorn, captured once and replayed several times, with eager work and
synchronisations in between; every replay must equal the eager result bit for bit.
The library launches only kernels on the caller's stream (no allocation, no memset,
no host synchronisation), so the step captures as it runs."""
import numpy as np
import pytest

from mhc_inputs import layer_inputs, sinkhorn_logits
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
