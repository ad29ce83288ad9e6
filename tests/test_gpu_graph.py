"""The forward call replayed from a captured HIP graph gives the eager result
bit for bit, on every replay, with other eager work and synchronizations in
between (the path records no memset node: its flags word is cleared by the
routing kernel)."""
import numpy as np
import pytest

from oracle import formats
from weight_quantized_moe_amd import synth

from gpu_helpers import GpuLayer, dev, log, random_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_quantized_moe_amd import load_library
    load_library()


@pytest.mark.parametrize("fmt,T", [(formats.INT4, 1), (formats.INT4, 64), (formats.FP8, 8),
                                   (formats.NVFP4, 700), (formats.FP8, 2048)])
def test_graph_replays_match_eager(fmt, T):
    import torch
    log(f"[graph] fmt={fmt} T={T}")
    E, H, I, K = 128, 2048, 768, 8
    g = GpuLayer(*random_layer(fmt, 77, E, H, I), K)
    lay = g.layer
    lg = dev(synth.router_logits(9, 0, T, E))
    x = dev(synth.hidden_bf16(9, 0, T, H).view(np.int16)).view(torch.bfloat16)
    res = dev(synth.residual_bf16(9, 0, T, H).view(np.int16)).view(torch.bfloat16)
    lg2 = dev(synth.router_logits(9, 1, T, E))
    x2 = dev(synth.hidden_bf16(9, 1, T, H).view(np.int16)).view(torch.bfloat16)
    ws = lay.workspace(T)
    ws2 = lay.workspace(T)
    ref = lay.forward(lg, x, residual=res, workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lay.forward(lg, x, residual=res, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lay.forward(lg, x, residual=res, out=out, workspace=ws)
    for rep in range(4):
        out.fill_(0)
        other = lay.forward(lg2, x2, workspace=ws2)     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        assert not lay.check(ws)
        del other
