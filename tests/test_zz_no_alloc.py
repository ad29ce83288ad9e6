"""The allocation-free forward (moe_quant_forward_noalloc, scratch in the
library's static device array) gives the workspace forward's output bit for
bit, on consecutive calls that reuse the scratch with a smaller batch, and
reports FP16 saturation through the caller's flag word."""
import numpy as np
import pytest

from oracle import formats
from weight_quantized_moe_amd import synth

from gpu_helpers import GpuLayer, dev, log, quantized_layer, random_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_quantized_moe_amd import load_library
    load_library()


def _inputs(T, E, H, seed):
    import torch
    lg = dev(synth.router_logits(seed, 0, T, E))
    x = dev(synth.hidden_bf16(seed, 0, T, H).view(np.int16)).view(torch.bfloat16)
    res = dev(synth.residual_bf16(seed, 0, T, H).view(np.int16)).view(torch.bfloat16)
    return lg, x, res


@pytest.mark.parametrize("fmt", [formats.INT4, formats.FP8, formats.NVFP4])
def test_noalloc_matches_workspace_forward(fmt):
    import torch
    E, H, I, K = 128, 2048, 768, 8
    g = GpuLayer(*random_layer(fmt, 41, E, H, I), K)
    lay = g.layer
    flag = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    # 1300 tokens (prefill path, ~63 MiB of scratch), then 64, 5 and 2 (decode
    # path; at 2 tokens the down projection writes the output itself) reusing
    # the scratch the larger call left behind
    for i, T in enumerate((1300, 64, 5, 2)):
        log(f"[noalloc] fmt={fmt} call {i}: T={T}")
        lg, x, res = _inputs(T, E, H, 50 + i)
        ref = lay.forward(lg, x, residual=res)
        got = lay.forward_noalloc(lg, x, residual=res, overflow_flag=flag)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"T={T}"
        assert int(flag.item()) == 0
        got2 = lay.forward_noalloc(lg, x)                    # no residual, no flag word
        ref2 = lay.forward(lg, x)
        torch.cuda.synchronize()
        assert torch.equal(got2.view(torch.int16), ref2.view(torch.int16)), f"T={T} no residual"


def test_noalloc_overflow_flag():
    import torch
    E, H, I, k, T = 4, 256, 128, 2, 16
    p13, p2 = quantized_layer(formats.INT4, 15, 0, E, H, I)
    p13.scale[:] = np.float16(60000.0)
    g = GpuLayer(p13, p2, k)
    lg, x, _ = _inputs(T, E, H, 15)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.layer.forward_noalloc(lg, x, overflow_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    # a following call without saturation clears it
    g2 = GpuLayer(*quantized_layer(formats.INT4, 15, 0, E, H, I), k)
    g2.layer.forward_noalloc(lg, x, overflow_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0


def test_noalloc_rejects_batches_beyond_the_scratch():
    import torch
    from weight_quantized_moe_amd import MoeQuantError
    E, H, I, K = 128, 2048, 768, 8
    g = GpuLayer(*random_layer(formats.INT4, 42, E, H, I), K)
    lg, x, _ = _inputs(2000, E, H, 60)
    with pytest.raises(MoeQuantError, match="scratch"):
        g.layer.forward_noalloc(lg, x)
    torch.cuda.synchronize()
