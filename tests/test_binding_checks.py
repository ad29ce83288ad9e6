"""The Python binding checks shapes, dtypes and contiguity before it calls
the library (runs without a GPU: every call here must raise before any launch)."""
import os

import pytest
import torch

from weight_quantized_moe_amd import binding
from weight_quantized_moe_amd.binding import Layer

E, H, I, K = 8, 256, 128, 2


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.fail("libmoe_quant.so is not built (run __graft_entry__.build())")
    binding.load_library()


def _weights(fmt):
    u8 = torch.uint8
    kd = 1 if fmt == "fp8_b128" else 2
    w13 = torch.zeros(E, 2 * I, H // kd, dtype=u8)
    w2 = torch.zeros(E, H, I // kd, dtype=u8)
    if fmt == "int4_g128":
        s13, s2 = torch.zeros(E, 2 * I, H // 128, dtype=torch.float16), torch.zeros(E, H, I // 128, dtype=torch.float16)
    elif fmt == "fp8_b128":
        s13, s2 = torch.zeros(E, 2 * I // 128, H // 128), torch.zeros(E, H // 128, I // 128)
    else:
        s13, s2 = torch.zeros(E, 2 * I, H // 16, dtype=u8), torch.zeros(E, H, I // 16, dtype=u8)
    g = (torch.ones(E), torch.ones(E)) if fmt == "nvfp4_g16" else (None, None)
    return w13, s13, w2, s2, g


@pytest.mark.parametrize("fmt", list(binding.FORMATS))
def test_layer_checks_weight_tensors(fmt):
    w13, s13, w2, s2, (g13, g2) = _weights(fmt)
    # right shapes: the only complaint left is that they are not on the GPU
    with pytest.raises(ValueError, match="GPU tensor"):
        Layer(fmt, w13, s13, w2, s2, K, w13_gscale=g13, w2_gscale=g2)
    with pytest.raises(ValueError, match="shape"):
        Layer(fmt, w13, s13[:, :-1], w2, s2, K, w13_gscale=g13, w2_gscale=g2)
    with pytest.raises(ValueError, match="dtype"):
        Layer(fmt, w13, s13.to(torch.float64), w2, s2, K, w13_gscale=g13, w2_gscale=g2)
    with pytest.raises(ValueError, match="contiguous"):
        Layer(fmt, w13.transpose(1, 2).contiguous().transpose(1, 2), s13, w2, s2, K,
              w13_gscale=g13, w2_gscale=g2)
    with pytest.raises(ValueError, match="shape"):
        Layer(fmt, w13, s13, w2[:, :, :-2], s2, K, w13_gscale=g13, w2_gscale=g2)


def _cpu_layer():
    lay = Layer.__new__(Layer)        # a layer object without a device handle
    lay._lib = binding.load_library()
    lay._h = None
    lay.fmt, lay.num_experts, lay.hidden, lay.inter, lay.top_k = "int4_g128", E, H, I, K
    lay.device = torch.device("cpu")
    lay.workspace_size = lambda t: 1 << 20
    return lay


def test_forward_checks_inputs():
    lay = _cpu_layer()
    T = 5
    lg = torch.zeros(T, E)
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        lay.forward(lg, x, workspace=ws)
    cases = [
        dict(logits=torch.zeros(T, E + 1)),                               # wrong E
        dict(logits=torch.zeros(T, E, dtype=torch.float16)),              # wrong dtype
        dict(hidden=torch.zeros(T, H + 8, dtype=torch.bfloat16)),         # wrong H
        dict(hidden=torch.zeros(H, T, dtype=torch.bfloat16).t()),         # transposed view
        dict(hidden=torch.zeros(T, H)),                                   # float32 hidden
        dict(residual=torch.zeros(T - 1, H, dtype=torch.bfloat16)),       # sliced batch
        dict(out=torch.zeros(T, H, dtype=torch.float16)),
        dict(probe={"topk_ids": torch.zeros(T, K + 1, dtype=torch.int32)}),
    ]
    for c in cases:
        args = dict(logits=lg, hidden=x, workspace=ws)
        args.update(c)
        with pytest.raises(ValueError) as ei:
            lay.forward(**args)
        assert "GPU tensor" not in str(ei.value), c


def test_forward_checks_workspace_bytes():
    """The byte count passed to the library is numel * element_size."""
    lay = _cpu_layer()
    lay.device = torch.device("cpu")
    assert binding._nbytes(torch.zeros(10, dtype=torch.float32)) == 40
    small = torch.zeros((1 << 20) // 4 - 1, dtype=torch.float32)    # 4 bytes short
    with pytest.raises(ValueError):
        lay.forward(torch.zeros(5, E), torch.zeros(5, H, dtype=torch.bfloat16), workspace=small)


def test_router_logits_checks_inputs():
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    w = torch.zeros(8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        binding.router_logits(x, w)
    with pytest.raises(ValueError, match="shape"):
        binding.router_logits(x, torch.zeros(8, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="dtype"):
        binding.router_logits(x.float(), w)
