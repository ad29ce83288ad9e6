"""Parity at the full Clef-Omni-shaped workloads (hidden 2048, expert
intermediate 768, 128 experts, top-8), in the launch configuration bench.py
times.  Routing and grouping are compared bit-exactly on every token; layer
outputs on every token for the decode batches and on sampled tokens (the
oracle computes each token independently) for the large batches."""
import numpy as np
import pytest

from oracle import formats, moe
from weight_quantized_moe_amd import synth

from gpu_helpers import (ATOL_MAX, RTOL_L2, GpuLayer, check_routing, errors, log,
                         quantized_layer)

pytestmark = pytest.mark.gpu

H, I, E, K = 2048, 768, 128, 8
_LAYERS = {}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_quantized_moe_amd import load_library
    load_library()


def _layer(name):
    if name not in _LAYERS:
        w = synth.WORKLOADS[name]
        log(f"  quantizing {name} ({w.fmt}) ...")
        p13, p2 = quantized_layer(w.fmt, w.wid, 0, E, H, I)
        _LAYERS[name] = GpuLayer(p13, p2, K)
    return _LAYERS[name]


def _sample(T, n=32, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, n - 2, replace=False)]))


@pytest.mark.parametrize("T", [1, 8, 64])
def test_decode_int4(T):
    log(f"[decode_int4] T={T}")
    w = synth.WORKLOADS["decode_int4"]
    g = _layer("decode_int4")
    lg = synth.router_logits(w.wid, 0, T, E, w.logits)
    x = synth.hidden_bf16(w.wid, 0, T, H)
    out, pr, ovf = g.run(lg, x, probe=True)
    check_routing(pr, lg, K, E)
    assert not ovf
    y, _, _ = moe.moe_forward(g.oracle, lg, x)
    rel, mx = errors(out, y)
    log(f"    rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= RTOL_L2 and mx <= ATOL_MAX


@pytest.mark.parametrize("name,T", [("prefill_fp8", 4096), ("nvfp4_zipf", 16384)])
def test_large_batches(name, T):
    log(f"[{name}] T={T}")
    w = synth.WORKLOADS[name]
    g = _layer(name)
    lg = synth.router_logits(w.wid, 0, T, E, w.logits)
    x = synth.hidden_bf16(w.wid, 0, T, H)
    out, pr, ovf = g.run(lg, x, probe=True)
    check_routing(pr, lg, K, E)
    assert not ovf
    tok = _sample(T)
    y, _, _ = moe.moe_forward(g.oracle, lg, x, tokens=tok)
    rel, mx = errors(out[tok], y)
    log(f"    sampled {len(tok)} tokens: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= RTOL_L2 and mx <= ATOL_MAX


@pytest.mark.parametrize("T", [64, 2048])
def test_stack48_teacher_forced(T):
    """48 layers (0-23 FP8, 24-47 INT4) chained with residual adds on the GPU:
    x_{l+1} = bf16(x_l + moe_l(n(x_l))), n = RMS normalisation with unit gain.
    The model normalises the residual stream before each expert block; without
    it the SwiGLU's quadratic gain makes the stream grow without bound.  At the
    checked layers the MoE output on that layer's own GPU input is compared
    with the oracle (teacher forcing)."""
    import torch
    from weight_quantized_moe_amd import Layer
    log(f"[stack48] T={T}")
    w = synth.WORKLOADS["stack48"]
    check_layers = (0, 23, 24, 47)
    x = synth.hidden_bf16(w.wid, 0, T, H)
    xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    tok = np.arange(T) if T <= 64 else _sample(T)
    ws = None
    worst = 0.0
    for layer in range(w.layers):
        fmt = synth.stack_layer_format(layer)
        t13 = synth.random_packed_torch(fmt, E, 2 * I, H, 5000 + 2 * layer)
        t2 = synth.random_packed_torch(fmt, E, H, I, 5001 + 2 * layer)
        lay = Layer(fmt, t13[0], t13[1], t2[0], t2[1], K, w13_gscale=t13[2], w2_gscale=t2[2])
        if ws is None:
            ws = lay.workspace(T)
        lg = synth.router_logits(w.wid, layer, T, E)
        lgt = torch.from_numpy(lg).cuda()
        xf = xt.float()
        xn = (xf * torch.rsqrt(xf.square().mean(dim=1, keepdim=True) + 1e-6)).to(torch.bfloat16)
        if layer in check_layers:
            y_gpu = lay.forward(lgt, xn, workspace=ws)
            torch.cuda.synchronize()
            assert not lay.check(ws)
            x_in = xn.view(torch.int16).cpu().numpy().view(np.uint16)
            cpu = lambda a: None if a is None else a.cpu().numpy()  # noqa: E731
            p13 = formats.Packed(fmt, *map(cpu, t13), 2 * I, H)
            p2 = formats.Packed(fmt, *map(cpu, t2), H, I)
            y, _, _ = moe.moe_forward(moe.Layer(p13, p2, K), lg, x_in, tokens=tok)
            o = y_gpu.view(torch.int16).cpu().numpy().view(np.uint16)
            rel, mx = errors(o[tok], y)
            log(f"    layer {layer} ({fmt}): rel_l2={rel:.3e} max_abs={mx:.3e}")
            assert rel <= RTOL_L2 and mx <= ATOL_MAX
            worst = max(worst, rel)
        xt = lay.forward(lgt, xn, residual=xt, workspace=ws)
        del lay, t13, t2
    torch.cuda.synchronize()
    assert torch.isfinite(xt.float()).all()
    log(f"    final residual stream rms={xt.float().square().mean().sqrt().item():.3f}")
    log(f"    worst checked layer rel_l2={worst:.3e}")
