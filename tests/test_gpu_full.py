"""Parity at the full Clef-Omni-shaped workloads (hidden 2048, expert
intermediate 768, 128 experts, top-8), in the launch configuration bench.py
times.  Routing and grouping are compared bit-exactly and the layer output
element by element on every token: relative L2 over the whole [T, H] output
and the largest absolute error, against the float64 oracle."""
import numpy as np
import pytest

from oracle import moe
from weight_quantized_moe_amd import synth

from gpu_helpers import (ATOL_MAX, RTOL_L2, GpuLayer, check_routing, errors, log,
                         oracle_forward_pool, quantized_layer, spawn_pool)

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


@pytest.fixture(scope="module")
def pool():
    p = spawn_pool()
    yield p
    p.shutdown()


def _layer(name):
    if name not in _LAYERS:
        w = synth.WORKLOADS[name]
        log(f"  quantizing {name} ({w.fmt}) ...")
        p13, p2 = quantized_layer(w.fmt, w.wid, 0, E, H, I)
        _LAYERS[name] = GpuLayer(p13, p2, K)
    return _LAYERS[name]


@pytest.mark.parametrize("T", [1, 8, 64, 128, 256])
def test_decode_int4(T):
    """Decode batches of the INT4 layer; T = 64, 128 and 256 (4, 8 and 16 rows
    per expert) run the streaming gate/up GEMM."""
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


@pytest.mark.parametrize("name,T", [("prefill_fp8", 4096), ("nvfp4_zipf", 16384),
                                    ("decode_int4", 4096)])
def test_large_batches(name, T, pool):
    """Every token of the batch: rel-L2 over the whole [T, H] output."""
    log(f"[{name}] T={T}")
    w = synth.WORKLOADS[name]
    g = _layer(name)
    lg = synth.router_logits(w.wid, 0, T, E, w.logits)
    x = synth.hidden_bf16(w.wid, 0, T, H)
    out, pr, ovf = g.run(lg, x, probe=True)
    check_routing(pr, lg, K, E)
    assert not ovf
    y, _, _ = oracle_forward_pool(pool, g.p13, g.p2, K, lg, x)
    rel, mx = errors(out, y)
    row = np.linalg.norm(moe.bf16_bits_to_f64(out) - y, axis=1) / np.maximum(
        np.linalg.norm(y, axis=1), 1e-300)
    log(f"    all {T} tokens: rel_l2={rel:.3e} max_abs={mx:.3e} (max row rel_l2 {row.max():.3e})")
    assert rel <= RTOL_L2 and mx <= ATOL_MAX
