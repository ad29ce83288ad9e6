"""Parity of the router logits kernel (moe_quant_router_logits) with the
float64 oracle, and of the routing that consumes its logits.

Each logit is a sum of H exact products; the kernel adds them in FP32 in the
matrix units' order, so it may differ from the float64 sum by at most
gamma_H * sum_h |x_h w_h| with gamma_H = H u / (1 - H u), the standard bound
on recursive summation that every summation order meets.  u = 2^-23, twice
the FP32 unit roundoff, so the bound also holds for an adder that truncates.
The top-k then decides on the FP32 logits themselves: the routing is checked
bit-exactly against the oracle's top-k of those same logits.
"""
import numpy as np
import pytest

from oracle import moe
from weight_quantized_moe_amd import synth

from gpu_helpers import GpuLayer, check_routing, dev, log, quantized_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_quantized_moe_amd import load_library
    load_library()      # fails loudly if the HIP library is missing


def _gate(seed, E, H):
    """BF16 gate weight [E, H] ~ N(0, 0.02) (the scale of a trained router's rows)."""
    rng = np.random.default_rng(seed)
    return synth.to_bf16_bits((rng.standard_normal((E, H)) * 0.02).astype(np.float32))


def _gpu_logits(x_bits, w_bits):
    import torch
    from weight_quantized_moe_amd import router_logits
    x = dev(x_bits.view(np.int16)).view(torch.bfloat16)
    w = dev(w_bits.view(np.int16)).view(torch.bfloat16)
    out = router_logits(x, w)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(x_bits, w_bits, tag):
    got = _gpu_logits(x_bits, w_bits).astype(np.float64)
    ref = moe.router_logits(x_bits, w_bits)
    H = x_bits.shape[1]
    u = 2.0 ** -23
    gamma = H * u / (1 - H * u)
    bound = gamma * (np.abs(moe.bf16_bits_to_f64(x_bits)) @ np.abs(moe.bf16_bits_to_f64(w_bits)).T)
    err = np.abs(got - ref)
    log(f"    {tag}: max err {err.max():.3e}, max err / bound {(err / np.maximum(bound, 1e-300)).max():.3f}")
    assert np.all(err <= bound), tag
    return got


@pytest.mark.parametrize("T,H,E", [(1, 64, 1), (5, 256, 8), (37, 2048, 128), (64, 2048, 128),
                                   (100, 384, 200), (33, 512, 130), (4096, 2048, 128)])
def test_router_logits_within_fp32_bound(T, H, E):
    """Ragged token and expert tiles (T, E not multiples of 32 / 128), E < 4 and
    E not a multiple of 4 (scalar stores), and the prefill workload's shape."""
    log(f"[router] T={T} H={H} E={E}")
    x = synth.hidden_bf16(30, T, T, H)
    _check(x, _gate(31 + E, E, H), f"T={T} H={H} E={E}")


def test_router_one_hot_rows_are_exact():
    """w[e] = unit vector at column c(e): every logit is one exact product, so
    the kernel must return x[:, c(e)] bit for bit (catches transposed operands
    and index mistakes that a tolerance could hide)."""
    T, H, E = 70, 256, 40
    rng = np.random.default_rng(5)
    x = synth.hidden_bf16(32, 0, T, H)
    cols = rng.choice(H, E, replace=False)
    w = np.zeros((E, H), dtype=np.float32)
    w[np.arange(E), cols] = 1.0
    got = _gpu_logits(x, synth.to_bf16_bits(w))
    assert np.array_equal(got.astype(np.float64), moe.bf16_bits_to_f64(x)[:, cols])


def test_router_feeds_the_layer():
    """Router logits from the kernel drive a prefill layer: routing bit-exact
    against the oracle's top-k of the same FP32 logits."""
    E, H, I, k, T = 16, 512, 256, 4, 300
    p13, p2 = quantized_layer("fp8_b128", 33, 0, E, H, I)
    g = GpuLayer(p13, p2, k)
    x = synth.hidden_bf16(33, 0, T, H)
    lg = _check(x, _gate(34, E, H), "layer router").astype(np.float32)
    out, pr, ovf = g.run(lg, x, probe=True)
    check_routing(pr, lg, k, E)
    assert not ovf


# ------------------------------------------------------------ router fused with the top-k

def _fused(g, x_bits, w_bits, res_bits=None):
    """moe_quant_forward_with_router with every probe output."""
    import torch
    lay = g.layer
    T, E, k, I = x_bits.shape[0], lay.num_experts, lay.top_k, lay.inter
    x = dev(x_bits.view(np.int16)).view(torch.bfloat16)
    w = dev(w_bits.view(np.int16)).view(torch.bfloat16)
    res = dev(res_bits.view(np.int16)).view(torch.bfloat16) if res_bits is not None else None
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    pr = dict(topk_ids=torch.empty((T, k), dtype=torch.int32, device="cuda"),
              topk_w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
              expert_offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
              sorted_token_ids=torch.empty(T * k, dtype=torch.int32, device="cuda"),
              inv_pos=torch.empty(T * k, dtype=torch.int32, device="cuda"))
    ws = lay.workspace(T)
    out = lay.forward_with_router(w, x, residual=res, workspace=ws, logits_out=lg, probe=pr)
    torch.cuda.synchronize()
    assert not lay.check(ws)
    return (out.view(torch.int16).cpu().numpy().view(np.uint16), lg.cpu().numpy(),
            {n: v.cpu().numpy() for n, v in pr.items()})


def _check_fused(g, x, w, tag, res=None):
    from gpu_helpers import ATOL_MAX, RTOL_L2, errors
    out, lg, pr = _fused(g, x, w, res)
    # the logits the top-k decided on: within the FP32 summation bound
    H = x.shape[1]
    u = 2.0 ** -23
    gamma = H * u / (1 - H * u)
    ref_lg = moe.router_logits(x, w)
    bound = gamma * (np.abs(moe.bf16_bits_to_f64(x)) @ np.abs(moe.bf16_bits_to_f64(w)).T)
    assert np.all(np.abs(lg.astype(np.float64) - ref_lg) <= bound), tag
    # routing and grouping bit-exact against the oracle's top-k of those logits
    check_routing(pr, lg, g.top_k, g.layer.num_experts)
    y, _, _ = moe.moe_forward(g.oracle, lg, x, res)
    rel, mx = errors(out, y)
    log(f"    {tag}: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= RTOL_L2 and mx <= ATOL_MAX, tag
    return out, lg


@pytest.mark.parametrize("T,E,k,fmt", [
    # below 4096 tokens: router logits kernel into the workspace, then routing
    (1, 128, 8, "int4_g128"), (37, 128, 8, "fp8_b128"), (64, 128, 8, "nvfp4_g16"),
    (300, 8, 2, "int4_g128"), (700, 200, 6, "fp8_b128"),
    # the fused router + top-k kernel: 16-token blocks up to 8192 tokens, 32
    # above; ragged token blocks and expert groups, E from 8 to 256
    (4096, 128, 8, "int4_g128"), (4099, 200, 6, "fp8_b128"), (4111, 40, 5, "nvfp4_g16"),
    (5000, 8, 2, "int4_g128"), (8193, 256, 8, "nvfp4_g16"), (9000, 32, 4, "fp8_b128")])
def test_forward_with_router(T, E, k, fmt):
    """Routing from the gate's weight on the decode (T*k <= 16 E) and the
    prefill paths, with ragged token blocks (T not a multiple of 16 or 32) and
    expert groups (E not a multiple of 32)."""
    log(f"[router+topk] T={T} E={E} k={k} {fmt}")
    H, I = 256, 128
    g = GpuLayer(*quantized_layer(fmt, 35, E, E, H, I), k)
    x = synth.hidden_bf16(36, T, T, H)
    res = synth.residual_bf16(36, T, T, H) if T % 2 else None
    out, lg = _check_fused(g, x, _gate(37 + E, E, H), f"T={T} E={E}", res)
    out2, lg2, _ = _fused(g, x, _gate(37 + E, E, H), res)
    assert np.array_equal(out, out2) and np.array_equal(lg, lg2), "repeat run differs"


def test_forward_with_router_full_shape():
    """The prefill workload's shape (hidden 2048, intermediate 768, 128
    experts, top-8, FP8, 4096 tokens), every token compared."""
    log("[router+topk] full shape T=4096 fp8")
    E, H, I, k, T = 128, 2048, 768, 8, 4096
    g = GpuLayer(*quantized_layer("fp8_b128", 3, 0, E, H, I), k)
    _check_fused(g, synth.hidden_bf16(38, 0, T, H), _gate(39, E, H), "full shape")
