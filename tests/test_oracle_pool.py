"""The pooled evaluation the full-size GPU tests use (oracle_forward_pool: the
oracle's route, permute and combine in the main process, its dequantize +
SwiGLU expert step in worker processes) gives moe.moe_forward's result."""
import numpy as np

from oracle import formats, moe
from weight_quantized_moe_amd import synth

from gpu_helpers import oracle_forward_pool, quantize_expert_job, quantized_layer, spawn_pool


def test_pooled_forward_matches_moe_forward():
    E, H, I, k, T = 8, 256, 128, 2, 50
    for fmt in formats.FORMATS:
        p13, p2 = quantized_layer(fmt, 1, 0, E, H, I)
        lg = synth.router_logits(1, 0, T, E)
        x = synth.hidden_bf16(1, 0, T, H)
        ref, ids, w = moe.moe_forward(moe.Layer(p13, p2, k), lg, x)
        with spawn_pool(2) as pool:
            got, ids2, w2 = oracle_forward_pool(pool, p13, p2, k, lg, x)
            # the stack test's per-expert quantize job gives the same packed bytes
            q = pool.submit(quantize_expert_job, (fmt, 1, 0, 3, H, I)).result()
        assert np.array_equal(ids, ids2) and np.array_equal(w, w2)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)
        assert np.array_equal(q[0][0], p13.w[3]) and np.array_equal(q[1][1], p2.scale[3])


def test_pooled_w4a4_matches_the_w4a4_oracle():
    """oracle_w4a4_pool gives moe_forward_w4a4's output, the intermediate of
    intermediate_w4a4, and down_from_values' teacher-forced output."""
    from oracle import w4a4
    from gpu_helpers import oracle_w4a4_pool
    E, H, I, k, T = 8, 256, 128, 2, 40
    p13, p2 = quantized_layer(formats.NVFP4, 2, 0, E, H, I)
    layer = moe.Layer(p13, p2, k)
    lg = synth.router_logits(2, 0, T, E)
    x = synth.hidden_bf16(2, 0, T, H)
    gx, gh = 500.0, 30000.0
    ref, _, _ = w4a4.moe_forward_w4a4(layer, lg, x, gx, gh)
    h_ref = w4a4.intermediate_w4a4(layer, lg, x, gx)
    hf = np.random.default_rng(0).standard_normal((T * k, I))
    with spawn_pool(2) as pool:
        got, forced, h32 = oracle_w4a4_pool(pool, p13, p2, k, lg, x, gx, gh, hf)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)
    assert np.array_equal(h32, h_ref)
    np.testing.assert_allclose(forced, w4a4.down_from_values(layer, lg, hf), rtol=1e-12, atol=1e-15)
