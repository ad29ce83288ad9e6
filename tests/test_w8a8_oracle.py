"""Pins of the W8A8 oracle (oracle/w8a8.py): hand-built groups whose scales and
codes follow from the definition, ties, zero groups, the group maximum, and a
brute-force layer written independently (torch's float8 cast, per-token
loops)."""
import numpy as np
import pytest
import torch

from oracle import codecs, formats, moe, w8a8

from gpu_helpers import quantized_layer


def test_exact_groups_round_trip():
    """amax = 448 * 2^-2 gives s = 2^-2 exactly; E4M3 values times s come back
    as their own codes."""
    rng = np.random.default_rng(0)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes = rng.choice(finite, size=(3, 256))
    codes[:, 0] = 0x7E                                  # 448: the group maximum
    codes[:, 128] = 0xFE                                # -448
    x = codecs.decode_e4m3(codes) * 0.25
    got, s = w8a8.quantize_act(x)
    assert np.all(s == np.float32(0.25))
    # -0 and +0 both decode to 0; the quantizer keeps the sign of the value
    same = (got == codes) | ((codecs.decode_e4m3(got) == 0) & (codecs.decode_e4m3(codes) == 0))
    assert same.all()
    np.testing.assert_array_equal(w8a8.dequantize_act(got, s), x)


def test_ties_round_to_even_and_zero_groups():
    x = np.zeros((2, 128))
    x[0, 0] = 448.0                                     # s = 1
    x[0, 1] = 1.0625                                    # midpoint of 1.0 and 1.125 -> 1.0 (even)
    x[0, 2] = 1.1875                                    # midpoint of 1.125 and 1.25 -> 1.25 (even)
    x[0, 3] = 232.0                                     # midpoint of 224 and 240 -> 224 (even)
    x[0, 4] = -0.0009765625                             # 2^-10: half the smallest subnormal 2^-9 -> 0
    x[0, 5] = 3 * 2.0 ** -10                            # midpoint of 2^-9 and 2^-8 -> 2^-8 (even)
    codes, s = w8a8.quantize_act(x)
    v = codecs.decode_e4m3(codes[0, :6])
    assert s[0, 0] == 1.0 and list(v) == [448.0, 1.0, 1.25, 224.0, 0.0, 2.0 ** -8]
    assert s[1, 0] == 1.0 and not codes[1].any()        # an all-zero group encodes zeros


def test_group_maximum_maps_to_448():
    """s = amax / 448 rounds in FP32, so amax / s may miss 448 by an ulp; the
    maximum still encodes as +-448 (saturation), for any amax."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 512)).astype(np.float32) * rng.uniform(1e-3, 1e3, (64, 1)).astype(np.float32)
    codes, s = w8a8.quantize_act(x)
    g = np.abs(x.reshape(64, 4, 128))
    idx = g.argmax(axis=2)
    c = codes.reshape(64, 4, 128)
    top = np.take_along_axis(c, idx[:, :, None], axis=2)[:, :, 0]
    assert np.all((top & 0x7F) == 0x7E)
    assert np.all(s == (g.max(axis=2) / np.float32(448)).astype(np.float32))


def _brute_w8a8(layer, logits, x_bits):
    """Independent evaluation: torch's float8_e4m3fn cast for the quantizer
    (after the same FP32 division and clamp), and per-token loops."""
    def quant(v):  # one row, FP32 values
        v = torch.from_numpy(np.asarray(v, np.float32))
        g = v.view(-1, 128)
        amax = g.abs().amax(dim=1, keepdim=True)
        s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (g / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float64)
        return (q * s.to(torch.float64)).reshape(-1).numpy()

    T, H = x_bits.shape
    k, E = layer.top_k, layer.num_experts
    x = moe.bf16_bits_to_f64(x_bits)
    I = layer.intermediate
    y = np.zeros((T, H))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        sel = np.array([float(logits[t, e]) for e in order])
        p = np.exp(sel - sel.max())
        p /= p.sum()
        xq = quant(x[t])
        for j, e in enumerate(order):
            w13 = formats.dequantize_expert(layer.w13, e)
            w2 = formats.dequantize_expert(layer.w2, e)
            gu = np.array([np.dot(xq, w13[n]) for n in range(2 * I)])
            h = np.array([gu[n] / (1 + np.exp(-gu[n])) * gu[I + n] for n in range(I)])
            hq = quant(h.astype(np.float32))
            y[t] += p[j] * np.array([np.dot(hq, w2[n]) for n in range(H)])
    return y


def test_forward_matches_brute_force():
    E, H, I, k, T = 4, 256, 128, 2, 6
    p13, p2 = quantized_layer(formats.FP8, 71, 0, E, H, I)
    layer = moe.Layer(p13, p2, k)
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    from weight_quantized_moe_amd import synth
    x = synth.hidden_bf16(71, 0, T, H)
    y, _, _ = w8a8.moe_forward_w8a8(layer, logits, x)
    ref = _brute_w8a8(layer, logits, x)
    np.testing.assert_allclose(y, ref, rtol=1e-9, atol=1e-12)
    # and it is not the 16-bit-activation layer (the quantization is applied)
    y16, _, _ = moe.moe_forward(layer, logits, x)
    assert np.linalg.norm(y - y16) / np.linalg.norm(y16) > 1e-3


def test_teacher_forced_down_reproduces_the_forward():
    """Quantizing the oracle's own intermediate and running down_from_codes on
    those codes gives moe_forward_w8a8's output (the pieces the GPU test
    composes are the forward's own)."""
    E, H, I, k, T = 4, 256, 256, 2, 9
    p13, p2 = quantized_layer(formats.FP8, 73, 0, E, H, I)
    layer = moe.Layer(p13, p2, k)
    from weight_quantized_moe_amd import synth
    lg = synth.router_logits(73, 0, T, E)
    x = synth.hidden_bf16(73, 0, T, H)
    y, _, _ = w8a8.moe_forward_w8a8(layer, lg, x)
    hc, hs = w8a8.quantize_act(w8a8.intermediate_w8a8(layer, lg, x))
    np.testing.assert_array_equal(w8a8.down_from_codes(layer, lg, hc, hs), y)


def test_rejects_other_formats():
    p13, p2 = quantized_layer(formats.INT4, 72, 0, 2, 256, 128)
    with pytest.raises(ValueError):
        w8a8.moe_forward_w8a8(moe.Layer(p13, p2, 1), np.zeros((1, 2), np.float32),
                              np.zeros((1, 256), np.uint16))
