"""Pins of the NVFP4 W4A4 oracle (oracle/w4a4.py): hand-built groups whose
scales and codes follow from the definition, E2M1 and E4M3 ties, zero and
underflowing groups, the group maximum, a saturated block scale, and a
brute-force layer written independently (per-binade rounding with numpy's
half-to-even, torch's float8 cast for the block scale, per-token loops)."""
import numpy as np
import pytest
import torch

from oracle import codecs, formats, moe, w4a4

from gpu_helpers import quantized_layer

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def test_exact_groups_round_trip():
    """amax = 6 s with s an E4M3 value and g = 1 gives the block scale s
    exactly; grid values times s come back as their own codes."""
    rng = np.random.default_rng(0)
    svals = np.array([2.0 ** -6, 0.125, 0.5, 1.0, 1.125, 2.0, 13.0, 448.0])
    x = np.zeros((len(svals), 64), np.float32)
    codes = rng.integers(0, 16, size=x.shape).astype(np.uint8)
    codes[:, ::16] = 0x7                                # +6: the maximum of each group
    codes[:, 5::16] = 0xF                               # -6
    for r, s in enumerate(svals):
        x[r] = codecs.decode_e2m1(codes[r]) * s
    got, sc = w4a4.quantize_act(x, 1.0)
    assert np.all(codecs.decode_e4m3(sc) == svals[:, None])
    same = (got == codes) | ((codecs.decode_e2m1(got) == 0) & (codecs.decode_e2m1(codes) == 0))
    assert same.all()
    np.testing.assert_array_equal(w4a4.dequantize_act(got, sc, 1.0), x)


def test_e2m1_ties_round_to_even():
    x = np.zeros((2, 16), np.float32)
    x[:, 0] = 6.0                                       # s = 1 (g = 1)
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]          # the even neighbour of each midpoint
    x[0, 1:8] = ties
    x[1, 1:8] = [-t for t in ties]
    x[0, 8:15] = np.nextafter(np.float32(ties), np.float32(10))   # just above: the upper neighbour
    codes, s = w4a4.quantize_act(x, 1.0)
    v = codecs.decode_e2m1(codes)
    assert np.all(codecs.decode_e4m3(s) == 1.0)
    assert list(v[0, 1:8]) == want
    assert list(v[1, 1:8]) == [-w for w in want]
    assert list(v[0, 8:15]) == [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_block_scale_rounds_to_even_and_the_maximum_saturates():
    """amax = 6.375 (g = 1): amax / 6 = 1.0625 is the E4M3 midpoint of 1 and
    1.125 and rounds to 1; the maximum 6.375 / 1 then saturates to 6."""
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 6.375
    x[0, 1] = 1.0
    codes, s = w4a4.quantize_act(x, 1.0)
    assert codecs.decode_e4m3(s)[0, 0] == 1.0
    assert codecs.decode_e2m1(codes)[0, 0] == 6.0 and codecs.decode_e2m1(codes)[0, 1] == 1.0


def test_zero_and_underflowing_groups():
    x = np.zeros((3, 32), np.float32)
    x[1, :16] = 1e-30                                   # g * amax / 6 underflows E4M3: s = 0
    x[2, 16:] = -0.0
    codes, s = w4a4.quantize_act(x, 1.0)
    assert not codecs.decode_e4m3(s).any()
    assert not codecs.decode_e2m1(codes).any()


def test_group_maximum_maps_to_6():
    """With the block scale in E4M3's normal range, the maximum over the scale
    lands within [6 / (1 + 2^-4), 6 (1 + 2^-4)], which rounds (or saturates)
    to 6, for any amax and g."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 256)) * 10.0 ** rng.uniform(-3, 3, (64, 1))).astype(np.float32)
    for r in range(64):
        gr = np.float32(448 * 6 / np.abs(x[r]).max()) * np.float32(rng.uniform(0.2, 1.0))
        codes, s = w4a4.quantize_act(x[r:r + 1], gr)
        sv = codecs.decode_e4m3(s)[0]
        blocks = np.abs(x[r]).reshape(-1, 16)
        top = np.take_along_axis(codes[0].reshape(-1, 16), blocks.argmax(axis=1)[:, None], axis=1)[:, 0]
        normal = sv >= 2.0 ** -6
        assert np.all((top[normal] & 0x7) == 0x7)


def test_saturated_block_scale():
    """g too large for the data: g * amax / 6 beyond 448 clamps the block scale
    to 448 and the values beyond 6 * 448 / g saturate to +-6."""
    x = np.zeros((1, 16), np.float32)
    x[0, :4] = [1.0, -1.0, 0.25, 0.5]
    codes, s = w4a4.quantize_act(x, 6000.0)             # 6000 / 6 = 1000 > 448
    assert codecs.decode_e4m3(s)[0, 0] == 448.0
    v = codecs.decode_e2m1(codes)[0]
    # x * g / 448: 13.4 -> 6, -13.4 -> -6, 3.35 -> 3, 6.7 -> 6
    assert list(v[:4]) == [6.0, -6.0, 3.0, 6.0]


def _brute_quant(row, g):
    """Independent quantize-dequantize of one FP32 row: block scale by torch's
    float8_e4m3fn cast, values rounded per binade of the E2M1 grid with
    numpy's half-to-even."""
    row = np.asarray(row, np.float32)
    g = np.float32(g)
    out = np.zeros(len(row))
    for b0 in range(0, len(row), 16):
        blk = row[b0:b0 + 16]
        u = np.float32(np.float32(np.abs(blk).max() * g) / np.float32(6))
        s = float(torch.tensor(min(float(u), 448.0)).to(torch.float8_e4m3fn).to(torch.float64))
        if s == 0:
            continue
        for i, xv in enumerate(blk):
            q = float(np.float32(np.float32(xv * g) / np.float32(s)))
            a = min(abs(q), 6.0)
            step = 0.5 if a < 2 else (1.0 if a < 4 else 2.0)
            v = min(np.round(a / step) * step, 6.0)
            out[b0 + i] = np.copysign(v, q) * s / float(g)
    return out


def test_quantizer_matches_brute_force():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((40, 128)) * 10.0 ** rng.uniform(-2, 2, (40, 1))).astype(np.float32)
    g = 448 * 6 / float(np.abs(x).max()) * 0.7
    c, s = w4a4.quantize_act(x, g)
    got = w4a4.dequantize_act(c, s, g)
    ref = np.stack([_brute_quant(r, g) for r in x])
    np.testing.assert_array_equal(got, ref)
    assert sorted(set(np.abs(codecs.decode_e2m1(c)).ravel())) == list(E2M1_GRID)


def _brute_w4a4(layer, logits, x_bits, gx, gh):
    T, H = x_bits.shape
    k, E, I = layer.top_k, layer.num_experts, layer.intermediate
    x = moe.bf16_bits_to_f64(x_bits)
    y = np.zeros((T, H))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        sel = np.array([float(logits[t, e]) for e in order])
        p = np.exp(sel - sel.max())
        p /= p.sum()
        xq = _brute_quant(x[t], gx)
        for j, e in enumerate(order):
            w13 = formats.dequantize_expert(layer.w13, e)
            w2 = formats.dequantize_expert(layer.w2, e)
            gu = np.array([np.dot(xq, w13[n]) for n in range(2 * I)])
            h = np.array([gu[n] / (1 + np.exp(-gu[n])) * gu[I + n] for n in range(I)])
            hq = _brute_quant(h.astype(np.float32), gh)
            y[t] += p[j] * np.array([np.dot(hq, w2[n]) for n in range(H)])
    return y


def _layer(seed, E, H, I, k):
    p13, p2 = quantized_layer(formats.NVFP4, seed, 0, E, H, I)
    return moe.Layer(p13, p2, k)


def test_forward_matches_brute_force():
    from weight_quantized_moe_amd import synth
    E, H, I, k, T = 4, 256, 128, 2, 5
    layer = _layer(91, E, H, I, k)
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = synth.hidden_bf16(91, 0, T, H)
    gx = 448 * 6 / float(np.abs(moe.bf16_bits_to_f64(x)).max())
    gh = 448 * 6 / 0.05
    y, _, _ = w4a4.moe_forward_w4a4(layer, logits, x, gx, gh)
    ref = _brute_w4a4(layer, logits, x, gx, gh)
    np.testing.assert_allclose(y, ref, rtol=1e-9, atol=1e-12)
    # and it is not the 16-bit-activation layer (the quantization is applied)
    y16, _, _ = moe.moe_forward(layer, logits, x)
    assert np.linalg.norm(y - y16) / np.linalg.norm(y16) > 1e-2


def test_teacher_forced_down_reproduces_the_forward():
    from weight_quantized_moe_amd import synth
    E, H, I, k, T = 4, 256, 256, 2, 9
    layer = _layer(93, E, H, I, k)
    lg = synth.router_logits(93, 0, T, E)
    x = synth.hidden_bf16(93, 0, T, H)
    gx, gh = 300.0, 20000.0
    y, _, _ = w4a4.moe_forward_w4a4(layer, lg, x, gx, gh)
    hc, hs = w4a4.quantize_act(w4a4.intermediate_w4a4(layer, lg, x, gx), gh)
    np.testing.assert_array_equal(w4a4.down_from_values(layer, lg, w4a4.dequantize_act(hc, hs, gh)), y)


def test_rejects_other_formats_and_bad_scales():
    p13, p2 = quantized_layer(formats.FP8, 92, 0, 2, 256, 128)
    with pytest.raises(ValueError):
        w4a4.moe_forward_w4a4(moe.Layer(p13, p2, 1), np.zeros((1, 2), np.float32),
                              np.zeros((1, 256), np.uint16), 1.0, 1.0)
    for g in (0.0, -1.0, np.inf, np.nan):
        with pytest.raises(ValueError):
            w4a4.quantize_act(np.ones((1, 16), np.float32), g)
