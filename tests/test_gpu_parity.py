"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Routing, grouping and dequantized weights are compared bit-exactly; layer
outputs within relative L2 2e-3 and max abs 2e-2 of the oracle.
"""
import numpy as np
import pytest

from oracle import codecs, formats, moe
from weight_quantized_moe_amd import synth

from gpu_helpers import (ATOL_MAX, RTOL_L2, GpuLayer, check_routing, errors, log,
                         quantized_layer, random_layer)

pytestmark = pytest.mark.gpu

FMTS = formats.FORMATS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_quantized_moe_amd import load_library
    load_library()      # fails loudly if the HIP library is missing


# ------------------------------------------------------------ dequantization

def _special_layer(fmt, rng):
    """Small layer whose codes cover every code value of the format."""
    E, H, I = 2, 256, 128
    p13, p2 = quantized_layer(fmt, 11, 0, E, H, I)
    for p in (p13, p2):
        flat = p.w.reshape(-1)
        if fmt == formats.FP8:
            codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
        else:
            codes = np.arange(256, dtype=np.uint8)        # all nibble pairs
        flat[:len(codes)] = codes
        if fmt == formats.NVFP4:
            sflat = p.scale.reshape(-1)
            sc = np.array([c for c in range(128) if c != 0x7F], np.uint8)
            sflat[:len(sc)] = sc
    return p13, p2


@pytest.mark.parametrize("fmt", FMTS)
def test_dequantize_bit_exact(fmt):
    log(f"[dequant] fmt={fmt}")
    p13, p2 = _special_layer(fmt, np.random.default_rng(0))
    g = GpuLayer(p13, p2, 2)
    for which, p in ((0, p13), (1, p2)):
        for e in range(p.num_experts):
            got = g.layer.dequantize(which, e).cpu().numpy()
            ref = formats.dequantize_expert(p, e)
            if fmt == formats.NVFP4:
                # the device divides the exact FP32 product by gscale once
                vals = codecs.decode_e2m1(codecs.unpack_nibbles(p.w[e])).reshape(p.n, p.k // 16, 16)
                s = codecs.decode_e4m3(p.scale[e])[:, :, None]
                ref32 = (vals * s).astype(np.float32).reshape(p.n, p.k) / np.float32(p.gscale[e])
            else:
                ref32 = ref.astype(np.float32)   # INT4 exact; FP8 one rounding
            assert np.array_equal(got, ref32), f"{fmt} which={which} e={e}"


# ------------------------------------------------------------ routing

@pytest.mark.parametrize("logit_kind", ["f32", "bf16_ties"])
@pytest.mark.parametrize("T,E,k", [(1, 128, 8), (2, 16, 16), (3, 512, 64), (4, 200, 20), (4, 40, 7),
                                   (16, 128, 8), (16, 512, 64), (11, 200, 20), (17, 128, 8),
                                   (37, 128, 8), (64, 128, 8), (65, 128, 8),
                                   (128, 128, 8), (256, 128, 8), (130, 512, 31), (255, 16, 16),
                                   (200, 128, 32), (257, 128, 8),
                                   (300, 128, 8), (2500, 128, 8), (37, 200, 20), (300, 200, 6),
                                   (50, 512, 64), (700, 512, 3)])
def test_routing_and_grouping_bit_exact(T, E, k, logit_kind):
    log(f"[routing] T={T} E={E} k={k} logits={logit_kind}")
    H, I = 256, 128
    p13, p2 = random_layer(formats.INT4, 5, E, H, I)
    g = GpuLayer(p13, p2, k)
    rng = np.random.default_rng(T)
    x = synth.hidden_bf16(6, 0, T, H)
    if logit_kind == "f32":
        lg = synth.router_logits(6, 0, T, E)
        out, pr, _ = g.run(lg, x, probe=True)
        check_routing(pr, lg, k, E)
    else:
        # coarse BF16 logits: many exact ties
        lgf = np.round(rng.standard_normal((T, E)) * 4) / 4
        bits = synth.to_bf16_bits(lgf.astype(np.float32))
        out, pr, _ = g.run(bits, x, probe=True, logits_bf16=True)
        check_routing(pr, moe.bf16_bits_to_f64(bits), k, E)


@pytest.mark.parametrize("logit_kind", ["f32", "bf16"])
def test_signed_zero_logits_tie(logit_kind):
    """-0 and +0 are equal logits: their order in the top-k falls to the expert
    id, as for any other tie (rows whose k-th largest logit is a zero of either
    sign, and rows of zeros only)."""
    log(f"[routing] signed zeros, logits={logit_kind}")
    T, E, k, H, I = 48, 16, 5, 256, 128
    rng = np.random.default_rng(3)
    lg = np.zeros((T, E), np.float32)
    for t in range(T):
        nz = rng.choice(E, size=int(rng.integers(0, 4)), replace=False)
        lg[t, nz] = rng.choice([1.0, 2.0, -1.0], size=len(nz))
        neg0 = rng.random(E) < 0.5
        z = lg[t] == 0
        lg[t, z & neg0] = -0.0
    assert np.signbit(lg[lg == 0]).any() and (~np.signbit(lg[lg == 0])).any()
    p13, p2 = random_layer(formats.INT4, 5, E, H, I)
    g = GpuLayer(p13, p2, k)
    x = synth.hidden_bf16(7, 0, T, H)
    if logit_kind == "f32":
        _, pr, _ = g.run(lg, x, probe=True)
        check_routing(pr, lg, k, E)
    else:
        bits = synth.to_bf16_bits(lg)
        _, pr, _ = g.run(bits, x, probe=True, logits_bf16=True)
        check_routing(pr, moe.bf16_bits_to_f64(bits), k, E)


# ------------------------------------------------------------ layer outputs

def _check_layer(g, lg, x, res=None, tokens=None, tag=""):
    out, pr, ovf = g.run(lg, x, res, probe=True)
    check_routing(pr, lg, g.top_k, g.layer.num_experts) if tokens is None else None
    assert not ovf
    y, _, _ = moe.moe_forward(g.oracle, lg, x, res, tokens=tokens)
    got = out if tokens is None else out[tokens]
    rel, mx = errors(got, y)
    log(f"    {tag} rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= RTOL_L2 and mx <= ATOL_MAX, (tag, rel, mx)
    return out, pr


def test_tiny_config_int4():
    """Tiny layer: H 256, I 128, 8 experts, top-2, 64 tokens, INT4 g128."""
    w = synth.WORKLOADS["tiny"]
    log("[tiny]")
    p13, p2 = quantized_layer(w.fmt, w.wid, 0, w.experts, w.hidden, w.inter)
    g = GpuLayer(p13, p2, w.top_k)
    lg = synth.router_logits(w.wid, 0, 64, w.experts)
    x = synth.hidden_bf16(w.wid, 0, 64, w.hidden)
    _check_layer(g, lg, x, tag="tiny")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T,k", [(1, 4), (5, 4), (64, 4), (300, 4), (1000, 2), (777, 16)])
def test_small_layers(fmt, T, k):
    """E 16, H 512, I 384: decode (T*k <= 16 E) and prefill paths, ragged tiles."""
    log(f"[small] fmt={fmt} T={T} k={k}")
    E, H, I = 16, 512, 384
    p13, p2 = quantized_layer(fmt, 12, k, E, H, I)
    g = GpuLayer(p13, p2, k)
    lg = synth.router_logits(12, T, T, E, "bias")
    x = synth.hidden_bf16(12, T, T, H)
    _check_layer(g, lg, x, tag=f"{fmt} T={T} k={k}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T", [65, 128])
def test_decode_after_chunked_grouping(fmt, T):
    """E 64, top-8, T 65 / 128: T > 64 takes the chunked grouping, while
    T * k <= 16 E keeps the weight-streaming decode GEMMs."""
    log(f"[decode T>64] fmt={fmt} T={T}")
    E, H, I, k = 64, 256, 128, 8
    p13, p2 = quantized_layer(fmt, 17, T, E, H, I)
    g = GpuLayer(p13, p2, k)
    lg = synth.router_logits(17, T, T, E)
    x = synth.hidden_bf16(17, T, T, H)
    _check_layer(g, lg, x, tag=f"{fmt} E=64 T={T}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T,k,E,H,I", [(16, 4, 8, 512, 256), (9, 8, 8, 256, 768),
                                       (40, 4, 16, 768, 512), (64, 8, 32, 1024, 1280),
                                       (100, 2, 16, 2048, 256), (200, 8, 128, 512, 384),
                                       (64, 8, 128, 2048, 768), (40, 2, 16, 256, 256)])
def test_streaming_decode(fmt, T, k, E, H, I):
    """Decode batches with 4 to 16 rows per expert on average and H a multiple
    of 256 (at most 2048) run the streaming gate/up GEMM: experts holding 0, 1
    and up to 49 rows (several 16-row chunks, the hidden rows staged again
    between units), 1 to 8 chunks per unit (odd counts alternate the ring
    slots across units), I not a multiple of 256, from one unit per busy block
    to many, and unit ranges aligned to row chunks (T=64, 128 experts: three
    units per block, half a chunk)."""
    log(f"[stream] fmt={fmt} T={T} k={k} E={E} H={H} I={I}")
    p13, p2 = quantized_layer(fmt, 23, T, E, H, I)
    g = GpuLayer(p13, p2, k)
    lg = synth.router_logits(23, T, T, E, "bias")
    x = synth.hidden_bf16(23, T, T, H)
    _, pr = _check_layer(g, lg, x, tag=f"{fmt} stream T={T} E={E} H={H} I={I}")
    counts = np.bincount(moe.route(lg, k)[0].ravel(), minlength=E)
    assert 4 * E <= T * k <= 16 * E
    if T >= 40:
        assert counts.max() > 16, counts   # some expert spans two row chunks


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T,k,E,H,I", [(24, 4, 32, 512, 256), (48, 8, 128, 384, 384),
                                       (40, 4, 64, 256, 256), (30, 2, 16, 768, 512),
                                       (64, 8, 128, 384, 256)])
def test_decode_skewed_experts(fmt, T, k, E, H, I):
    """Zipf-skewed routing with experts of up to 50 rows: the register-streaming
    decode GEMMs then take one 16-row chunk of an expert per unit, so an
    expert's chunks spread over blocks (gate/up below 4 rows per expert on
    average or with H not a multiple of 256, the down projection always)."""
    log(f"[skew] fmt={fmt} T={T} k={k} E={E} H={H} I={I}")
    p13, p2 = quantized_layer(fmt, 29, T, E, H, I)
    g = GpuLayer(p13, p2, k)
    lg = synth.router_logits(29, T, T, E, "zipf")
    x = synth.hidden_bf16(29, T, T, H)
    counts = np.bincount(moe.route(lg, k)[0].ravel(), minlength=E)
    assert (T * k < 4 * E or H % 256) and T > 16 and counts.max() > 16, counts
    _check_layer(g, lg, x, tag=f"{fmt} skew T={T} E={E} H={H} I={I}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T,k,E,H,I", [(1, 8, 128, 2048, 768), (1, 3, 16, 256, 384),
                                       (2, 12, 32, 512, 256), (2, 8, 64, 384, 1152),
                                       (2, 1, 8, 256, 128), (3, 8, 64, 384, 1152)])
@pytest.mark.parametrize("with_res", [False, True])
def test_decode_down_fused_combine(fmt, T, k, E, H, I, with_res):
    """One or two tokens: the decode down projection adds each token's slots
    itself (slot values in FP32, slots in order, then the residual) and writes
    the BF16 output; no combine launch.  Covers both column-block widths (8
    columns at T = 1, 16 at T = 2), more slots than waves (k = 12), k parts
    without a chunk (I = 128, 256, 384) and uneven ones (I = 1152), H not a
    multiple of 256, and the first batch size past the limit (T = 3: the
    expert-major GEMM and the combine)."""
    log(f"[down-fused] fmt={fmt} T={T} k={k} E={E} H={H} I={I} res={with_res}")
    p13, p2 = quantized_layer(fmt, 37, T, E, H, I)
    g = GpuLayer(p13, p2, k)
    lg = synth.router_logits(37, T, T, E)
    x = synth.hidden_bf16(37, T, T, H)
    res = synth.residual_bf16(37, T, T, H) if with_res else None
    out1, _ = _check_layer(g, lg, x, res, tag=f"{fmt} fused down T={T} k={k} I={I}")
    out2, _, _ = g.run(lg, x, res)
    assert np.array_equal(out1, out2), "repeat runs differ"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T", [20, 700])
def test_hidden_not_multiple_of_256(fmt, T):
    """H = 384: the prefill down projection's last 256-column tile is half full."""
    log(f"[h384] fmt={fmt} T={T}")
    E, H, I, k = 8, 384, 256, 2
    p13, p2 = quantized_layer(fmt, 16, T, E, H, I)
    g = GpuLayer(p13, p2, k)
    lg = synth.router_logits(16, T, T, E)
    x = synth.hidden_bf16(16, T, T, H)
    _check_layer(g, lg, x, tag=f"{fmt} H=384 T={T}")


@pytest.mark.parametrize("fmt", FMTS)
def test_prefill_tile_edges(fmt):
    """Routing crafted so the experts hold 1, 31, 32, 33, 96, 97, 128 and 130
    rows: the prefill GEMMs see every count of 32-row subtiles that hold rows
    in a 128-row tile (1 to 4), a full tile, and a second tile with 2 rows."""
    log(f"[tile-edges] fmt={fmt}")
    E, H, I, k = 8, 256, 256, 2
    counts = np.array([1, 31, 32, 33, 96, 97, 128, 130])
    T = int(counts.sum()) // k
    assert T * k > 16 * E                     # the prefill path
    ids = np.repeat(np.arange(E), counts)     # sorted; no expert holds more than T rows,
    first, second = ids[:T], ids[T:]          # so a token's two experts differ
    assert np.all(first != second)
    rng = np.random.default_rng(21)
    perm = rng.permutation(T)
    first, second = first[perm], second[perm]
    lg = rng.uniform(-1.0, 0.0, size=(T, E)).astype(np.float32)
    lg[np.arange(T), first] = 3.0 + rng.uniform(0.0, 0.5, size=T).astype(np.float32)
    lg[np.arange(T), second] = 2.0 + rng.uniform(0.0, 0.5, size=T).astype(np.float32)
    p13, p2 = quantized_layer(fmt, 21, 0, E, H, I)
    g = GpuLayer(p13, p2, k)
    x = synth.hidden_bf16(21, 0, T, H)
    ids, _ = moe.route(lg, k)
    assert np.array_equal(np.bincount(ids.ravel(), minlength=E), counts)
    _check_layer(g, lg, x, tag=f"{fmt} tile edges")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T", [3, 100])
def test_hidden_above_2048(fmt, T):
    """H = 2304 > 2048: decode (T=3) scans each row for its power of two inside
    the gate/up GEMM instead of taking it from the routing kernel; prefill
    (T=100) stages the FP16 rows in two passes over the row."""
    log(f"[h2304] fmt={fmt} T={T}")
    E, H, I, k = 4, 2304, 256, 2
    p13, p2 = quantized_layer(fmt, 18, T, E, H, I)
    g = GpuLayer(p13, p2, k)
    lg = synth.router_logits(18, T, T, E)
    x = synth.hidden_bf16(18, T, T, H)
    _check_layer(g, lg, x, tag=f"{fmt} H=2304 T={T}")


@pytest.mark.parametrize("fmt", FMTS)
def test_residual_and_determinism(fmt):
    log(f"[residual] fmt={fmt}")
    E, H, I, k, T = 16, 256, 256, 4, 200
    p13, p2 = quantized_layer(fmt, 13, 0, E, H, I)
    g = GpuLayer(p13, p2, k)
    lg = synth.router_logits(13, 0, T, E)
    x = synth.hidden_bf16(13, 0, T, H)
    res = synth.residual_bf16(13, 0, T, H)
    out1, _ = _check_layer(g, lg, x, res, tag="residual")
    out2, _, _ = g.run(lg, x, res)
    assert np.array_equal(out1, out2), "repeat runs differ"


def test_edge_cases():
    log("[edge] k=1, k=E, single expert, empty experts")
    H, I = 256, 128
    for (E, k, T) in [(8, 1, 50), (8, 8, 20), (1, 1, 9), (64, 2, 3)]:
        p13, p2 = quantized_layer(formats.INT4, 14, E, E, H, I)
        g = GpuLayer(p13, p2, k)
        lg = synth.router_logits(14, E, T, E)
        x = synth.hidden_bf16(14, E, T, H)
        _check_layer(g, lg, x, tag=f"E={E} k={k} T={T}")


def test_zero_tokens_is_a_noop():
    import torch
    E, H, I = 8, 256, 128
    p13, p2 = random_layer(formats.FP8, 3, E, H, I)
    g = GpuLayer(p13, p2, 2)
    out = torch.full((0, H), 7, dtype=torch.bfloat16, device="cuda")
    g.layer.forward(torch.empty((0, E), device="cuda"), torch.empty((0, H), dtype=torch.bfloat16,
                    device="cuda"), out=out, workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()


@pytest.mark.parametrize("T", [16, 64])
@pytest.mark.parametrize("which", ["h", "partial"])
def test_fp16_overflow_flag_both_paths(which, T):
    """Saturating the SwiGLU intermediate h or the routing-weighted FP16
    partials sets the flag, on the decode (T=16) and the prefill (T=64) GEMMs,
    and the outputs stay finite."""
    log(f"[overflow2] which={which} T={T}")
    E, H, I, k = 4, 256, 128, 2
    p13, p2 = quantized_layer(formats.INT4, 19, T, E, H, I)
    if which == "h":
        p13.scale[:] = np.float16(60000.0)
    else:
        p2.scale[:] = np.float16(60000.0)
    g = GpuLayer(p13, p2, k)
    lg = synth.router_logits(19, T, T, E)
    x = synth.hidden_bf16(19, T, T, H)
    out, pr, ovf = g.run(lg, x, probe=True)
    assert ovf
    assert np.nanmax(np.abs(pr["h"].astype(np.float32))) <= 65504.0
    assert np.all(np.isfinite(moe.bf16_bits_to_f64(out)))


def test_fp16_intermediate_overflow_flag():
    """Saturating the FP16 SwiGLU intermediate sets the flag and clamps."""
    log("[overflow]")
    E, H, I, k, T = 4, 256, 128, 2, 16
    p13, p2 = quantized_layer(formats.INT4, 15, 0, E, H, I)
    p13.scale[:] = np.float16(60000.0)
    g = GpuLayer(p13, p2, k)
    lg = synth.router_logits(15, 0, T, E)
    x = synth.hidden_bf16(15, 0, T, H)
    _, pr, ovf = g.run(lg, x, probe=True)
    assert ovf
    assert np.nanmax(np.abs(pr["h"].astype(np.float32))) <= 65504.0
