"""NVFP4 W4A4 (moe_quant_forward_w4a4) against the W4A4 oracle
(oracle/w4a4.py).

The activation quantizer takes its decisions (the FP32 product and quotient
of the block scale, its RNE to E4M3, the FP32 product and quotient of each
value, its RNE to E2M1) in FP32 on both sides, so its codes and block scales
are compared bit for bit.  In the layer, the codes of the hidden rows are
therefore identical on both sides; the SwiGLU intermediate h is quantized
from FP32 values whose summation order differs between the GPU's FP16 matrix
units and the oracle's float64, so an h value can land on the neighbouring
E2M1 code where its quotient sits within a rounding error of a midpoint, and
a whole group can take the neighbouring E4M3 scale where its maximum does.
Parity is checked in three parts: the output against the oracle's down
projection of the GPU's own h values (the layer tolerance, relative L2 2e-3
and max abs 2e-2 over the whole [T, H] output); the h values against the
oracle's (a bounded fraction differ, each explained by one of the two
near-midpoint cases); and the unforced output.  The global scales are
calibrated on the oracle's values (448 * 6 over the maximum of a calibration
batch), as the pages calibrate them on records.
"""
import numpy as np
import pytest

from oracle import codecs, formats, moe, w4a4
from weight_quantized_moe_amd import synth

from gpu_helpers import (ATOL_MAX, RTOL_L2, GpuLayer, check_routing, dev, errors, log,
                         oracle_w4a4_pool, quantized_layer, spawn_pool)

pytestmark = pytest.mark.gpu

FLIP_FRACTION = 1e-2    # h values allowed to differ from the oracle's
Q_DIST = 1e-3           # E2M1 code units: quotient distance past a midpoint (GPU h error ~1e-5 relative)
S_DIST = 1e-3           # relative distance of a group's pre-rounding scale from an E4M3 midpoint
UNFORCED_RTOL = 3e-3    # unforced output rel-L2

E2M1_LINE = np.array([-6.0, -4.0, -3.0, -2.0, -1.5, -1.0, -0.5, 0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E4M3_LINE = np.unique(np.abs(codecs.decode_e4m3(np.arange(0x7F, dtype=np.uint8))))   # 0 .. 448


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_quantized_moe_amd import load_library
    load_library()


def _gpu_quant(x, g):
    import torch
    from weight_quantized_moe_amd.binding import quantize_act_nvfp4
    c, s = quantize_act_nvfp4(dev(np.ascontiguousarray(x, np.float32)), g)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def _boundary_rows():
    """g = 1 and groups whose maximum is 6 (block scale exactly 1) holding
    every E2M1 magnitude, every midpoint (the RNE ties) and the FP32
    neighbours of each, with both signs; then groups whose maximum sits on an
    E4M3 midpoint of the block scale (6 x the midpoint) or next to it, and
    groups in the subnormal and underflowing range of the scale."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mags, mids, np.nextafter(mids, np.float32(9)), np.nextafter(mids, np.float32(0)),
                           np.float32([1e-3, 0.1, 0.2, 0.3])])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    per = 15
    groups = -(-len(vals) // per)
    flat = np.zeros(groups * per, np.float32)
    flat[:len(vals)] = vals
    a = np.zeros((groups, 16), np.float32)
    a[:, 1:] = flat.reshape(groups, per)
    a[:, 0] = 6.0
    e4 = E4M3_LINE[1:].astype(np.float32)
    smid = ((e4[:-1] + e4[1:]) / 2).astype(np.float32)
    amax = np.concatenate([6 * smid, np.nextafter(6 * smid, np.float32(1e9)), np.nextafter(6 * smid, np.float32(0)),
                           np.float32([2.0 ** -12, 2.0 ** -13, 1e-6])]).astype(np.float32)
    b = np.zeros((len(amax), 16), np.float32)
    b[:, 0] = amax
    b[:, 1:] = amax[:, None] * np.linspace(-0.97, 0.93, 15, dtype=np.float32)[None]
    rows = np.concatenate([a, b])
    rows = np.concatenate([rows, np.zeros(((-len(rows)) % 32, 16), np.float32)])
    return rows.reshape(-1, 512)


@pytest.mark.parametrize("case", ["normal", "boundaries", "magnitudes", "zeros", "saturating"])
def test_activation_quantizer_bit_exact(case):
    log(f"[w4a4 quant] {case}")
    rng = np.random.default_rng(4)
    g = 1.0
    if case == "normal":
        x = rng.standard_normal((300, 2048)).astype(np.float32)
        g = 448 * 6 / float(np.abs(x).max())
    elif case == "boundaries":
        x = _boundary_rows()
    elif case == "magnitudes":
        x = (rng.standard_normal((64, 768)) * 10.0 ** rng.uniform(-12, 12, (64, 1))).astype(np.float32)
        g = 448 * 6 / 3.0
    elif case == "zeros":
        x = rng.standard_normal((20, 384)).astype(np.float32)
        x[3] = 0.0
        x[5, 128:256] = 0.0
        x[7, :16] = -0.0
        g = 448 * 6 / float(np.abs(x).max())
    else:  # a global scale far too large: block scales clamp to 448, values saturate to +-6
        x = rng.standard_normal((16, 256)).astype(np.float32)
        g = 448 * 6 / float(np.abs(x).max()) * 50.0
    c, s = _gpu_quant(x, g)
    rc, rs = w4a4.quantize_act(x, g)
    assert np.array_equal(s, rs), f"{int((s != rs).sum())} block scales differ"
    assert np.array_equal(c, codecs.pack_nibbles(rc)), "codes differ"


def _run_w4a4(g, lg, x, gx, gh, res=None):
    import torch
    lay = g.layer
    T, k, E, I = x.shape[0], lay.top_k, lay.num_experts, lay.inter
    R = T * k
    pr = dict(topk_ids=torch.empty((T, k), dtype=torch.int32, device="cuda"),
              topk_w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
              expert_offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
              sorted_token_ids=torch.empty(R, dtype=torch.int32, device="cuda"),
              inv_pos=torch.empty(R, dtype=torch.int32, device="cuda"),
              h=torch.empty((R, I), dtype=torch.float16, device="cuda"))
    ws = lay.workspace(T)
    out = lay.forward_w4a4(dev(lg), dev(x.view(np.int16)).view(torch.bfloat16), gx, gh,
                           residual=None if res is None else dev(res.view(np.int16)).view(torch.bfloat16),
                           workspace=ws, probe=pr)
    torch.cuda.synchronize()
    assert not lay.check(ws)
    h = pr.pop("h").cpu().numpy().astype(np.float64)
    return out.view(torch.int16).cpu().numpy().view(np.uint16), {n: v.cpu().numpy() for n, v in pr.items()}, h


def _check_h(h_gpu, h32, gh):
    """The GPU's h values (e2m1 * s, FP16) against the oracle's quantization
    of its own FP32 intermediate; returns the fraction that differ."""
    rc, rs = w4a4.quantize_act(h32, gh)
    vo = w4a4.block_values(rc, rs)
    diff = vo != h_gpu
    frac = float(diff.mean())
    if not diff.any():
        return frac
    R, I = h32.shape
    G = I // 16
    so = codecs.decode_e4m3(rs)                                    # [R, G]
    sg = np.abs(h_gpu.reshape(R, G, 16)).max(axis=2) / 6.0         # the group maximum carries code 6
    gdiff = diff.reshape(R, G, 16).any(axis=2)
    # groups whose scale differs: adjacent E4M3 values, the oracle's
    # pre-rounding scale within S_DIST of their midpoint
    sdiff = gdiff & (sg != so)
    if sdiff.any():
        amax = np.abs(h32.reshape(R, G, 16)).max(axis=2)[sdiff]
        u = ((amax * np.float32(gh)).astype(np.float32) / np.float32(6)).astype(np.float64)
        io, ig = np.searchsorted(E4M3_LINE, so[sdiff]), np.searchsorted(E4M3_LINE, sg[sdiff])
        assert np.all(np.abs(io - ig) == 1), "a group's scale differs by more than one E4M3 step"
        mid = (so[sdiff] + sg[sdiff]) / 2
        assert np.all(np.abs(u - mid) <= S_DIST * mid), "a differing group scale is not near a midpoint"
    # values of groups with the oracle's scale: the oracle's quotient within
    # Q_DIST of the GPU code's rounding interval
    vd = diff & np.repeat(sg == so, 16, axis=1)
    n_vals = int(vd.sum())
    if n_vals:
        s_el = np.repeat(so, 16, axis=1)[vd]
        assert np.all(s_el > 0)
        cg = h_gpu[vd] / s_el
        q = ((h32[vd] * np.float32(gh)).astype(np.float32) / s_el.astype(np.float32)).astype(np.float64)
        ig = np.searchsorted(E2M1_LINE, cg)
        assert np.all(E2M1_LINE[np.minimum(ig, len(E2M1_LINE) - 1)] == cg), "a GPU h value is off the E2M1 grid"
        lo = np.where(ig > 0, (E2M1_LINE[np.maximum(ig - 1, 0)] + E2M1_LINE[ig]) / 2, -np.inf)
        hi = np.where(ig < len(E2M1_LINE) - 1, (E2M1_LINE[ig] + E2M1_LINE[np.minimum(ig + 1, len(E2M1_LINE) - 1)]) / 2,
                      np.inf)
        dist = np.maximum(0.0, np.maximum(lo - q, q - hi))
        log(f"    h values differing: {int(diff.sum())} ({frac:.2e}); in {int(sdiff.sum())} groups with "
            f"the neighbouring scale; {n_vals} single values, distance past the midpoint max {dist.max():.3e}")
        assert np.all(dist <= Q_DIST), "a differing h value is beyond the rounding error"
    else:
        log(f"    h values differing: {int(diff.sum())} ({frac:.2e}), all in {int(sdiff.sum())} groups "
            f"with the neighbouring scale")
    return frac


def _scales(layer, lg_cal, x_cal):
    """Calibrated global scales: 448 * 6 over the largest hidden value and the
    largest intermediate value of a calibration batch (oracle values)."""
    gx = 448 * 6 / float(np.abs(moe.bf16_bits_to_f64(x_cal)).max())
    h = w4a4.intermediate_w4a4(layer, lg_cal, x_cal, gx)
    return gx, 448 * 6 / float(np.abs(h).max())


@pytest.mark.parametrize("T,E,H,I,k", [(5, 8, 256, 128, 2), (64, 16, 512, 256, 4), (300, 8, 384, 384, 2),
                                       (1000, 32, 256, 640, 8), (129, 6, 1024, 128, 3)])
def test_w4a4_layer(T, E, H, I, k):
    """Ragged M tiles (experts with 1..300 rows), N tiles past I or H, every
    batch size on the many-rows kernels."""
    log(f"[w4a4] T={T} E={E} H={H} I={I} k={k}")
    p13, p2 = quantized_layer(formats.NVFP4, 85, T, E, H, I)
    g = GpuLayer(p13, p2, k)
    lg = synth.router_logits(85, T, T, E, "bias")
    x = synth.hidden_bf16(85, T, T, H)
    gx, gh = _scales(g.oracle, synth.router_logits(86, T, 32, E), synth.hidden_bf16(86, T, 32, H))
    res = synth.residual_bf16(85, T, T, H) if T % 2 else None
    out, pr, h = _run_w4a4(g, lg, x, gx, gh, res)
    check_routing(pr, lg, k, E)
    rel, mx = errors(out, w4a4.down_from_values(g.oracle, lg, h / np.float64(np.float32(gh)), res))
    y, _, _ = w4a4.moe_forward_w4a4(g.oracle, lg, x, gx, gh, res)
    rel_u, _ = errors(out, y)
    frac = _check_h(h, w4a4.intermediate_w4a4(g.oracle, lg, x, gx), gh)
    log(f"    forced rel_l2={rel:.3e} max_abs={mx:.3e}; h differing {frac:.2e}; unforced rel_l2={rel_u:.3e}")
    assert rel <= RTOL_L2 and mx <= ATOL_MAX
    assert frac <= FLIP_FRACTION and rel_u <= UNFORCED_RTOL
    out2, _, _ = _run_w4a4(g, lg, x, gx, gh, res)
    assert np.array_equal(out, out2), "repeat run differs"


@pytest.mark.timeout(600)
def test_w4a4_full_shape():
    """The NVFP4 workload the bench times (hidden 2048, intermediate 768, 128
    experts, top-8, 16384 tokens, Zipf-skewed logits): every token compared,
    the oracle's per-expert work in a pool of CPU workers."""
    log("[w4a4] full shape T=16384 nvfp4 zipf")
    wl = synth.WORKLOADS["nvfp4_zipf"]
    E, H, I, k, T = wl.experts, wl.hidden, wl.inter, wl.top_k, 16384
    with spawn_pool() as pool:
        p13, p2 = quantized_layer(formats.NVFP4, wl.wid, 0, E, H, I)
        g = GpuLayer(p13, p2, k)
        lg = synth.router_logits(wl.wid, 0, T, E, wl.logits)
        x = synth.hidden_bf16(wl.wid, 0, T, H)
        # calibration: the first 128 tokens of the batch
        gx = 448 * 6 / float(np.abs(moe.bf16_bits_to_f64(x[:128])).max())
        _, _, h_cal = oracle_w4a4_pool(pool, p13, p2, k, lg[:128], x[:128], gx, 1.0)
        gh = 448 * 6 / float(np.abs(h_cal).max())
        log(f"    calibrated gx={gx:.4g} gh={gh:.4g}")
        out, pr, h = _run_w4a4(g, lg, x, gx, gh)
        check_routing(pr, lg, k, E)
        y, y_forced, h32 = oracle_w4a4_pool(pool, p13, p2, k, lg, x, gx, gh, h / np.float64(np.float32(gh)))
    rel, mx = errors(out, y_forced)
    rel_u, _ = errors(out, y)
    frac = _check_h(h, h32, gh)
    log(f"    forced rel_l2={rel:.3e} max_abs={mx:.3e}; h differing {frac:.2e}; unforced rel_l2={rel_u:.3e}")
    assert rel <= RTOL_L2 and mx <= ATOL_MAX
    assert frac <= FLIP_FRACTION and rel_u <= UNFORCED_RTOL
