"""Checkpoint importers (moe_quant_import_expert): source tensors written by
the oracle's exporters (oracle/checkpoints.py, from the library formats by the
source formats' definitions) are imported on the GPU, and the packed bytes
must equal the oracle's packed layer bit for bit; a forward over an imported
layer then matches the oracle.  Parity with real checkpoint files is
unpinned: none is available here."""
import numpy as np
import pytest

from oracle import checkpoints as ck
from oracle import formats, moe
from weight_quantized_moe_amd import synth

from gpu_helpers import ATOL_MAX, RTOL_L2, GpuLayer, dev, errors, log, quantized_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_quantized_moe_amd import load_library
    load_library()


def _empty_like_packed(p13, p2):
    import torch
    z = lambda a: None if a is None else torch.full(a.shape, 0xAB if a.dtype == np.uint8 else 7,  # noqa: E731
                                                    dtype=torch.from_numpy(a[:1]).dtype, device="cuda")
    return (z(p13.w), z(p13.scale), z(p2.w), z(p2.scale), z(p13.gscale), z(p2.gscale))


def _src_dev(fmt, t):
    import torch
    if fmt == formats.NVFP4:
        return (dev(t[0]), dev(t[1]), float(t[2]))
    return tuple(dev(np.ascontiguousarray(a)) for a in t)


def _import(fmt, p13, p2, experts, dst, bad=None):
    import torch
    from weight_quantized_moe_amd import import_expert
    for e in experts:
        src = ck.export_expert(fmt, p13, p2, e)
        import_expert(fmt, dst, e, *(_src_dev(fmt, src[n]) for n in ("gate_proj", "up_proj", "down_proj")),
                      bad_zero_points=bad)
    torch.cuda.synchronize()


def _same(dst, p13, p2, experts):
    host = [None if t is None else t.cpu().numpy() for t in dst]
    ref = (p13.w, p13.scale, p2.w, p2.scale, p13.gscale, p2.gscale)
    for name, h, r in zip(("w13", "w13_scale", "w2", "w2_scale", "w13_gscale", "w2_gscale"), host, ref):
        if r is None:
            continue
        for e in experts:
            assert np.array_equal(np.atleast_1d(h[e]).view(np.uint8),
                                  np.atleast_1d(np.asarray(r[e])).view(np.uint8)), f"{name} expert {e}"


@pytest.mark.parametrize("fmt", formats.FORMATS)
def test_import_small_layer_bit_exact_and_forward(fmt):
    import torch
    log(f"[import] {fmt} small layer")
    E, H, I, k, T = 6, 256, 384, 2, 100
    p13, p2 = quantized_layer(fmt, 51, 0, E, H, I)
    dst = _empty_like_packed(p13, p2)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    _import(fmt, p13, p2, range(E), dst, bad if fmt == formats.INT4 else None)
    _same(dst, p13, p2, range(E))
    assert int(bad.item()) == 0
    from weight_quantized_moe_amd import Layer
    lay = Layer(fmt, dst[0], dst[1], dst[2], dst[3], k, w13_gscale=dst[4], w2_gscale=dst[5])
    lg = synth.router_logits(52, 0, T, E)
    x = synth.hidden_bf16(52, 0, T, H)
    out = lay.forward(dev(lg), dev(x.view(np.int16)).view(torch.bfloat16))
    torch.cuda.synchronize()
    y, _, _ = moe.moe_forward(moe.Layer(p13, p2, k), lg, x)
    rel, mx = errors(out.view(torch.int16).cpu().numpy().view(np.uint16), y)
    log(f"    imported layer forward: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= RTOL_L2 and mx <= ATOL_MAX


@pytest.mark.parametrize("fmt", formats.FORMATS)
def test_import_full_shape_experts(fmt):
    """The Clef-Omni shape (128 experts, hidden 2048, intermediate 768): the
    first, a middle and the last expert imported into full-size buffers; the
    other experts' bytes are left as they were."""
    log(f"[import] {fmt} full shape")
    E, H, I = 128, 2048, 768
    g13, g2 = synth.random_packed(fmt, E, 2 * I, H, 61), synth.random_packed(fmt, E, H, I, 62)
    p13 = formats.Packed(fmt, *g13, 2 * I, H)
    p2 = formats.Packed(fmt, *g2, H, I)
    dst = _empty_like_packed(p13, p2)
    experts = (0, 77, 127)
    _import(fmt, p13, p2, experts, dst)
    _same(dst, p13, p2, experts)
    w13 = dst[0][1].cpu().numpy()
    assert np.all(w13 == 0xAB), "an expert that was not imported changed"


def test_gptq_zero_point_check():
    """A group whose zero point is not 8 cannot be represented: the flag is set."""
    import torch
    from weight_quantized_moe_amd import import_expert
    E, H, I = 2, 256, 256
    p13, p2 = quantized_layer(formats.INT4, 53, 0, E, H, I)
    src = ck.export_expert(formats.INT4, p13, p2, 1)
    qw, qz, sc = src["down_proj"]
    qz = qz.copy()
    qz.view(np.uint32)[0, 3] = 0x77767777     # column 28 of group 0: zero point 7
    dst = _empty_like_packed(p13, p2)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    import_expert(formats.INT4, dst, 1, _src_dev(formats.INT4, src["gate_proj"]),
                  _src_dev(formats.INT4, src["up_proj"]), _src_dev(formats.INT4, (qw, qz, sc)),
                  bad_zero_points=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 1
    bad.zero_()
    _import(formats.INT4, p13, p2, [0], dst, bad)
    assert int(bad.item()) == 0
