"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching the GPU (runs without a GPU)."""
import ctypes
import os
import re

import pytest

from weight_quantized_moe_amd import binding
from weight_quantized_moe_amd.binding import LayerDesc, Probe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_quant.h")

MQ_OK, MQ_E_NULL, MQ_E_SHAPE, MQ_E_ALIGN, MQ_E_FORMAT, MQ_E_DTYPE, MQ_E_WORKSPACE, MQ_E_ABI = range(8)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.fail("libmoe_quant.so is not built (run __graft_entry__.build())")
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_quant_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.moe_quant_abi_version() == 1


def test_struct_layouts_match_header():
    # mq_layer_desc: 6 x 4-byte fields then 6 pointers
    assert ctypes.sizeof(LayerDesc) == 24 + 6 * 8
    assert LayerDesc.w13.offset == 24
    # mq_probe: 6 pointers then 10 event pointers
    assert ctypes.sizeof(Probe) == 16 * 8


def _desc(fmt=1, e=8, h=256, i=128, k=2, base=0x10000, gscale=False, abi=1):
    g = base + 0x4000 if (fmt == 3 or gscale) else None
    g2 = base + 0x5000 if (fmt == 3 or gscale) else None
    return LayerDesc(abi, e, h, i, k, fmt, base, base + 0x1000, g, base + 0x2000, base + 0x3000, g2)


def _init(lib, d):
    h = ctypes.c_void_p()
    st = lib.moe_quant_init(ctypes.byref(d) if d is not None else None, ctypes.byref(h))
    return st, h


def test_init_accepts_valid_descriptors(lib):
    for fmt in (1, 2, 3):
        st, h = _init(lib, _desc(fmt))
        assert st == MQ_OK, lib.moe_quant_last_error()
        lib.moe_quant_destroy(h)


@pytest.mark.parametrize("change,expect", [
    (dict(abi=2), MQ_E_ABI),
    (dict(fmt=0), MQ_E_FORMAT),
    (dict(fmt=4), MQ_E_FORMAT),
    (dict(e=0), MQ_E_SHAPE),
    (dict(e=513), MQ_E_SHAPE),
    (dict(k=0), MQ_E_SHAPE),
    (dict(k=9, e=8), MQ_E_SHAPE),
    (dict(h=200), MQ_E_SHAPE),
    (dict(i=64), MQ_E_SHAPE),
    (dict(fmt=3, h=272), MQ_E_SHAPE),
    (dict(h=4736), MQ_E_SHAPE),           # decode rows of 4736 values exceed 160 KiB of LDS
    (dict(i=4736), MQ_E_SHAPE),
    (dict(fmt=2, h=65536, i=128), MQ_E_SHAPE),
    (dict(base=0x10008), MQ_E_ALIGN),
    (dict(fmt=1, gscale=True), MQ_E_NULL),
])
def test_init_rejects(lib, change, expect):
    st, h = _init(lib, _desc(**change))
    assert st == expect, (change, st, lib.moe_quant_last_error())
    assert h.value is None
    assert lib.moe_quant_last_error()


def test_init_accepts_the_largest_dimensions(lib):
    for fmt in (1, 2, 3):
        st, h = _init(lib, _desc(fmt, h=4608, i=4608))
        assert st == MQ_OK, lib.moe_quant_last_error()
        lib.moe_quant_destroy(h)


def test_init_null_and_missing_pointers(lib):
    st, _ = _init(lib, None)
    assert st == MQ_E_NULL
    d = _desc(3)
    d.w13_gscale = None
    assert _init(lib, d)[0] == MQ_E_NULL
    d = _desc(1)
    d.w2 = None
    assert _init(lib, d)[0] == MQ_E_NULL


def test_status_strings(lib):
    for s in range(10):
        assert lib.moe_quant_status_string(s).startswith(b"MQ_")


def test_workspace_size_grows_with_tokens(lib):
    st, h = _init(lib, _desc(1, e=128, h=2048, i=768, k=8))
    assert st == MQ_OK
    n = ctypes.c_size_t()
    sizes = []
    for t in (0, 1, 64, 4096):
        assert lib.moe_quant_workspace_size(h, t, ctypes.byref(n)) == MQ_OK
        sizes.append(n.value)
    assert sizes == sorted(sizes) and sizes[0] > 0
    # dominant terms: the per-slot FP16 partials, the FP16 intermediate and
    # the FP16 staged hidden rows
    r = 4096 * 8
    assert sizes[-1] >= r * 2048 * 2 + r * 768 * 2 + 4096 * 2048 * 2
    assert lib.moe_quant_workspace_size(h, -1, ctypes.byref(n)) == MQ_E_SHAPE
    lib.moe_quant_destroy(h)


def test_forward_rejects_before_any_launch(lib):
    st, h = _init(lib, _desc(1))
    assert st == MQ_OK
    n = ctypes.c_size_t()
    lib.moe_quant_workspace_size(h, 64, ctypes.byref(n))
    ws_need = n.value
    P = 0x100000

    def fwd(handle=h, logits=P, dtype=0, hidden=P + 0x10000, res=None, t=64, out=P + 0x20000,
            ws=P + 0x40000, wsb=ws_need):
        return lib.moe_quant_forward(handle, logits, dtype, hidden, res, t, out, ws, wsb, None, None)

    assert fwd(handle=None) == MQ_E_NULL
    assert fwd(dtype=7) == MQ_E_DTYPE
    assert fwd(t=-1) == MQ_E_SHAPE
    assert fwd(t=0, logits=None, hidden=None, out=None, ws=None) == MQ_OK
    assert fwd(hidden=None) == MQ_E_NULL
    assert fwd(logits=P + 4) == MQ_E_ALIGN
    assert fwd(res=P + 0x30002) == MQ_E_ALIGN
    assert fwd(ws=None) == MQ_E_WORKSPACE
    assert fwd(ws=P + 0x40010) == MQ_E_ALIGN
    assert fwd(wsb=ws_need - 1) == MQ_E_WORKSPACE
    lib.moe_quant_destroy(h)


def test_forward_noalloc_rejects_before_any_launch(lib):
    """The allocation-free forward checks its arguments and the scratch bound
    on the host before it touches the GPU."""
    st, h = _init(lib, _desc(1, e=128, h=2048, i=768, k=8))
    assert st == MQ_OK
    P = 0x100000
    f = lib.moe_quant_forward_noalloc
    assert f(None, P, 0, P, None, 64, P, None, None) == MQ_E_NULL
    assert f(h, P, 0, P, None, -1, P, None, None) == MQ_E_SHAPE
    assert f(h, None, 0, None, None, 0, None, None, None) == MQ_OK        # T = 0: nothing to do
    assert f(h, P, 0, P, None, 64, P, P + 2, None) == MQ_E_ALIGN         # overflow flag
    # 4096 tokens need ~200 MiB of scratch, above the static 64 MiB
    assert f(h, P, 0, P, None, 4096, P, None, None) == MQ_E_WORKSPACE
    assert b"64" in lib.moe_quant_last_error() or b"scratch" in lib.moe_quant_last_error()
    n = ctypes.c_size_t()
    assert lib.moe_quant_workspace_size(h, 1300, ctypes.byref(n)) == MQ_OK
    assert n.value <= 64 << 20          # the documented capacity: ~1350 tokens at this shape
    assert lib.moe_quant_workspace_size(h, 1400, ctypes.byref(n)) == MQ_OK
    assert n.value > 64 << 20
    lib.moe_quant_destroy(h)


def test_forward_with_router_rejects_before_any_launch(lib):
    P = 0x100000
    f = lib.moe_quant_forward_with_router
    st, h = _init(lib, _desc(1, e=128, h=2048, i=768, k=8))
    assert st == MQ_OK
    n = ctypes.c_size_t()
    lib.moe_quant_workspace_size(h, 64, ctypes.byref(n))
    ws = n.value
    assert f(h, P, None, None, 64, P, P + 0x100000, ws, None, None, None) == MQ_E_NULL   # no router
    assert f(h, P, P + 8, None, 64, P, P + 0x100000, ws, None, None, None) == MQ_E_ALIGN
    assert f(h, P, P, None, 64, P, P + 0x100000, ws - 1, None, None, None) == MQ_E_WORKSPACE
    assert f(h, P, P, None, 64, P, P + 0x100000, ws, P + 2, None, None) == MQ_E_ALIGN    # logits_out
    assert f(h, P, P, None, 0, P, None, 0, None, None, None) == MQ_OK                     # T = 0
    lib.moe_quant_destroy(h)
    st, h = _init(lib, _desc(1, e=300, k=8))          # more experts than the fused router holds
    assert st == MQ_OK
    assert f(h, P, P, None, 4, P, P + 0x100000, 1 << 30, None, None, None) == MQ_E_SHAPE
    lib.moe_quant_destroy(h)


def test_import_expert_rejects_before_any_launch(lib):
    from weight_quantized_moe_amd.binding import SrcProj
    f = lib.moe_quant_import_expert
    P = 0x100000
    ok = SrcProj(P, P + 0x1000, P + 0x2000, 1.0)
    for fmt in (1, 2, 3):
        d = _desc(fmt)
        assert f(ctypes.byref(d), 8, ctypes.byref(ok), ctypes.byref(ok), ctypes.byref(ok), 1, None, None) == MQ_E_SHAPE
        assert f(ctypes.byref(d), -1, ctypes.byref(ok), ctypes.byref(ok), ctypes.byref(ok), 1, None, None) == MQ_E_SHAPE
        nul = SrcProj(None, P, P, 1.0)
        assert f(ctypes.byref(d), 0, ctypes.byref(ok), ctypes.byref(nul), ctypes.byref(ok), 1, None, None) == MQ_E_NULL
        mis = SrcProj(P + 8, P, P, 1.0)
        assert f(ctypes.byref(d), 0, ctypes.byref(mis), ctypes.byref(ok), ctypes.byref(ok), 1, None, None) == MQ_E_ALIGN
        bad_desc = _desc(fmt, h=200)
        assert f(ctypes.byref(bad_desc), 0, ctypes.byref(ok), ctypes.byref(ok), ctypes.byref(ok), 1, None, None) == MQ_E_SHAPE
    # INT4 needs qzeros
    noz = SrcProj(P, P, None, 0.0)
    d = _desc(1)
    assert f(ctypes.byref(d), 0, ctypes.byref(noz), ctypes.byref(ok), ctypes.byref(ok), 1, None, None) == MQ_E_NULL
    # NVFP4: gate and up share W13's global scale
    d = _desc(3)
    g1, g2 = SrcProj(P, P, None, 2.0), SrcProj(P, P, None, 3.0)
    assert f(ctypes.byref(d), 0, ctypes.byref(g1), ctypes.byref(g2), ctypes.byref(g1), 1, None, None) == MQ_E_FORMAT


def test_forward_w8a8_and_quantize_act_reject_before_any_launch(lib):
    P = 0x100000
    st, h = _init(lib, _desc(1))               # INT4: W8A8 needs the FP8 format
    assert st == MQ_OK
    f = lib.moe_quant_forward_w8a8
    assert f(h, P, 0, P, None, 4, P, P, 1 << 20, None, None) == 4          # MQ_E_FORMAT
    lib.moe_quant_destroy(h)
    st, h = _init(lib, _desc(2))
    assert f(h, P, 0, P, None, 4, P, P, 16, None, None) == MQ_E_WORKSPACE
    lib.moe_quant_destroy(h)
    q = lib.moe_quant_quantize_act
    assert q(P, 4, 200, P, P, None) == MQ_E_SHAPE
    assert q(P, -1, 256, P, P, None) == MQ_E_SHAPE
    assert q(None, 0, 256, None, None, None) == MQ_OK
    assert q(None, 4, 256, P, P, None) == MQ_E_NULL
    assert q(P + 4, 4, 256, P, P, None) == MQ_E_ALIGN


def test_forward_w4a4_and_quantize_act_nvfp4_reject_before_any_launch(lib):
    P = 0x100000
    st, h = _init(lib, _desc(2))               # FP8: W4A4 needs the NVFP4 format
    assert st == MQ_OK
    f = lib.moe_quant_forward_w4a4
    assert f(h, P, 0, P, None, 4, P, P, 1 << 20, 1.0, 1.0, None, None) == MQ_E_FORMAT
    lib.moe_quant_destroy(h)
    st, h = _init(lib, _desc(3))
    assert st == MQ_OK
    for g13, g2 in ((0.0, 1.0), (1.0, -2.0), (float("inf"), 1.0), (1.0, float("nan"))):
        assert f(h, P, 0, P, None, 4, P, P, 1 << 20, g13, g2, None, None) == MQ_E_SHAPE
    assert f(h, P, 0, P, None, 4, P, P, 16, 1.0, 1.0, None, None) == MQ_E_WORKSPACE
    assert f(h, P, 0, P, None, 0, P, P, 0, 1.0, 1.0, None, None) == MQ_OK   # T = 0 enqueues nothing
    lib.moe_quant_destroy(h)
    q = lib.moe_quant_quantize_act_nvfp4
    assert q(P, 4, 200, 1.0, P, P, None) == MQ_E_SHAPE        # K not a multiple of 16
    assert q(P, -1, 256, 1.0, P, P, None) == MQ_E_SHAPE
    assert q(P, 4, 256, 0.0, P, P, None) == MQ_E_SHAPE
    assert q(None, 0, 256, 1.0, None, None, None) == MQ_OK
    assert q(None, 4, 256, 1.0, P, P, None) == MQ_E_NULL
    assert q(P + 4, 4, 256, 1.0, P, P, None) == MQ_E_ALIGN
    assert q(P, 4, 256, 1.0, P + 2, P, None) == MQ_E_ALIGN


def test_dequantize_rejects(lib):
    st, h = _init(lib, _desc(2))
    assert st == MQ_OK
    assert lib.moe_quant_dequantize(h, 2, 0, 0x1000, None) == MQ_E_SHAPE
    assert lib.moe_quant_dequantize(h, 0, 8, 0x1000, None) == MQ_E_SHAPE
    assert lib.moe_quant_dequantize(h, 0, 0, None, None) == MQ_E_NULL
    assert lib.moe_quant_dequantize(h, 0, 0, 0x1004, None) == MQ_E_ALIGN
    lib.moe_quant_destroy(h)


def test_router_logits_rejects_before_any_launch(lib):
    """Shape, NULL and alignment errors return before anything is enqueued."""
    f = lib.moe_quant_router_logits
    P = 0x100000
    assert f(P, P + 0x10000, 0, 2048, 128, P + 0x20000, None) == MQ_OK     # T = 0: nothing to do
    assert f(None, None, 0, 2048, 128, None, None) == MQ_OK
    assert f(P, P + 0x10000, -1, 2048, 128, P + 0x20000, None) == MQ_E_SHAPE
    assert f(P, P + 0x10000, 4, 2000, 128, P + 0x20000, None) == MQ_E_SHAPE  # H % 64
    assert f(P, P + 0x10000, 4, 2048, 0, P + 0x20000, None) == MQ_E_SHAPE
    assert f(None, P + 0x10000, 4, 2048, 128, P + 0x20000, None) == MQ_E_NULL
    assert f(P, P + 0x10000, 4, 2048, 128, None, None) == MQ_E_NULL
    assert f(P + 2, P + 0x10000, 4, 2048, 128, P + 0x20000, None) == MQ_E_ALIGN
    assert f(P, P + 0x10000, 4, 2048, 128, P + 0x20004, None) == MQ_E_ALIGN
