"""ctypes binding of libmoe_quant.so (argument marshalling only).

Every step of the layer runs in the HIP library; PyTorch supplies device
memory (tensors' ``data_ptr()``) and the current HIP stream.  If the library is
missing, constructing a :class:`Layer` raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

HERE = os.path.dirname(os.path.abspath(__file__))

ABI_VERSION = 1
FORMATS = {"int4_g128": 1, "fp8_b128": 2, "nvfp4_g16": 3}
MQ_F32, MQ_BF16 = 0, 1
STAGES = ("route", "permute", "gate_up", "down", "combine")

EXPORTED = (
    "moe_quant_init",
    "moe_quant_workspace_size",
    "moe_quant_forward",
    "moe_quant_forward_noalloc",
    "moe_quant_forward_with_router",
    "moe_quant_forward_w8a8",
    "moe_quant_forward_w4a4",
    "moe_quant_quantize_act",
    "moe_quant_quantize_act_nvfp4",
    "moe_quant_import_expert",
    "moe_quant_check",
    "moe_quant_dequantize",
    "moe_quant_router_logits",
    "moe_quant_destroy",
    "moe_quant_status_string",
    "moe_quant_last_error",
    "moe_quant_abi_version",
)


class MoeQuantError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"moe_quant status {status}: {message}")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_uint32),
        ("num_experts", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("format", ctypes.c_int32),
        ("w13", ctypes.c_void_p),
        ("w13_scale", ctypes.c_void_p),
        ("w13_gscale", ctypes.c_void_p),
        ("w2", ctypes.c_void_p),
        ("w2_scale", ctypes.c_void_p),
        ("w2_gscale", ctypes.c_void_p),
    ]


class SrcProj(ctypes.Structure):
    _fields_ = [
        ("weight", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("qzeros", ctypes.c_void_p),
        ("global_scale", ctypes.c_float),
    ]


class Probe(ctypes.Structure):
    _fields_ = [
        ("topk_ids", ctypes.c_void_p),
        ("topk_w", ctypes.c_void_p),
        ("expert_offsets", ctypes.c_void_p),
        ("sorted_token_ids", ctypes.c_void_p),
        ("inv_pos", ctypes.c_void_p),
        ("h", ctypes.c_void_p),
        ("events", ctypes.c_void_p * (2 * len(STAGES))),
    ]


def library_path() -> str:
    return os.environ.get("MOE_QUANT_LIB", os.path.join(HERE, "libmoe_quant.so"))


_LIB = None


def load_library():
    """Load libmoe_quant.so and declare its signatures (raises if missing)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise MoeQuantError(-1, f"{path} is not built; run weight_quantized_moe_amd.build.build()")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.moe_quant_init.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(vp)]
    lib.moe_quant_init.restype = i32
    lib.moe_quant_workspace_size.argtypes = [vp, i64, ctypes.POINTER(sz)]
    lib.moe_quant_workspace_size.restype = i32
    lib.moe_quant_forward.argtypes = [vp, vp, i32, vp, vp, i64, vp, vp, sz,
                                      ctypes.POINTER(Probe), vp]
    lib.moe_quant_forward.restype = i32
    lib.moe_quant_forward_noalloc.argtypes = [vp, vp, i32, vp, vp, i64, vp, vp, vp]
    lib.moe_quant_forward_noalloc.restype = i32
    lib.moe_quant_forward_with_router.argtypes = [vp, vp, vp, vp, i64, vp, vp, sz, vp,
                                                  ctypes.POINTER(Probe), vp]
    lib.moe_quant_forward_with_router.restype = i32
    lib.moe_quant_import_expert.argtypes = [ctypes.POINTER(LayerDesc), i32, ctypes.POINTER(SrcProj),
                                            ctypes.POINTER(SrcProj), ctypes.POINTER(SrcProj), i32, vp, vp]
    lib.moe_quant_import_expert.restype = i32
    lib.moe_quant_forward_w8a8.argtypes = [vp, vp, i32, vp, vp, i64, vp, vp, sz, ctypes.POINTER(Probe), vp]
    lib.moe_quant_forward_w8a8.restype = i32
    lib.moe_quant_quantize_act.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.moe_quant_quantize_act.restype = i32
    f32 = ctypes.c_float
    lib.moe_quant_forward_w4a4.argtypes = [vp, vp, i32, vp, vp, i64, vp, vp, sz, f32, f32,
                                           ctypes.POINTER(Probe), vp]
    lib.moe_quant_forward_w4a4.restype = i32
    lib.moe_quant_quantize_act_nvfp4.argtypes = [vp, i64, i32, f32, vp, vp, vp]
    lib.moe_quant_quantize_act_nvfp4.restype = i32
    lib.moe_quant_check.argtypes = [vp, vp, vp]
    lib.moe_quant_check.restype = i32
    lib.moe_quant_dequantize.argtypes = [vp, i32, i32, vp, vp]
    lib.moe_quant_dequantize.restype = i32
    lib.moe_quant_router_logits.argtypes = [vp, vp, i64, i32, i32, vp, vp]
    lib.moe_quant_router_logits.restype = i32
    lib.moe_quant_destroy.argtypes = [vp]
    lib.moe_quant_destroy.restype = None
    lib.moe_quant_status_string.argtypes = [i32]
    lib.moe_quant_status_string.restype = ctypes.c_char_p
    lib.moe_quant_last_error.argtypes = []
    lib.moe_quant_last_error.restype = ctypes.c_char_p
    lib.moe_quant_abi_version.argtypes = []
    lib.moe_quant_abi_version.restype = ctypes.c_uint32
    if lib.moe_quant_abi_version() != ABI_VERSION:
        raise MoeQuantError(7, "library ABI version differs from the binding's")
    _LIB = lib
    return lib


def _check(lib, status: int):
    if status != 0:
        raise MoeQuantError(status, lib.moe_quant_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t, name, shape, dtypes, device=None):
    """Raise ValueError unless tensor ``t`` is contiguous, of the given shape
    (None entries match any size) and one of ``dtypes``.  Checked before any
    launch: a wrong shape or a strided view would otherwise become
    out-of-bounds device accesses.  (``device`` is checked by _on_gpu.)"""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != len(shape) or any(s is not None and s != d for s, d in zip(shape, t.shape)):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(device, **tensors):
    """Raise ValueError unless every given tensor is a GPU tensor on ``device``
    (the first one's device if ``device`` is None)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        device = device if device is not None else t.device
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def router_logits(hidden, router_w, out=None, stream=None):
    """Router logits float32 [T, E] = hidden [T, H] . router_w [E, H]^T, both
    bfloat16 on the GPU (moe_quant_router_logits)."""
    import torch
    lib = load_library()
    if hidden.dim() != 2 or router_w.dim() != 2:
        raise ValueError("need hidden [T, H] and router weight [E, H]")
    t, h = hidden.shape
    e = router_w.shape[0]
    _need(hidden, "hidden", (t, h), (torch.bfloat16,))
    _need(router_w, "router_w", (e, h), (torch.bfloat16,))
    if out is None:
        out = torch.empty((t, e), dtype=torch.float32, device=hidden.device)
    _need(out, "out", (t, e), (torch.float32,))
    _on_gpu(None, hidden=hidden, router_w=router_w, out=out)
    _check(lib, lib.moe_quant_router_logits(_ptr(hidden), _ptr(router_w), t, h, e, _ptr(out),
                                            _stream(stream)))
    return out


def import_expert(fmt: str, dst, expert: int, gate, up, down, gptq_zero_offset: int = 1,
                  bad_zero_points=None, stream=None):
    """Write one expert's checkpoint tensors into packed layer buffers
    (moe_quant_import_expert).  ``dst`` = (w13, w13_scale, w2, w2_scale,
    w13_gscale, w2_gscale) GPU tensors in the library layouts (gscales None
    except for NVFP4).  ``gate``/``up``/``down`` per format: FP8 (weight uint8
    [N, K], weight_scale_inv float32 [N/128, K/128]); INT4 auto_gptq (qweight
    int32 [K/8, N], qzeros int32 [K/128, N/8], scales float16 [K/128, N]);
    NVFP4 compressed-tensors (weight_packed uint8 [N, K/2], weight_scale
    uint8 [N, K/16], weight_global_scale float)."""
    import torch
    lib = load_library()
    w13, s13, w2, s2, g13, g2 = dst
    e, n13, _ = w13.shape
    h = w2.shape[1]
    i = n13 // 2
    kdiv = 1 if fmt == "fp8_b128" else 2
    _need(w13, "w13", (e, 2 * i, h // kdiv), (torch.uint8,))
    _need(w2, "w2", (e, h, i // kdiv), (torch.uint8,))

    def src(p, n, k, name):
        if fmt == "fp8_b128":
            w, s = p
            _need(w, f"{name}.weight", (n, k), (torch.uint8,))
            _need(s, f"{name}.weight_scale_inv", (n // 128, k // 128), (torch.float32,))
            _on_gpu(w13.device, w=w, s=s)
            return SrcProj(w.data_ptr(), s.data_ptr(), None, 0.0)
        if fmt == "int4_g128":
            qw, qz, sc = p
            _need(qw, f"{name}.qweight", (k // 8, n), (torch.int32,))
            _need(qz, f"{name}.qzeros", (k // 128, n // 8), (torch.int32,))
            _need(sc, f"{name}.scales", (k // 128, n), (torch.float16,))
            _on_gpu(w13.device, qw=qw, qz=qz, sc=sc)
            return SrcProj(qw.data_ptr(), sc.data_ptr(), qz.data_ptr(), 0.0)
        wp, ws, g = p
        _need(wp, f"{name}.weight_packed", (n, k // 2), (torch.uint8,))
        _need(ws, f"{name}.weight_scale", (n, k // 16), (torch.uint8,))
        _on_gpu(w13.device, wp=wp, ws=ws)
        return SrcProj(wp.data_ptr(), ws.data_ptr(), None, float(g))

    sg, su, sd = src(gate, i, h, "gate_proj"), src(up, i, h, "up_proj"), src(down, h, i, "down_proj")
    d = LayerDesc(ABI_VERSION, e, h, i, 1, FORMATS[fmt], _ptr(w13), _ptr(s13), _ptr(g13),
                  _ptr(w2), _ptr(s2), _ptr(g2))
    if bad_zero_points is not None:
        _need(bad_zero_points, "bad_zero_points", (1,), (torch.int32,))
    _check(lib, lib.moe_quant_import_expert(ctypes.byref(d), expert, ctypes.byref(sg), ctypes.byref(su),
                                            ctypes.byref(sd), gptq_zero_offset, _ptr(bad_zero_points),
                                            _stream(stream)))


def quantize_act(x, codes=None, scales=None, stream=None):
    """Dynamic 1x128 FP8 quantization of float32 rows x [rows, K] on the GPU
    (moe_quant_quantize_act): returns (codes uint8 [rows, K], scales float32
    [rows, K/128])."""
    import torch
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be [rows, K]")
    r, k = x.shape
    _need(x, "x", (r, k), (torch.float32,))
    if codes is None:
        codes = torch.empty((r, k), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((r, k // 128), dtype=torch.float32, device=x.device)
    _need(codes, "codes", (r, k), (torch.uint8,))
    _need(scales, "scales", (r, k // 128), (torch.float32,))
    _on_gpu(None, x=x, codes=codes, scales=scales)
    _check(lib, lib.moe_quant_quantize_act(_ptr(x), r, k, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def quantize_act_nvfp4(x, gscale: float, codes=None, scales=None, stream=None):
    """NVFP4 quantization of float32 rows x [rows, K] with global scale
    ``gscale`` on the GPU (moe_quant_quantize_act_nvfp4): returns (codes uint8
    [rows, K/2], two E2M1 codes per byte, even k in the low nibble; E4M3 block
    scales uint8 [rows, K/16])."""
    import torch
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be [rows, K]")
    r, k = x.shape
    _need(x, "x", (r, k), (torch.float32,))
    if codes is None:
        codes = torch.empty((r, k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((r, k // 16), dtype=torch.uint8, device=x.device)
    _need(codes, "codes", (r, k // 2), (torch.uint8,))
    _need(scales, "scales", (r, k // 16), (torch.uint8,))
    _on_gpu(None, x=x, codes=codes, scales=scales)
    _check(lib, lib.moe_quant_quantize_act_nvfp4(_ptr(x), r, k, float(gscale), _ptr(codes), _ptr(scales),
                                                 _stream(stream)))
    return codes, scales


class Layer:
    """One MoE expert layer over packed weights resident on the GPU.

    ``w13`` [E, 2I, H/2] (4-bit formats) or [E, 2I, H] (FP8) uint8, ``w2``
    [E, H, I/2] or [E, H, I]; scales and global scales as documented in
    ``include/moe_quant.h``.  All tensors must live on the GPU and stay alive
    as long as the layer.
    """

    def __init__(self, fmt: str, w13, w13_scale, w2, w2_scale, top_k: int,
                 w13_gscale=None, w2_gscale=None):
        self._lib = load_library()
        if fmt not in FORMATS:
            raise ValueError(f"unknown format {fmt!r}")
        self.fmt = fmt
        import torch
        if w13.dim() != 3 or w2.dim() != 3:
            raise ValueError("w13 and w2 must be [E, N, K-bytes] tensors")
        e, n13, kb = w13.shape
        e2, h, _ = w2.shape
        if e2 != e:
            raise ValueError("w13 and w2 disagree on the number of experts")
        i = n13 // 2
        kdiv = 1 if fmt == "fp8_b128" else 2
        u8 = (torch.uint8,)
        _need(w13, "w13", (e, 2 * i, h // kdiv), u8)
        _need(w2, "w2", (e, h, i // kdiv), u8)
        if fmt == "int4_g128":
            _need(w13_scale, "w13_scale", (e, 2 * i, h // 128), (torch.float16,))
            _need(w2_scale, "w2_scale", (e, h, i // 128), (torch.float16,))
        elif fmt == "fp8_b128":
            _need(w13_scale, "w13_scale", (e, 2 * i // 128, h // 128), (torch.float32,))
            _need(w2_scale, "w2_scale", (e, h // 128, i // 128), (torch.float32,))
        else:
            _need(w13_scale, "w13_scale", (e, 2 * i, h // 16), u8)
            _need(w2_scale, "w2_scale", (e, h, i // 16), u8)
            _need(w13_gscale, "w13_gscale", (e,), (torch.float32,))
            _need(w2_gscale, "w2_gscale", (e,), (torch.float32,))
        _on_gpu(None, w13=w13, w13_scale=w13_scale, w2=w2, w2_scale=w2_scale,
                w13_gscale=w13_gscale, w2_gscale=w2_gscale)
        self.device = w13.device
        self.num_experts, self.hidden, self.inter, self.top_k = e, h, n13 // 2, top_k
        self._keep = (w13, w13_scale, w2, w2_scale, w13_gscale, w2_gscale)
        d = LayerDesc(ABI_VERSION, e, h, n13 // 2, top_k, FORMATS[fmt],
                      _ptr(w13), _ptr(w13_scale), _ptr(w13_gscale),
                      _ptr(w2), _ptr(w2_scale), _ptr(w2_gscale))
        handle = ctypes.c_void_p()
        _check(self._lib, self._lib.moe_quant_init(ctypes.byref(d), ctypes.byref(handle)))
        self._h = handle

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.moe_quant_destroy(h)
            self._h = None

    def workspace_size(self, num_tokens: int) -> int:
        n = ctypes.c_size_t()
        _check(self._lib, self._lib.moe_quant_workspace_size(self._h, num_tokens, ctypes.byref(n)))
        return n.value

    def workspace(self, num_tokens: int, device=None):
        import torch
        return torch.empty(max(self.workspace_size(num_tokens), 256), dtype=torch.uint8,
                           device=device or self.device)

    def forward(self, logits, hidden, residual=None, out=None, workspace=None,
                probe: Optional[Dict] = None, events=None, stream=None):
        """Enqueue one forward from router logits; returns ``out`` (bfloat16 [T, H])."""
        return self._forward(logits, None, hidden, residual, out, workspace, probe, events,
                             stream, None)

    def forward_w8a8(self, logits, hidden, residual=None, out=None, workspace=None,
                     probe: Optional[Dict] = None, events=None, stream=None):
        """W8A8 forward of an FP8 layer (moe_quant_forward_w8a8): dynamic 1x128
        FP8 activations on the FP8 matrix units."""
        return self._forward(logits, None, hidden, residual, out, workspace, probe, events,
                             stream, None, w8a8=True)

    def forward_w4a4(self, logits, hidden, act_gscale13: float, act_gscale2: float, residual=None,
                     out=None, workspace=None, probe: Optional[Dict] = None, events=None,
                     stream=None):
        """W4A4 forward of an NVFP4 layer (moe_quant_forward_w4a4): hidden rows
        and the SwiGLU intermediate quantized to NVFP4 with the calibrated
        global scales ``act_gscale13`` (gate/up input) and ``act_gscale2``
        (down input)."""
        return self._forward(logits, None, hidden, residual, out, workspace, probe, events,
                             stream, None, w4a4=(float(act_gscale13), float(act_gscale2)))

    def forward_with_router(self, router_w, hidden, residual=None, out=None, workspace=None,
                            logits_out=None, probe: Optional[Dict] = None, events=None,
                            stream=None):
        """Enqueue one forward whose router logits (BF16 gate ``router_w`` [E, H])
        are computed in the same kernel as the top-k; ``logits_out`` (float32
        [T, E]) optionally receives them."""
        return self._forward(None, router_w, hidden, residual, out, workspace, probe, events,
                             stream, logits_out)

    def _forward(self, logits, router_w, hidden, residual, out, workspace, probe, events, stream,
                 logits_out, w8a8=False, w4a4=None):
        import torch
        if hidden.dim() != 2:
            raise ValueError("hidden must be [T, H]")
        t = hidden.shape[0]
        dev = self.device
        bf16 = (torch.bfloat16,)
        _need(hidden, "hidden", (t, self.hidden), bf16)
        if router_w is None:
            _need(logits, "logits", (t, self.num_experts), (torch.float32, torch.bfloat16))
        else:
            _need(router_w, "router_w", (self.num_experts, self.hidden), bf16)
            if logits_out is not None:
                _need(logits_out, "logits_out", (t, self.num_experts), (torch.float32,))
        if residual is not None:
            _need(residual, "residual", (t, self.hidden), bf16)
        if out is None:
            out = torch.empty((t, self.hidden), dtype=torch.bfloat16, device=dev)
        _need(out, "out", (t, self.hidden), bf16)
        shapes = {"topk_ids": ((t, self.top_k), torch.int32), "topk_w": ((t, self.top_k), torch.float32),
                  "expert_offsets": ((self.num_experts + 1,), torch.int32),
                  "sorted_token_ids": ((t * self.top_k,), torch.int32),
                  "inv_pos": ((t * self.top_k,), torch.int32),
                  "h": ((t * self.top_k, self.inter), torch.float16)}
        for name, v in (probe or {}).items():
            if name not in shapes:
                raise ValueError(f"unknown probe output {name!r}")
            if v is not None:
                _need(v, f"probe[{name!r}]", shapes[name][0], (shapes[name][1],))
        if workspace is not None and not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        _on_gpu(dev, hidden=hidden, logits=logits, router_w=router_w, residual=residual, out=out,
                workspace=workspace, logits_out=logits_out,
                **{f"probe[{n!r}]": v for n, v in (probe or {}).items()})
        if workspace is None:
            workspace = self.workspace(t, dev)
        if t > 0 and _nbytes(workspace) < self.workspace_size(t):   # T = 0 enqueues nothing
            raise ValueError(f"workspace holds {_nbytes(workspace)} bytes, "
                             f"{self.workspace_size(t)} needed for {t} tokens")
        pr = None
        if probe is not None or events is not None:
            pr = Probe()
            probe = probe or {}
            for name in ("topk_ids", "topk_w", "expert_offsets", "sorted_token_ids", "inv_pos", "h"):
                setattr(pr, name, _ptr(probe.get(name)))
            if events is not None:
                for i, ev in enumerate(events):
                    pr.events[i] = None if ev is None else ev.cuda_event
        prp = ctypes.byref(pr) if pr is not None else None
        if router_w is None:
            ldt = MQ_F32 if logits.dtype == torch.float32 else MQ_BF16
            if w4a4 is not None:
                st = self._lib.moe_quant_forward_w4a4(
                    self._h, _ptr(logits), ldt, _ptr(hidden), _ptr(residual), t, _ptr(out),
                    _ptr(workspace), _nbytes(workspace), w4a4[0], w4a4[1], prp, _stream(stream))
            else:
                fn = self._lib.moe_quant_forward_w8a8 if w8a8 else self._lib.moe_quant_forward
                st = fn(
                    self._h, _ptr(logits), ldt, _ptr(hidden), _ptr(residual), t, _ptr(out),
                    _ptr(workspace), _nbytes(workspace), prp, _stream(stream))
        else:
            st = self._lib.moe_quant_forward_with_router(
                self._h, _ptr(hidden), _ptr(router_w), _ptr(residual), t, _ptr(out),
                _ptr(workspace), _nbytes(workspace), _ptr(logits_out), prp, _stream(stream))
        _check(self._lib, st)
        return out

    def forward_noalloc(self, logits, hidden, residual=None, out=None, overflow_flag=None,
                        stream=None):
        """Enqueue one forward whose scratch is the library's static device
        array (moe_quant_forward_noalloc); ``overflow_flag``: None or an int32
        tensor of one element that receives the saturation flag."""
        import torch
        if hidden.dim() != 2:
            raise ValueError("hidden must be [T, H]")
        t = hidden.shape[0]
        dev = self.device
        bf16 = (torch.bfloat16,)
        _need(hidden, "hidden", (t, self.hidden), bf16)
        _need(logits, "logits", (t, self.num_experts), (torch.float32, torch.bfloat16))
        if residual is not None:
            _need(residual, "residual", (t, self.hidden), bf16)
        if out is None:
            out = torch.empty((t, self.hidden), dtype=torch.bfloat16, device=dev)
        _need(out, "out", (t, self.hidden), bf16)
        if overflow_flag is not None:
            _need(overflow_flag, "overflow_flag", (1,), (torch.int32,))
        _on_gpu(dev, hidden=hidden, logits=logits, residual=residual, out=out,
                overflow_flag=overflow_flag)
        ldt = MQ_F32 if logits.dtype == torch.float32 else MQ_BF16
        st = self._lib.moe_quant_forward_noalloc(
            self._h, _ptr(logits), ldt, _ptr(hidden), _ptr(residual), t, _ptr(out),
            _ptr(overflow_flag), _stream(stream))
        _check(self._lib, st)
        return out

    def check(self, workspace, stream=None) -> bool:
        """True if the last forward on ``workspace`` saturated its FP16 intermediate."""
        st = self._lib.moe_quant_check(self._h, _ptr(workspace), _stream(stream))
        if st == 9:
            return True
        _check(self._lib, st)
        return False

    def dequantize(self, which: int, expert: int, stream=None):
        import torch
        n, k = (2 * self.inter, self.hidden) if which == 0 else (self.hidden, self.inter)
        out = torch.empty((n, k), dtype=torch.float32, device=self.device)
        _check(self._lib, self._lib.moe_quant_dequantize(self._h, which, expert, _ptr(out),
                                                          _stream(stream)))
        return out
