"""NVFP4 W4A4: the NVFP4 layer with 4-bit activations (oracle).

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

The "clef-omni-fp8" card, table "Which Clef-Omni quant should I use?", lists
an NVFP4 W4A4 build of the same model beside the W4A16 one, for engines with
native FP4 units; the "clef-flash-NVFP4-Hybrid" card, section "Quantization
details", gives the format of its W4A4 layers: NVFP4 on weights and
activations, 16-element groups with FP8 (E4M3) group scales and one FP32
global scale per tensor, the activation global scales calibrated on records.

Reading taken: the input of each projection (the hidden rows into gate/up,
the SwiGLU intermediate into down) is quantized the way the NVFP4 weights are
(two-level scaling, "clef-omni-NVFP4" card, section "How it was made"), with
a given FP32 global scale g per layer and projection input (the calibrated
constant; all experts of the layer share it).  Per row and per 16
consecutive features, in FP32 arithmetic (the pages fix no precision; this is
the kernel's):

    s_b  = e4m3(fp32(fp32(g * amax_b) / 6))      RNE, saturated to 448
    code = e2m1(fp32(fp32(x * g) / s_b))         RNE, saturated to +-6
                                                 (s_b = 0 gives code 0)
    value = e2m1(code) * s_b / g

The layer is then the plain layer of oracle.moe over the values of the
quantized hidden rows, with the SwiGLU intermediate rounded to FP32 (the
precision the GEMM accumulates in) and quantized the same way, with its own
global scale, before the down projection.  Weights are the NVFP4 format of
oracle.formats.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import codecs, formats, moe

GROUP = 16


def quantize_act(x: np.ndarray, g: float):
    """NVFP4 quantization of rows ``x`` [n, K] (values that are FP32 numbers)
    with global scale ``g``.  Returns (codes uint8 [n, K] 0..15, E4M3 block
    scale codes uint8 [n, K/16])."""
    x32 = np.asarray(x, dtype=np.float32)
    g32 = np.float32(g)
    if not np.isfinite(g32) or g32 <= 0:
        raise ValueError("the global scale must be finite and positive")
    n, k = x32.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 16")
    b = x32.reshape(n, k // GROUP, GROUP)
    amax = np.abs(b).max(axis=2)
    with np.errstate(over="ignore"):
        t = (amax * g32).astype(np.float32)
        u = (t / np.float32(codecs.E2M1_MAX)).astype(np.float32)
    s_codes = codecs.quantize_e4m3(u.astype(np.float64))
    s = codecs.decode_e4m3(s_codes).astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        xg = (b * g32).astype(np.float32)
        q = np.where(s > 0, xg / np.where(s > 0, s, np.float32(1)), np.float32(0)).astype(np.float32)
    codes = codecs.quantize_e2m1(q.astype(np.float64)).reshape(n, k)
    return codes, s_codes.astype(np.uint8)


def block_values(codes: np.ndarray, s_codes: np.ndarray) -> np.ndarray:
    """e2m1(code) * s_b per element, float64 [n, K] (exact; the global scale
    not yet divided out)."""
    n, k = codes.shape
    v = codecs.decode_e2m1(codes).reshape(n, k // GROUP, GROUP)
    return (v * codecs.decode_e4m3(s_codes)[:, :, None]).reshape(n, k)


def dequantize_act(codes: np.ndarray, s_codes: np.ndarray, g: float) -> np.ndarray:
    """Float64 values e2m1(code) * s_b / g of quantize_act's output."""
    return block_values(codes, s_codes) / np.float64(np.float32(g))


def quantize_dequantize(x: np.ndarray, g: float) -> np.ndarray:
    """Float64 values of rows ``x`` after NVFP4 quantization with global
    scale ``g``."""
    c, s = quantize_act(x, g)
    return dequantize_act(c, s, g)


def expert_w4a4(xq: np.ndarray, w13: np.ndarray, w2: np.ndarray, g_h: float):
    """One SwiGLU expert on quantized activation rows ``xq`` [n, H] (their
    float64 values): h is rounded to FP32, quantized with global scale
    ``g_h``, and multiplied by the down projection.  Returns (expert output
    [n, H], h in FP32 [n, I])."""
    i = w13.shape[0] // 2
    gu = xq @ w13.T
    h32 = (moe.silu(gu[:, :i]) * gu[:, i:]).astype(np.float32)
    return quantize_dequantize(h32, g_h) @ w2.T, h32


def intermediate_w4a4(layer: moe.Layer, logits: np.ndarray, x_bf16_bits: np.ndarray, g_x: float):
    """The SwiGLU intermediate in FP32 [T*k, I], grouped row order (experts
    ascending, tokens ascending inside one), before its quantization."""
    ids, _ = moe.route(logits, layer.top_k)
    perm = moe.permute(ids, layer.num_experts)
    xq = quantize_dequantize(moe.bf16_bits_to_f64(x_bf16_bits), g_x)
    i = layer.intermediate
    h32 = np.empty((len(ids) * layer.top_k, i), dtype=np.float32)
    for e in range(layer.num_experts):
        lo, hi = perm.offsets[e], perm.offsets[e + 1]
        if hi > lo:
            gu = xq[perm.sorted_token_ids[lo:hi]] @ formats.dequantize_expert(layer.w13, e).T
            h32[lo:hi] = (moe.silu(gu[:, :i]) * gu[:, i:]).astype(np.float32)
    return h32


def down_from_values(layer: moe.Layer, logits: np.ndarray, h_values: np.ndarray,
                     residual_bf16_bits: Optional[np.ndarray] = None):
    """The layer output from given intermediate values (teacher forcing):
    ``h_values`` float64 [T*k, I] in grouped row order, the inputs of the down
    projection as they are (already divided by their global scale); the down
    projection and the slot-ordered combine."""
    ids, w = moe.route(logits, layer.top_k)
    perm = moe.permute(ids, layer.num_experts)
    expert_out = np.empty((len(ids) * layer.top_k, layer.hidden), dtype=np.float64)
    for e in range(layer.num_experts):
        lo, hi = perm.offsets[e], perm.offsets[e + 1]
        if hi > lo:
            expert_out[lo:hi] = h_values[lo:hi] @ formats.dequantize_expert(layer.w2, e).T
    y = moe.combine(perm, w, expert_out)
    if residual_bf16_bits is not None:
        y = y + moe.bf16_bits_to_f64(residual_bf16_bits)
    return y


def moe_forward_w4a4(layer: moe.Layer, logits: np.ndarray, x_bf16_bits: np.ndarray, g_x: float,
                     g_h: float, residual_bf16_bits: Optional[np.ndarray] = None):
    """Float64 W4A4 layer output y [T, H] (plus the residual if given), with
    the routing and combine of moe.moe_forward.  Returns (y, ids, w)."""
    if layer.w13.fmt != formats.NVFP4:
        raise ValueError("W4A4 applies to the NVFP4 format")
    ids, w = moe.route(logits, layer.top_k)
    perm = moe.permute(ids, layer.num_experts)
    xq = quantize_dequantize(moe.bf16_bits_to_f64(x_bf16_bits), g_x)
    expert_out = np.empty((len(ids) * layer.top_k, layer.hidden), dtype=np.float64)
    for e in range(layer.num_experts):
        lo, hi = perm.offsets[e], perm.offsets[e + 1]
        if hi == lo:
            continue
        expert_out[lo:hi], _ = expert_w4a4(xq[perm.sorted_token_ids[lo:hi]],
                                           formats.dequantize_expert(layer.w13, e),
                                           formats.dequantize_expert(layer.w2, e), g_h)
    y = moe.combine(perm, w, expert_out)
    if residual_bf16_bits is not None:
        y = y + moe.bf16_bits_to_f64(residual_bf16_bits)
    return y, ids, w
