"""W8A8 block FP8: the FP8 layer with FP8 activations (oracle).

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

The "clef-omni-fp8" card, table "What was quantized", gives the thinker experts
as FP8 E4M3 weights with one FP32 scale per 128x128 block and activations in
BF16 "or dynamic FP8 per 1x128 group in engines"; the same card's section "How
this checkpoint runs" names the engines (vLLM and SGLang load the format), and
its version history reports an FP8 activation replay.  The card gives no
formula for the activation scale.  Reading taken (the plainest one, the
engines' per-token-group quantizer): for each row (a token for the gate/up
input, a grouped row for the down input) and each 128 consecutive input
features,

    s = amax / 448                (FP32 division; amax = 0 gives codes 0)
    code = RNE-to-E4M3(x / s)     (FP32 division, saturated to +-448)

and the layer is the plain MoE layer of oracle.moe over the dequantized
activations code * s, with the SwiGLU intermediate quantized the same way
from its FP32 value (the precision the GEMM accumulates in) before the down
projection.  Weights are the FP8 128x128 format of oracle.formats.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import codecs, formats, moe

GROUP = 128


def quantize_act(x: np.ndarray):
    """Dynamic 1x128 FP8 quantization of rows ``x`` [n, K] (values that are
    FP32 numbers).  Returns (codes uint8 [n, K], scales float32 [n, K/128])."""
    x32 = np.asarray(x, dtype=np.float32)
    n, k = x32.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 128")
    g = x32.reshape(n, k // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where(amax > 0, amax / np.float32(codecs.E4M3_MAX), np.float32(1.0)).astype(np.float32)
        q = (g / s[:, :, None]).astype(np.float32)        # one FP32 division per value
    codes = codecs.quantize_e4m3(q.astype(np.float64)).reshape(n, k)
    return codes, s


def dequantize_act(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Float64 values code * s of quantize_act's output (exact)."""
    n, k = codes.shape
    v = codecs.decode_e4m3(codes).reshape(n, k // GROUP, GROUP)
    return (v * np.asarray(scales, np.float64)[:, :, None]).reshape(n, k)


def expert_w8a8(xq: np.ndarray, w13: np.ndarray, w2: np.ndarray,
                h32: Optional[np.ndarray] = None):
    """One SwiGLU expert on dequantized FP8 activation rows ``xq`` [n, H].
    The intermediate h is rounded to FP32 and quantized per 1x128 before the
    down projection.  ``h32`` replaces h (for a teacher-forced check).
    Returns (expert output [n, H], h in FP32)."""
    i = w13.shape[0] // 2
    gu = xq @ w13.T
    h = moe.silu(gu[:, :i]) * gu[:, i:]
    if h32 is None:
        h32 = h.astype(np.float32)
    hc, hs = quantize_act(h32)
    return dequantize_act(hc, hs) @ w2.T, h32


def down_from_codes(layer: moe.Layer, logits: np.ndarray, hcodes: np.ndarray,
                    hscales: np.ndarray, residual_bf16_bits: Optional[np.ndarray] = None):
    """The layer output from given quantized intermediates (teacher forcing):
    ``hcodes`` uint8 [T*k, I] and ``hscales`` float32 [T*k, I/128] in grouped
    row order (experts ascending, tokens ascending inside one), the down
    projection over their dequantized values and the slot-ordered combine."""
    ids, w = moe.route(logits, layer.top_k)
    perm = moe.permute(ids, layer.num_experts)
    hq = dequantize_act(hcodes, hscales)
    expert_out = np.empty((len(ids) * layer.top_k, layer.hidden), dtype=np.float64)
    for e in range(layer.num_experts):
        lo, hi = perm.offsets[e], perm.offsets[e + 1]
        if hi > lo:
            expert_out[lo:hi] = hq[lo:hi] @ formats.dequantize_expert(layer.w2, e).T
    y = moe.combine(perm, w, expert_out)
    if residual_bf16_bits is not None:
        y = y + moe.bf16_bits_to_f64(residual_bf16_bits)
    return y


def intermediate_w8a8(layer: moe.Layer, logits: np.ndarray, x_bf16_bits: np.ndarray):
    """The SwiGLU intermediate in FP32 [T*k, I], grouped row order, before its
    quantization (for comparing the quantized codes)."""
    ids, _ = moe.route(logits, layer.top_k)
    perm = moe.permute(ids, layer.num_experts)
    x = moe.bf16_bits_to_f64(x_bf16_bits)
    xc, xs = quantize_act(x)
    xq = dequantize_act(xc, xs)
    i = layer.intermediate
    h32 = np.empty((len(ids) * layer.top_k, i), dtype=np.float32)
    for e in range(layer.num_experts):
        lo, hi = perm.offsets[e], perm.offsets[e + 1]
        if hi > lo:
            gu = xq[perm.sorted_token_ids[lo:hi]] @ formats.dequantize_expert(layer.w13, e).T
            h32[lo:hi] = (moe.silu(gu[:, :i]) * gu[:, i:]).astype(np.float32)
    return h32


def moe_forward_w8a8(layer: moe.Layer, logits: np.ndarray, x_bf16_bits: np.ndarray,
                     residual_bf16_bits: Optional[np.ndarray] = None):
    """Float64 W8A8 layer output y [T, H] (plus the residual if given), with
    the routing and combine of moe.moe_forward.  Returns (y, ids, w)."""
    if layer.w13.fmt != formats.FP8:
        raise ValueError("W8A8 applies to the FP8 128x128 format")
    ids, w = moe.route(logits, layer.top_k)
    perm = moe.permute(ids, layer.num_experts)
    x = moe.bf16_bits_to_f64(x_bf16_bits)
    xc, xs = quantize_act(x)
    xq = dequantize_act(xc, xs)
    expert_out = np.empty((len(ids) * layer.top_k, layer.hidden), dtype=np.float64)
    for e in range(layer.num_experts):
        lo, hi = perm.offsets[e], perm.offsets[e + 1]
        if hi == lo:
            continue
        rows = perm.sorted_token_ids[lo:hi]
        w13 = formats.dequantize_expert(layer.w13, e)
        w2 = formats.dequantize_expert(layer.w2, e)
        expert_out[lo:hi], _ = expert_w8a8(xq[rows], w13, w2)
    y = moe.combine(perm, w, expert_out)
    if residual_bf16_bits is not None:
        y = y + moe.bf16_bits_to_f64(residual_bf16_bits)
    return y, ids, w
