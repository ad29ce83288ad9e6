"""The three packed expert-weight formats: quantize, pack, dequantize (oracle).

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

Every projection is a stack of per-expert matrices W[e] of shape [N, K], row
major, K (the input dimension) contiguous.  For the fused gate/up projection
N = 2*I with the gate rows first ("clef-omni-NVFP4" card, section "How it was
made": gate_proj and up_proj are concatenated in the layout transformers uses);
for the down projection N = H and K = I.

Byte layouts are this library's own (the pages give none):

=========  ======================  ==========================  ==============
format     weights                 scales                      global scale
=========  ======================  ==========================  ==============
int4_g128  uint8 [E, N, K/2]       float16 [E, N, K/128]       -
fp8_b128   uint8 [E, N, K] (E4M3)  float32 [E, N/128, K/128]   -
nvfp4_g16  uint8 [E, N, K/2]       uint8 [E, N, K/16] (E4M3)   float32 [E]
=========  ======================  ==========================  ==============

4-bit codes are packed two per byte, even k in the low nibble.

Dequantization (the exact definitions the GPU must reproduce):

* int4_g128: w = (c - 8) * s[n, k // 128]
* fp8_b128:  w = e4m3(b) * sinv[n // 128, k // 128]
* nvfp4_g16: w = e2m1(c) * e4m3(s[n, k // 16]) / g[e]
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import codecs

INT4 = "int4_g128"
FP8 = "fp8_b128"
NVFP4 = "nvfp4_g16"
FORMATS = (INT4, FP8, NVFP4)


@dataclass
class Packed:
    """One stacked projection tensor in a packed format."""

    fmt: str
    w: np.ndarray
    scale: np.ndarray
    gscale: Optional[np.ndarray]
    n: int
    k: int

    @property
    def num_experts(self) -> int:
        return self.w.shape[0]

    def nbytes(self) -> int:
        b = self.w.nbytes + self.scale.nbytes
        if self.gscale is not None:
            b += self.gscale.nbytes
        return b


def check_dims(fmt: str, n: int, k: int) -> None:
    if fmt == INT4:
        ok = k % 128 == 0
    elif fmt == FP8:
        ok = k % 128 == 0 and n % 128 == 0
    elif fmt == NVFP4:
        ok = k % 16 == 0
    else:
        raise ValueError(f"unknown format {fmt!r}")
    if not ok:
        raise ValueError(f"{fmt}: dims N={n} K={k} do not fit the block size")


# --------------------------------------------------------------------------
# INT4 W4A16, symmetric, group 128 along K
# "clef-omni-int4" card: intro and "What was quantized" (W4A16, group size 128,
# symmetric).  The tuned AutoRound rounding is replaced by plain
# round-to-nearest (the signed-gradient tuning needs calibration records); the
# scale rule s = amax/7 and offset-binary codes are this library's reading.
# --------------------------------------------------------------------------

def quantize_int4_expert(w: np.ndarray):
    """w [N, K] -> (codes uint8 [N, K] in 0..15, scales float16 [N, K/128])."""
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    g = w.reshape(n, k // 128, 128)
    amax = np.abs(g).max(axis=2)
    s16 = (amax / 7.0).astype(np.float16)
    s = s16.astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(g / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, -8, 7)
    codes = (q + 8).astype(np.uint8).reshape(n, k)
    return codes, s16


def dequantize_int4_expert(packed_w: np.ndarray, scale: np.ndarray) -> np.ndarray:
    codes = codecs.unpack_nibbles(packed_w)
    n, k = codes.shape
    vals = codecs.decode_int4(codes).reshape(n, k // 128, 128)
    return (vals * scale.astype(np.float64)[:, :, None]).reshape(n, k)


# --------------------------------------------------------------------------
# FP8 E4M3, one FP32 scale per 128x128 block
# "clef-omni-fp8" card, section "Recipe": per 128x128 tile scale = 448/amax,
# round-to-nearest cast to F8_E4M3, store weight plus weight_scale_inv (F32).
# weight_scale_inv is read as 1/scale, the dequantization multiplier.
# --------------------------------------------------------------------------

def quantize_fp8_expert(w: np.ndarray):
    """w [N, K] -> (E4M3 codes uint8 [N, K], sinv float32 [N/128, K/128])."""
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    t = w.reshape(n // 128, 128, k // 128, 128)
    amax = np.abs(t).max(axis=(1, 3))
    scale = np.where(amax > 0, codecs.E4M3_MAX / np.where(amax > 0, amax, 1.0), 1.0)
    sinv = (1.0 / scale).astype(np.float32)
    codes = codecs.quantize_e4m3(t * scale[:, None, :, None]).reshape(n, k)
    return codes, sinv


def dequantize_fp8_expert(codes: np.ndarray, sinv: np.ndarray) -> np.ndarray:
    n, k = codes.shape
    vals = codecs.decode_e4m3(codes).reshape(n // 128, 128, k // 128, 128)
    return (vals * sinv.astype(np.float64)[:, None, :, None]).reshape(n, k)


# --------------------------------------------------------------------------
# NVFP4: E2M1 values, one E4M3 scale per 16 weights along K, one FP32 global
# scale per expert matrix.
# "clef-omni-NVFP4" card, section "How it was made": global = 448*6/amax,
# plain min-max scaling, round-to-nearest-even on the FP4 grid.
# Block scale s_b = E4M3(g * amax_b / 6); codes c = E2M1(w * g / s_b).
# A zero block scale gives zero codes; an all-zero matrix gets g = 1.
# --------------------------------------------------------------------------

def quantize_nvfp4_expert(w: np.ndarray):
    """w [N, K] -> (codes uint8 [N, K] 0..15, block scales uint8 [N, K/16], g)."""
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    amax = np.abs(w).max()
    g = np.float32(codecs.E4M3_MAX * codecs.E2M1_MAX / amax) if amax > 0 else np.float32(1.0)
    g64 = np.float64(g)
    b = w.reshape(n, k // 16, 16)
    amax_b = np.abs(b).max(axis=2)
    s_codes = codecs.quantize_e4m3(g64 * amax_b / codecs.E2M1_MAX)
    s_vals = codecs.decode_e4m3(s_codes)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(s_vals > 0, b * g64 / np.where(s_vals > 0, s_vals, 1.0), 0.0)
    codes = codecs.quantize_e2m1(y).reshape(n, k)
    return codes, s_codes.astype(np.uint8), g


def dequantize_nvfp4_expert(packed_w: np.ndarray, s_codes: np.ndarray, g) -> np.ndarray:
    codes = codecs.unpack_nibbles(packed_w)
    n, k = codes.shape
    vals = codecs.decode_e2m1(codes).reshape(n, k // 16, 16)
    s = codecs.decode_e4m3(s_codes).astype(np.float64)[:, :, None]
    return (vals * s / np.float64(g)).reshape(n, k)


# --------------------------------------------------------------------------
# Stacked tensors
# --------------------------------------------------------------------------

def quantize_expert(fmt: str, w: np.ndarray):
    """Quantize one expert matrix; returns (packed_w, scale, gscale-or-None)."""
    n, k = w.shape
    check_dims(fmt, n, k)
    if fmt == INT4:
        codes, s = quantize_int4_expert(w)
        return codecs.pack_nibbles(codes), s, None
    if fmt == FP8:
        codes, s = quantize_fp8_expert(w)
        return codes, s, None
    codes, s, g = quantize_nvfp4_expert(w)
    return codecs.pack_nibbles(codes), s, g


def empty_packed(fmt: str, e: int, n: int, k: int) -> Packed:
    check_dims(fmt, n, k)
    if fmt == INT4:
        return Packed(fmt, np.zeros((e, n, k // 2), np.uint8),
                      np.zeros((e, n, k // 128), np.float16), None, n, k)
    if fmt == FP8:
        return Packed(fmt, np.zeros((e, n, k), np.uint8),
                      np.ones((e, n // 128, k // 128), np.float32), None, n, k)
    return Packed(fmt, np.zeros((e, n, k // 2), np.uint8),
                  np.zeros((e, n, k // 16), np.uint8), np.ones((e,), np.float32), n, k)


def quantize_stack(fmt: str, experts) -> Packed:
    """Quantize an iterable/array of per-expert float matrices [N, K]."""
    experts = list(experts)
    e = len(experts)
    n, k = np.asarray(experts[0]).shape
    out = empty_packed(fmt, e, n, k)
    for i, w in enumerate(experts):
        pw, s, g = quantize_expert(fmt, np.asarray(w))
        out.w[i] = pw
        out.scale[i] = s
        if g is not None:
            out.gscale[i] = g
    return out


def dequantize_expert(p: Packed, e: int) -> np.ndarray:
    """Float64 [N, K] dequantized weights of expert ``e`` (exact definition)."""
    if p.fmt == INT4:
        return dequantize_int4_expert(p.w[e], p.scale[e])
    if p.fmt == FP8:
        return dequantize_fp8_expert(p.w[e], p.scale[e])
    if p.fmt == NVFP4:
        return dequantize_nvfp4_expert(p.w[e], p.scale[e], p.gscale[e])
    raise ValueError(p.fmt)


def bytes_per_expert(fmt: str, n: int, k: int) -> int:
    """Packed bytes (weights + scales + global scale) of one expert matrix."""
    check_dims(fmt, n, k)
    if fmt == INT4:
        return n * k // 2 + n * (k // 128) * 2
    if fmt == FP8:
        return n * k + (n // 128) * (k // 128) * 4
    return n * k // 2 + n * (k // 16) + 4
