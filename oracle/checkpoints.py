"""Checkpoint source layouts of the three quantized releases (oracle).

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

The model cards name the tensor layouts their checkpoints use, per expert
linear layer (gate_proj, up_proj, down_proj; out_features N, in_features K):

* FineGrainedFP8 ("clef-omni-fp8" card, intro and section "Recipe"): ``weight``
  E4M3 [N, K] and ``weight_scale_inv`` FP32 [N/128, K/128], the dequantization
  multiplier of each 128x128 tile: w[n, k] = e4m3(weight[n, k]) *
  weight_scale_inv[n // 128, k // 128].
* INT4 in auto_gptq packing ("clef-omni-int4" card, section "What was
  quantized": auto_round format, auto_gptq packing, group size 128,
  symmetric).  The GPTQ tensors of a linear layer: ``qweight`` int32 [K/8, N]
  whose word [i, n] holds the 4-bit codes of k = 8 i + j (j = 0..7) at bits
  4 j .. 4 j + 3; ``qzeros`` int32 [K/128, N/8] whose word [g, c] holds the
  zero point of column n = 8 c + j at bits 4 j; ``scales`` FP16 [K/128, N].
  w[k, n] = (q[k, n] - (z[g, n] + offset)) * scales[g, n], g = k // 128, where
  ``offset`` is 1 in the auto_gptq convention (the stored zero point is one
  less than the zero point) and 0 otherwise.  A symmetric 4-bit group has
  zero point 8.
* compressed-tensors NVFP4 ("clef-omni-NVFP4" card, section "How it was
  made"): ``weight_packed`` uint8 [N, K/2] (E2M1 codes two per byte, the even
  k in the low nibble), ``weight_scale`` E4M3 [N, K/16], ``weight_global_scale``
  FP32 (448 * 6 / amax): w = e2m1(code) * e4m3(weight_scale) /
  weight_global_scale.  The card's quantizer concatenates gate_proj and
  up_proj before quantizing, so the two share one global scale.

The bit-level conventions (nibble order inside the GPTQ words, the zero-point
offset, the FP4 nibble order) are the public formats' own; the cards name the
formats without spelling them out.  Real checkpoint files are not available
here, so parity with them is unpinned; these functions define the layouts and
produce synthetic checkpoints from the library's packed format.
"""
from __future__ import annotations

import numpy as np

from . import codecs, formats

GPTQ_ZERO_OFFSET = 1   # auto_gptq convention: zero point = stored value + 1


# --------------------------------------------------------------- FineGrainedFP8

def dequantize_fp8_block(weight: np.ndarray, scale_inv: np.ndarray) -> np.ndarray:
    """Float64 [N, K] of a FineGrainedFP8 linear layer."""
    n, k = weight.shape
    vals = codecs.decode_e4m3(weight).reshape(n // 128, 128, k // 128, 128)
    return (vals * np.asarray(scale_inv, np.float64)[:, None, :, None]).reshape(n, k)


# --------------------------------------------------------------- GPTQ INT4

def gptq_codes(qweight: np.ndarray) -> np.ndarray:
    """Unsigned 4-bit codes q [K, N] of a GPTQ ``qweight`` int32 [K/8, N]."""
    u = np.asarray(qweight).astype(np.uint32)
    kk, n = u.shape
    q = np.empty((kk * 8, n), dtype=np.uint8)
    for j in range(8):
        q[j::8] = (u >> (4 * j)) & 0xF
    return q


def gptq_zero_points(qzeros: np.ndarray, offset: int = GPTQ_ZERO_OFFSET) -> np.ndarray:
    """Zero points z [K/128, N] of a GPTQ ``qzeros`` int32 [K/128, N/8]."""
    u = np.asarray(qzeros).astype(np.uint32)
    g, c = u.shape
    z = np.empty((g, c * 8), dtype=np.int64)
    for j in range(8):
        z[:, j::8] = (u >> (4 * j)) & 0xF
    return z + offset


def dequantize_gptq(qweight, qzeros, scales, offset: int = GPTQ_ZERO_OFFSET) -> np.ndarray:
    """Float64 [N, K] (the library's orientation) of a GPTQ linear layer."""
    q = gptq_codes(qweight).astype(np.int64)              # [K, N]
    z = gptq_zero_points(qzeros, offset)                   # [K/128, N]
    s = np.asarray(scales).astype(np.float64)              # [K/128, N]
    k = q.shape[0]
    g = np.arange(k) // 128
    return ((q - z[g]) * s[g]).T


def export_gptq(p: formats.Packed, e: int, offset: int = GPTQ_ZERO_OFFSET):
    """One expert matrix of an INT4 ``Packed`` as GPTQ tensors (qweight, qzeros,
    scales): codes c = q + 8 are the unsigned GPTQ codes of a symmetric group
    with zero point 8."""
    assert p.fmt == formats.INT4
    c = codecs.unpack_nibbles(p.w[e]).astype(np.uint32)    # [N, K]
    n, k = c.shape
    ct = c.T                                               # [K, N]
    qweight = np.zeros((k // 8, n), dtype=np.uint32)
    for j in range(8):
        qweight |= ct[j::8] << (4 * j)
    zstore = np.uint32(8 - offset)
    qzeros = np.zeros((k // 128, n // 8), dtype=np.uint32)
    for j in range(8):
        qzeros |= zstore << (4 * j)
    scales = np.ascontiguousarray(p.scale[e].T)            # [K/128, N] float16
    return qweight.view(np.int32), qzeros.view(np.int32), scales


# --------------------------------------------------------------- compressed-tensors NVFP4

def dequantize_ct_nvfp4(weight_packed, weight_scale, global_scale) -> np.ndarray:
    """Float64 [N, K] of a compressed-tensors NVFP4 linear layer."""
    codes = codecs.unpack_nibbles(weight_packed)
    n, k = codes.shape
    vals = codecs.decode_e2m1(codes).reshape(n, k // 16, 16)
    s = codecs.decode_e4m3(weight_scale)[:, :, None]
    return (vals * s / np.float64(np.float32(global_scale))).reshape(n, k)


# --------------------------------------------------------------- per expert, three projections

def export_expert(fmt: str, p13: formats.Packed, p2: formats.Packed, e: int):
    """Expert ``e`` of a packed layer as per-projection checkpoint tensors:
    {"gate_proj": ..., "up_proj": ..., "down_proj": ...}, each the source
    format's tensors (FP8: weight, weight_scale_inv; INT4: qweight, qzeros,
    scales; NVFP4: weight_packed, weight_scale, weight_global_scale)."""
    i = p13.n // 2
    out = {}
    if fmt == formats.FP8:
        w, s = p13.w[e], p13.scale[e]
        out["gate_proj"] = (w[:i].copy(), s[:i // 128].copy())
        out["up_proj"] = (w[i:].copy(), s[i // 128:].copy())
        out["down_proj"] = (p2.w[e].copy(), p2.scale[e].copy())
    elif fmt == formats.INT4:
        for name, rows in (("gate_proj", slice(0, i)), ("up_proj", slice(i, 2 * i))):
            sub = formats.Packed(fmt, p13.w[e:e + 1, rows], p13.scale[e:e + 1, rows], None, i, p13.k)
            out[name] = export_gptq(sub, 0)
        out["down_proj"] = export_gptq(p2, e)
    elif fmt == formats.NVFP4:
        w, s, g = p13.w[e], p13.scale[e], np.float32(p13.gscale[e])
        out["gate_proj"] = (w[:i].copy(), s[:i].copy(), g)
        out["up_proj"] = (w[i:].copy(), s[i:].copy(), g)
        out["down_proj"] = (p2.w[e].copy(), p2.scale[e].copy(), np.float32(p2.gscale[e]))
    else:
        raise ValueError(fmt)
    return out


def dequantize_source(fmt: str, tensors) -> np.ndarray:
    """Float64 [N, K] of one source projection by its own format's definition."""
    if fmt == formats.FP8:
        return dequantize_fp8_block(*tensors)
    if fmt == formats.INT4:
        return dequantize_gptq(*tensors)
    if fmt == formats.NVFP4:
        return dequantize_ct_nvfp4(*tensors)
    raise ValueError(fmt)
