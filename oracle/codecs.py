"""Exact code tables and round-to-nearest-even quantizers (oracle, float64).

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

Sources:
* FP8 E4M3 weights: "clef-omni-fp8" model card, intro and section "What was
  quantized" (E4M3 weights) and section "Recipe" (round-to-nearest cast).  The
  bit fields are the OCP 8-bit floating point E4M3FN encoding: bias 7, no
  infinities, codes 0x7F/0xFF are NaN, largest finite magnitude 448.
* FP4 E2M1 values: "clef-omni-NVFP4" model card, section "How it was made"
  (FP4 E2M1 weights, round-to-nearest-even on the FP4 grid).  Bit fields are the
  OCP MX E2M1 encoding: sign bit 3, two exponent bits (bias 1), one mantissa
  bit; magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* INT4: "clef-omni-int4" model card, intro and section "What was quantized"
  (4-bit symmetric weights).  The stored nibble is offset binary, c = q + 8.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def e4m3_decode_table() -> np.ndarray:
    """Value of every E4M3FN code 0..255 as float64 (NaN for 0x7F and 0xFF).

    Closed form: sign * 2**(e-7) * (1 + m/8) for exponent field e >= 1, and
    sign * (m/8) * 2**-6 for e == 0 (subnormals).  e == 15 with m == 7 is NaN.
    """
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            out[code] = s * 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return out


def e2m1_decode_table() -> np.ndarray:
    """Value of every E2M1 code 0..15 as float64.

    Closed form: sign * 2**(e-1) * (1 + m/2) for e >= 1 and sign * m/2 for the
    subnormal e == 0.
    """
    out = np.empty(16, dtype=np.float64)
    for code in range(16):
        s = -1.0 if code & 0x8 else 1.0
        e = (code >> 1) & 0x3
        m = code & 0x1
        if e == 0:
            out[code] = s * (m / 2.0)
        else:
            out[code] = s * 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return out


def int4_decode_table() -> np.ndarray:
    """Value of every offset-binary INT4 nibble: c - 8."""
    return np.arange(16, dtype=np.float64) - 8.0


_E4M3 = e4m3_decode_table()
_E2M1 = e2m1_decode_table()


def _rne_to_grid(x: np.ndarray, mags: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Nearest grid magnitude for |x| (x already clamped into the grid's range).

    ``mags`` is the sorted list of non-negative representable magnitudes and
    ``codes`` their codes.  Ties go to the even code (the one whose mantissa
    LSB, i.e. the code's LSB, is 0): this is IEEE round-half-to-even applied to
    the grid.
    """
    a = np.abs(x)
    hi = np.searchsorted(mags, a, side="left")          # first mag >= a
    hi = np.clip(hi, 0, len(mags) - 1)
    lo = np.clip(hi - 1, 0, len(mags) - 1)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    pick_hi = np.where(tie, (codes[hi] & 1) == 0, pick_hi)
    return np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)


_E4M3_POS_CODES = np.arange(0x7F, dtype=np.int64)      # 0x00..0x7E, monotone
_E4M3_POS_MAGS = _E4M3[:0x7F].copy()
_E2M1_POS_CODES = np.arange(8, dtype=np.int64)
_E2M1_POS_MAGS = _E2M1[:8].copy()


def quantize_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float64 values to E4M3FN codes: saturate to +-448, then RNE.

    Saturation follows the quantizer of the "clef-omni-fp8" card, section
    "Recipe": values are scaled so the tile maximum maps to 448 and cast with
    round-to-nearest; anything outside +-448 is clamped first.
    """
    x = np.asarray(x, dtype=np.float64)
    xc = np.clip(x, -E4M3_MAX, E4M3_MAX)
    mag = _rne_to_grid(xc, _E4M3_POS_MAGS, _E4M3_POS_CODES)
    sign = np.where(np.signbit(xc), 0x80, 0x00).astype(np.uint8)
    return (mag | sign).astype(np.uint8)


def quantize_e2m1(x: np.ndarray) -> np.ndarray:
    """Round float64 values to E2M1 codes: saturate to +-6, then RNE.

    "clef-omni-NVFP4" card, section "How it was made": round-to-nearest-even on
    the FP4 grid.
    """
    x = np.asarray(x, dtype=np.float64)
    xc = np.clip(x, -E2M1_MAX, E2M1_MAX)
    mag = _rne_to_grid(xc, _E2M1_POS_MAGS, _E2M1_POS_CODES)
    sign = np.where(np.signbit(xc), 0x8, 0x0).astype(np.uint8)
    return (mag | sign).astype(np.uint8)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    return _E2M1[np.asarray(codes, dtype=np.uint8) & 0xF]


def decode_int4(codes: np.ndarray) -> np.ndarray:
    return np.asarray(codes, dtype=np.float64) - 8.0


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes two per byte along the last axis: even index in the low
    nibble, odd index in the high nibble (the byte layout of this library)."""
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape[-1] % 2 == 0
    lo = codes[..., 0::2] & 0xF
    hi = codes[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_nibbles`."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out
