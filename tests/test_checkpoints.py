"""Pins of the checkpoint source layouts (oracle/checkpoints.py): hand-built
words whose values follow from the formats' definitions, and round trips that
tie each source format's dequantization to the library format's own
(oracle/formats.py, independent code)."""
import numpy as np
import pytest

from oracle import checkpoints as ck
from oracle import codecs, formats

from gpu_helpers import quantized_layer


def test_gptq_word_layout_by_hand():
    """qweight word [i, n] holds k = 8 i + j at bits 4 j (low nibble first);
    qzeros word [g, c] holds column 8 c + j at bits 4 j; auto_gptq stores the
    zero point minus one, so a symmetric group stores 7."""
    K, N = 128, 8
    qweight = np.zeros((K // 8, N), dtype=np.uint32)
    qweight[0, 0] = 0x76543210            # k = 0..7 of column 0: codes 0..7
    qweight[0, 1] = 0xFEDCBA98            # column 1: codes 8..15
    qweight[1, 0] = 0x00000008            # k = 8 of column 0: code 8 (value 0)
    qzeros = np.full((1, 1), 0x77777777, dtype=np.uint32)
    scales = np.full((1, N), 0.5, dtype=np.float16)
    scales[0, 1] = 0.25
    w = ck.dequantize_gptq(qweight.view(np.int32), qzeros.view(np.int32), scales)
    assert w.shape == (N, K)
    np.testing.assert_array_equal(w[0, :8], (np.arange(8) - 8) * 0.5)
    np.testing.assert_array_equal(w[1, :8], (np.arange(8, 16) - 8) * 0.25)
    assert w[0, 8] == 0.0 and w[0, 9] == -4.0          # code 0 elsewhere: (0 - 8) * 0.5
    # the same zero point stored without the offset
    w0 = ck.dequantize_gptq(qweight.view(np.int32), np.full((1, 1), 0x88888888, np.uint32).view(np.int32),
                            scales, offset=0)
    np.testing.assert_array_equal(w0, w)
    # per-column zero points: column 3 (nibble 3 of the word) at zero point 5
    qz = np.full((1, 1), 0x77774777, dtype=np.uint32)
    z = ck.gptq_zero_points(qz.view(np.int32))
    assert list(z[0]) == [8, 8, 8, 5, 8, 8, 8, 8]


def test_fp8_block_and_nvfp4_by_hand():
    w = np.zeros((256, 256), dtype=np.uint8)
    w[0, 0] = 0x38                        # E4M3 1.0
    w[0, 200] = 0xC0                      # E4M3 -2.0
    w[130, 5] = 0x01                      # smallest subnormal 2^-9
    sinv = np.array([[0.25, 3.0], [8.0, 1.0]], dtype=np.float32)
    d = ck.dequantize_fp8_block(w, sinv)
    assert d[0, 0] == 0.25 and d[0, 200] == -6.0 and d[130, 5] == 8.0 * 2.0 ** -9
    assert np.count_nonzero(d) == 3
    packed = np.zeros((1, 8), dtype=np.uint8)
    packed[0, 0] = 0x21                   # k = 0: code 1 (0.5), k = 1: code 2 (1.0)
    packed[0, 7] = 0xF0 | 0x7            # k = 14: code 7 (6.0), k = 15: code 15 (-6.0)
    scale = np.array([[0x38]], dtype=np.uint8)   # E4M3 1.0
    d = ck.dequantize_ct_nvfp4(packed, scale, np.float32(2.0))
    assert d[0, 0] == 0.25 and d[0, 1] == 0.5 and d[0, 14] == 3.0 and d[0, 15] == -3.0


@pytest.mark.parametrize("fmt", formats.FORMATS)
def test_export_round_trip_matches_library_format(fmt):
    """Source tensors exported from a packed layer dequantize, by the source
    format's own definition, to exactly the library format's dequantization."""
    E, H, I = 3, 256, 256
    p13, p2 = quantized_layer(fmt, 21, 0, E, H, I)
    for e in range(E):
        src = ck.export_expert(fmt, p13, p2, e)
        d13 = formats.dequantize_expert(p13, e)
        d2 = formats.dequantize_expert(p2, e)
        np.testing.assert_array_equal(ck.dequantize_source(fmt, src["gate_proj"]), d13[:I])
        np.testing.assert_array_equal(ck.dequantize_source(fmt, src["up_proj"]), d13[I:])
        np.testing.assert_array_equal(ck.dequantize_source(fmt, src["down_proj"]), d2)


def test_gptq_export_shapes_and_dtypes():
    p13, p2 = quantized_layer(formats.INT4, 22, 0, 2, 256, 128)
    qw, qz, sc = ck.export_gptq(p2, 1)
    assert qw.shape == (128 // 8, 256) and qw.dtype == np.int32
    assert qz.shape == (1, 256 // 8) and qz.dtype == np.int32
    assert sc.shape == (1, 256) and sc.dtype == np.float16
    assert np.all(qz.view(np.uint32) == 0x77777777)
    # nibble j of word [i, n] is the library code of k = 8 i + j
    codes = codecs.unpack_nibbles(p2.w[1])
    assert (int(qw.view(np.uint32)[3, 5]) >> 8) & 0xF == codes[5, 8 * 3 + 2]
