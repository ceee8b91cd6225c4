"""Pins of the 8-bit weight formats of the oracle (oracle/formats8.py): the E4M3
table against the format's defining values, hand-worked quantizations with
exact scales (ties included), exact round trips and the error bounds."""
import math

import numpy as np
import pytest

from oracle import formats8 as f8


def test_e4m3_table_defining_values():
    v = f8.E4M3_VALUES
    assert v[0x7E] == 448.0                 # largest finite
    assert v[0x08] == 2.0 ** -6             # smallest normal
    assert v[0x01] == 2.0 ** -9             # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9         # largest subnormal
    assert v[0x38] == 1.0 and v[0x3C] == 1.5 and v[0x39] == 1.125
    assert math.isnan(v[0x7F]) and math.isnan(v[0xFF])
    assert v[0x00] == 0.0 and math.copysign(1.0, v[0x80]) == -1.0
    # sign symmetry, and the 127 non-negative finite codes increase strictly
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])
    assert np.all(np.diff(v[:0x7F]) > 0)
    # every value is a 4-significant-bit number times a power of two
    for c in range(1, 0x7F):
        m, e = math.frexp(v[c])
        assert (m * 16) == int(m * 16)


def _block(values, fill_max):
    """A [1, 64] weight row: the given values, the rest zero, and one element = fill_max
    (so the block's absmax is known)."""
    W = np.zeros((1, 64), dtype=np.float32)
    W[0, :len(values)] = values
    W[0, 63] = fill_max
    return W


def test_int8_hand_worked():
    # absmax 127 makes the scale exactly 1
    codes, s = f8.quantize_int8(_block([2.5, 3.5, -2.5, -127.0, 0.49, -0.5, 126.5], 127.0))
    assert s[0, 0] == 1.0
    assert list(codes[0, :7]) == [2, 4, 0xFE, 0x81, 0, 0, 126]   # half to even, two's complement
    assert codes[0, 63] == 127
    # absmax 254: scale 2, W = 5 -> 2.5 -> 2
    codes, s = f8.quantize_int8(_block([5.0, -7.0], 254.0))
    assert s[0, 0] == 2.0 and list(codes[0, :2]) == [2, 0xFC]


def test_fp8_hand_worked():
    # absmax 448 makes the scale exactly 1
    codes, s = f8.quantize_fp8(_block([1.0, 1.0625, 1.1875, 224.0, -1.0, 2.0 ** -9, 1.4 * 2.0 ** -10, 440.0],
                                      448.0))
    assert s[0, 0] == 1.0
    # 1.0625 lies between 1.0 (0x38) and 1.125 (0x39): tie to the even code; 1.1875 -> 1.25 (0x3A)
    # 224 = 1.75 * 2^7 (0x76); -1 -> 0xB8; 2^-9 -> 0x01; 0.7 * 2^-9 -> 0x01; 440 -> 448 (0x7E)
    assert list(codes[0, :8]) == [0x38, 0x38, 0x3A, 0x76, 0xB8, 0x01, 0x01, 0x7E]
    assert codes[0, 63] == 0x7E
    # absmax 1: scale 1/448 in fp32; W = absmax saturates to 448
    codes, s = f8.quantize_fp8(_block([-1.0], 1.0))
    assert s[0, 0] == np.float32(1.0) / np.float32(448.0)
    assert codes[0, 0] == 0xFE and codes[0, 63] == 0x7E


@pytest.mark.parametrize("fmt", [f8.FMT_INT8, f8.FMT_FP8])
def test_zero_block_and_sign(fmt):
    W = np.zeros((2, 128), dtype=np.float32)
    W[1, 64:] = np.linspace(-1, 1, 64, dtype=np.float32)
    codes, s = f8.quantize(W, fmt)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0 and not codes[0].any() and not codes[1, :64].any()
    Wh = f8.dequantize(codes, s, fmt)
    assert not Wh[0].any()
    assert np.all(np.sign(Wh[1, 64:]) == np.sign(W[1, 64:]) * (Wh[1, 64:] != 0))


@pytest.mark.parametrize("fmt", [f8.FMT_INT8, f8.FMT_FP8])
def test_representable_weights_round_trip_exactly(fmt):
    rng = np.random.default_rng(11)
    qmax = 127 if fmt == f8.FMT_INT8 else 448
    s = np.float32(2.0 ** -7)
    if fmt == f8.FMT_INT8:
        v = rng.integers(-127, 128, size=(3, 128)).astype(np.float64)
    else:
        v = f8.E4M3_VALUES[rng.integers(0, 0x7F, size=(3, 128))] * rng.choice([-1, 1], size=(3, 128))
    v[:, 0] = qmax
    v[:, 64] = -qmax       # every block reaches the full range: its scale is exactly s
    W = (v * float(s)).astype(np.float32)
    codes, sc = f8.quantize(W, fmt)
    assert np.all(sc == s)
    assert np.array_equal(f8.dequantize(codes, sc, fmt), W)


def test_error_bounds():
    rng = np.random.default_rng(12)
    W = (0.02 * rng.standard_normal((16, 256))).astype(np.float32)
    for fmt in (f8.FMT_INT8, f8.FMT_FP8):
        codes, s = f8.quantize(W, fmt)
        err = np.abs(f8.dequantize(codes, s, fmt).astype(np.float64) - W)
        srep = np.repeat(s.astype(np.float64), 64, axis=1)
        if fmt == f8.FMT_INT8:
            assert np.all(err <= 0.5 * srep * (1 + 1e-6) + 1e-12)
        else:
            # half a unit in the last place of E4M3 (2^-4 relative) above the subnormal
            # range, half the subnormal step (2^-10 * s) below it
            bound = np.maximum(np.abs(W) * 2.0 ** -4, 2.0 ** -10 * srep) * (1 + 1e-6)
            assert np.all(err <= bound)
