"""Pins for the oracle's element formats (CPU only).

The e4m3fn decoder is the closed form of the OCP format; it is pinned by the
format's defining points (zero, smallest subnormal, smallest normal, one,
largest finite, NaN codes) and against PyTorch's own float8_e4m3fn
conversion (an independent library routine) on all 256 codes. The encoder is
pinned by round trips, by round-half-to-even midpoints and against PyTorch's
rounding on random in-range values.
"""

import math

import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e4m3_defining_points():
    dec = F.e4m3fn_bits_to_f64
    assert dec(np.uint8([0x00]))[0] == 0.0
    assert math.copysign(1.0, dec(np.uint8([0x80]))[0]) == -1.0  # negative zero
    assert dec(np.uint8([0x01]))[0] == 2.0 ** -9  # smallest subnormal
    assert dec(np.uint8([0x07]))[0] == 7 * 2.0 ** -9  # largest subnormal
    assert dec(np.uint8([0x08]))[0] == 2.0 ** -6  # smallest normal
    assert dec(np.uint8([0x38]))[0] == 1.0
    assert dec(np.uint8([0x3C]))[0] == 1.5
    assert dec(np.uint8([0x7E]))[0] == 448.0
    assert dec(np.uint8([0xFE]))[0] == -448.0
    assert np.isnan(dec(np.uint8([0x7F]))[0]) and np.isnan(dec(np.uint8([0xFF]))[0])
    # no infinities anywhere in the format
    assert not np.isinf(dec(np.arange(256, dtype=np.uint8))).any()
    # exactly two NaN codes
    assert np.isnan(dec(np.arange(256, dtype=np.uint8))).sum() == 2


def test_e4m3_decode_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3fn_bits_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert (both_nan | (ours == ref)).all()
    assert (np.signbit(ours[~both_nan]) == np.signbit(ref[~both_nan])).all()


def test_e4m3_encode_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = F.e4m3fn_bits_to_f64(codes)
    assert (F.e4m3fn_encode(vals) == codes).all()


def test_e4m3_encode_round_half_even_and_saturation():
    enc = F.e4m3fn_encode
    # midway between 1.0 (0x38, even mantissa) and 1.125 (0x39): to 1.0
    assert enc(np.float64([1.0625]))[0] == 0x38
    # midway between 1.125 (0x39) and 1.25 (0x3A, even): to 1.25
    assert enc(np.float64([1.1875]))[0] == 0x3A
    # midway between 0 and the smallest subnormal: to 0 (even)
    assert enc(np.float64([2.0 ** -10]))[0] == 0x00
    # midway between subnormals 1 and 2 units: to 2 (even)
    assert enc(np.float64([1.5 * 2.0 ** -9]))[0] == 0x02
    # midway between 7 units (largest subnormal) and 2^-6: to 2^-6 (code 8)
    assert enc(np.float64([7.5 * 2.0 ** -9]))[0] == 0x08
    # beyond the largest finite value: saturate, keep sign
    assert enc(np.float64([1e6]))[0] == 0x7E
    assert enc(np.float64([-1e6]))[0] == 0xFE
    assert enc(np.float64([470.0]))[0] == 0x7E
    assert enc(np.float64([np.nan]))[0] == 0x7F


def test_e4m3_encode_matches_torch_rounding_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 100, 20000),
                        rng.uniform(-448, 448, 20000), rng.normal(0, 0.01, 20000)])
    x = x.astype(np.float32).astype(np.float64)  # torch converts from float32
    ours = F.e4m3fn_encode(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ours == ref).all()


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 16, 50000, dtype=np.int64).astype(np.uint16)
    ours = F.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert (both_nan | (ours == ref)).all()
    # defining points: 1.0 = 0x3F80, -2.0 = 0xC000, smallest normal 2^-126 = 0x0080
    assert F.bf16_bits_to_f64(np.uint16([0x3F80, 0xC000, 0x0080])).tolist() == [1.0, -2.0, 2.0 ** -126]


@pytest.mark.parametrize("dtype,size", [(F.F32, 4), (F.BF16, 2), (F.FP8, 1)])
def test_itemsize(dtype, size):
    assert F.itemsize(dtype) == size
