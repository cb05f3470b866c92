"""Exact element formats of the KV cache and queries — oracle side (test infrastructure).

The pages only say that KV may be held in FP8 (the DeepSeek-V4.1-Flash
write-up, "一、先搞清这个模型特殊在哪": the sliding-window KV is stored in FP8;
the inference-notes page lists ``--kv-cache-dtype``). They do not fix the FP8
variant. The reading taken here is OCP e4m3fn (the format gfx950 converts
natively): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
subnormals at exponent 0, no infinities, and S.1111.111 (0x7F / 0xFF) as NaN.
Largest finite magnitude 1.75 * 2**8 = 448.

bf16 is the upper half of an IEEE binary32, so every bf16 value is exact in
float64; fp32 likewise. The oracle therefore sees exactly the values that the
GPU stores, and tolerances only have to cover accumulation order and output
rounding.
"""

from __future__ import annotations

import numpy as np

F32 = "f32"
BF16 = "bf16"
FP8 = "fp8_e4m3"

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 storage (uint16 / int16 bits) -> float64, exactly.

    A bf16 number is the high 16 bits of a binary32 number with the low 16 bits
    zero, so shifting the bits up and reinterpreting is the definition itself.
    """
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN payloads stay NaN
        return b.view(np.float32).astype(np.float64)


def e4m3fn_bits_to_f64(codes) -> np.ndarray:
    """OCP e4m3fn byte -> float64 by the closed form of the format.

    normal (e >= 1):    (-1)^s * (1 + m/8) * 2^(e-7)
    subnormal (e == 0): (-1)^s * (m/8) * 2^(-6)
    e == 15 and m == 7: NaN (no infinities in this format)
    """
    c = np.asarray(codes).view(np.uint8).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * (m / 8.0) * 2.0 ** -6
    out = np.where(e == 0, sub, normal)
    out = np.where((c & 0x7F) == 0x7F, np.nan, out)
    return out


def e4m3fn_encode(x) -> np.ndarray:
    """float64 -> OCP e4m3fn byte, round-to-nearest-even, saturating at +-448.

    Saturation (instead of producing NaN for large finite inputs) is the
    reading taken for the quantising KV write; NaN inputs map to the NaN code
    with the input's sign.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.abs(x)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    code = np.zeros(a.shape, dtype=np.int64)

    # Subnormal range (a < 2^-6): the codes 0..8 step linearly by 2^-9, and
    # code 8 is exactly the smallest normal 2^-6, so the rounded count of
    # 2^-9 units is the code.
    sub = a < 2.0 ** -6
    code = np.where(sub, np.rint(a / 2.0 ** -9).astype(np.int64), code)

    # Normal range: a = f * 2^e with f in [1, 2); 8 mantissa steps per binade.
    with np.errstate(divide="ignore", invalid="ignore"):
        mant, ex = np.frexp(np.where(sub, 1.0, a))  # a = mant * 2^ex, mant in [0.5, 1)
    e = ex.astype(np.int64) - 1  # a = (2*mant) * 2^e, 2*mant in [1, 2)
    n = np.rint(a / np.exp2((e - 3).astype(np.float64))).astype(np.int64)  # in [8, 16]
    carry = n == 16
    e = np.where(carry, e + 1, e)
    n = np.where(carry, 8, n)
    normal_code = ((e + 7) << 3) | (n - 8)
    normal_code = np.minimum(normal_code, 0x7E)  # a rounded past 448 saturates
    code = np.where(sub, code, normal_code)
    code = np.where(nan, 0x7F, code)
    return (code | sign).astype(np.uint8)


def to_f64(raw, dtype: str) -> np.ndarray:
    """Decode raw storage of the given element type to float64."""
    if dtype == F32:
        return np.asarray(raw).view(np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_bits_to_f64(raw)
    if dtype == FP8:
        return e4m3fn_bits_to_f64(raw)
    raise ValueError(f"unknown dtype {dtype!r}")


def itemsize(dtype: str) -> int:
    return {F32: 4, BF16: 2, FP8: 1}[dtype]
