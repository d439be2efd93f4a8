"""fp8 e4m3fn codec, written from the format definition (oracle, tests only).

The pages name FP8 only as a precision option ("TensorRT对Multi-Query
Attention的专项优化支持", closing paragraph on Hopper FP8; the TensorRT-LLM
guide on sider.ai, FP16/INT8/FP8 engine section). The reading taken is the
OCP 8-bit floating point format E4M3 in its "fn" form: 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits, no infinities, NaN only at S.1111.111, so
the largest finite magnitude is 1.75 * 2^8 = 448.

  decode(code):  e = bits 6..3, m = bits 2..0
      e == 15 and m == 7  -> NaN
      e == 0              -> (-1)^s * 2^-6 * m/8          (subnormal)
      otherwise           -> (-1)^s * 2^(e-7) * (1 + m/8)

  encode(y), y float32: the finite code whose value is nearest to y, ties to
  the code with an even mantissa (round to nearest even); magnitudes at or
  beyond 448 saturate to +-448; NaN maps to 0x7F; the sign of zero is kept.
"""
from __future__ import annotations

import numpy as np

MAX = 448.0
NAN_CODE = 0x7F


def decode_closed_form(codes) -> np.ndarray:
    """Value of each e4m3fn code as float64 (NaN for 0x7F / 0xFF), from the
    format's definition."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = np.ldexp(m / 8.0, -6)
    nor = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    val = s * np.where(e == 0, sub, nor)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


# The value of every code, from the definition: decode() looks codes up here.
DECODE_TABLE = decode_closed_form(np.arange(256))


def decode(codes) -> np.ndarray:
    """Value of each e4m3fn code as float64 (NaN for 0x7F / 0xFF): the
    definition above, evaluated once per code and looked up."""
    return DECODE_TABLE[np.asarray(codes).astype(np.uint8)]


# All non-negative finite codes 0x00..0x7E in increasing value order.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALS = decode_closed_form(_POS_CODES)
assert np.all(np.diff(_POS_VALS) > 0)


def encode(y) -> np.ndarray:
    """Round float32 values to e4m3fn codes (uint8), RNE, saturating."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    a = np.abs(y)
    sign = np.signbit(y)
    hi = np.searchsorted(_POS_VALS, a, side="left")      # first value >= a
    hi = np.clip(hi, 0, len(_POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALS) - 1)
    d_hi = np.abs(_POS_VALS[hi] - a)
    d_lo = np.abs(a - _POS_VALS[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (_POS_CODES[lo] % 2 == 0))
    mag = np.where(pick_lo, _POS_CODES[lo], _POS_CODES[hi])
    mag = np.where(a >= MAX, 0x7E, mag)
    code = mag | np.where(sign, 0x80, 0)
    code = np.where(np.isnan(y), NAN_CODE, code)
    return code.astype(np.uint8)


def quantize_direct(x_fp16, scale_fp32) -> np.ndarray:
    """Cache-append rule for fp8: encode(float32(x) / float32(scale)).

    The division is one IEEE float32 division (round to nearest even), the
    reading taken for applying a per-head fp32 scale; the independent
    per-tensor K/V scales follow the quantisation paragraph of
    "TensorRT对Multi-Query Attention的专项优化支持".
    """
    x32 = np.asarray(x_fp16).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = x32 / np.asarray(scale_fp32, dtype=np.float32)
    return encode(y.astype(np.float32))


ALL_FP16 = np.arange(65536, dtype=np.uint16).view(np.float16)


def quantize(x_fp16, scale_fp32) -> np.ndarray:
    """quantize_direct for fp16 input, evaluated per scale value as a table
    over all 65536 fp16 inputs (the same arithmetic on the same operands)
    and looked up by each element's bit pattern."""
    x = np.asarray(x_fp16, dtype=np.float16)
    scale = np.asarray(scale_fp32, dtype=np.float32)
    if np.isnan(scale).any():
        return quantize_direct(x, scale)
    shape = np.broadcast_shapes(x.shape, scale.shape)
    bits = np.broadcast_to(x.view(np.uint16), shape)
    out = np.empty(shape, np.uint8)
    for u in np.unique(scale):
        table = quantize_direct(ALL_FP16, u)
        sel = np.broadcast_to(scale == u, shape)
        out[sel] = table[bits[sel]]
    return out
