"""Symmetric int8 KV codec, written from its definition (oracle, tests only).

The pages name INT8 as the cache precision whose per-tensor scale must not
be shared between K and V ("TensorRT对Multi-Query Attention的专项优化支持",
quantisation paragraph: with K and V shared across heads, one common scale
risks collapsing precision, so Q, K and V are calibrated independently; the
TensorRT-LLM guide on sider.ai lists INT8 among the engine precisions). They
give no rounding rule or code range; the reading taken is the plain
symmetric one:

  code(x)  = clamp(round_half_even(float32(x) / float32(scale)), -127, 127)
  value(c) = c * scale

with one IEEE float32 division, NaN input -> code 0, +-inf -> +-127. The
code -128 is never produced (the range is symmetric); pools use it as the
"never written" marker.
"""
from __future__ import annotations

import numpy as np

QMAX = 127
POISON_CODE = -128


def decode(codes) -> np.ndarray:
    """Value of each int8 code as float64 (before the per-head scale)."""
    return np.asarray(codes).astype(np.int64).astype(np.float64)


def encode(y) -> np.ndarray:
    """float32 values -> int8 codes: round half to even, saturate at +-127."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    r = np.rint(np.where(np.isnan(y), 0.0, y))          # numpy rint: half to even
    return np.clip(r, -QMAX, QMAX).astype(np.int8)


def quantize(x_fp16, scale_fp32) -> np.ndarray:
    """Cache-append rule for int8: encode(float32(x) / float32(scale))."""
    x32 = np.asarray(x_fp16).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = x32 / np.asarray(scale_fp32, dtype=np.float32)
    return encode(y.astype(np.float32))
