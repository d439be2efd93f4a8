"""Decode projection with M == 1 over transposed weights (oracle, tests only).

Source: "优化" on tiny-llm (open-infra-ai.github.io/tiny-llm/performance/
optimization), section 4 (M==1 转置权重 GEMM 快路径): a decode step
multiplies one activation row by a [K, N] weight; storing the weight
transposed, [N, K], lets the lanes of one output read consecutive k. Section
1 (W8A16): int8 weights with fp16 activations, symmetric group-wise scales
(group size 128 by default, no zero point).

What is computed, in float64:

  W[k, n]  = wt[n, k]                                  (fp16 weights)
  W[k, n]  = wt[n, k] * scales_t[n, k // group_size]   (int8 codes)
  y[m, n]  = sum_k x[m, k] * W[k, n]                   (x: [M, K] fp16)

transpose() is the load-time build of the [N, K] copy from a [K, N] weight.
"""
from __future__ import annotations

import numpy as np


def transpose(w):
    """The [N, K] copy of a [K, N] weight (any element type, bit for bit)."""
    w = np.asarray(w)
    return np.ascontiguousarray(w.T)


def dequantize_t(wt, scales_t=None, group_size=128):
    """Transposed weight values [N, K] as float64: fp16 as is, int8 codes
    times the scale of their group of group_size consecutive k."""
    wt = np.asarray(wt)
    if scales_t is None:
        return wt.astype(np.float64)
    N, K = wt.shape
    s = np.asarray(scales_t, np.float64)
    assert s.shape == (N, K // group_size)
    return wt.astype(np.float64) * np.repeat(s, group_size, axis=1)


def gemm_m1(x, wt, scales_t=None, group_size=128):
    """y [M, N] = x [M, K] @ W, with W given transposed as wt [N, K]."""
    x = np.asarray(x).astype(np.float64)
    W_t = dequantize_t(wt, scales_t, group_size)
    return x @ W_t.T


def abs_products(x, wt, scales_t=None, group_size=128):
    """sum_k |x[m, k] * W[k, n]| [M, N]: the scale of the rounding error of
    any summation order of y[m, n]."""
    x = np.abs(np.asarray(x).astype(np.float64))
    W_t = np.abs(dequantize_t(wt, scales_t, group_size))
    return x @ W_t.T
