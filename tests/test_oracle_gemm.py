"""Pins for the oracle's M == 1 decode projection (CPU only).

Checked against pure-Python sums on tiny inputs (brute force), closed forms
(one-hot activations pick a weight column, a diagonal weight scales x, a
constant group scale factors out) and group boundaries worked by hand.
"""
import numpy as np
import pytest

from oracle import gemm


def test_transpose_is_bitwise():
    rng = np.random.default_rng(1)
    w = rng.integers(-128, 128, (5, 7)).astype(np.int8)
    wt = gemm.transpose(w)
    assert wt.shape == (7, 5) and wt.flags.c_contiguous
    for k in range(5):
        for n in range(7):
            assert wt[n, k] == w[k, n]
    h = rng.standard_normal((3, 4)).astype(np.float16)
    assert np.array_equal(gemm.transpose(h).view(np.uint16).T, h.view(np.uint16))


def test_fp16_matches_brute_force_sums():
    rng = np.random.default_rng(2)
    M, K, N = 2, 9, 5
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = rng.standard_normal((K, N)).astype(np.float16)          # [K, N] as stored before
    y = gemm.gemm_m1(x, gemm.transpose(w))
    for m in range(M):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += float(x[m, k]) * float(w[k, n])
            assert abs(y[m, n] - s) < 1e-12


def test_int8_groups_match_brute_force_sums():
    rng = np.random.default_rng(3)
    M, K, N, g = 1, 12, 3, 4
    x = rng.standard_normal((M, K)).astype(np.float16)
    codes = rng.integers(-127, 128, (N, K)).astype(np.int8)     # transposed [N, K]
    scales = rng.uniform(0.01, 0.1, (N, K // g)).astype(np.float32)
    y = gemm.gemm_m1(x, codes, scales, g)
    for n in range(N):
        s = 0.0
        for k in range(K):
            s += float(x[0, k]) * int(codes[n, k]) * float(scales[n, k // g])
        assert abs(y[0, n] - s) < 1e-12
    # the group boundary by hand: k = 3 uses group 0, k = 4 group 1
    W = gemm.dequantize_t(codes, scales, g)
    assert W[1, 3] == int(codes[1, 3]) * float(scales[1, 0])
    assert W[1, 4] == int(codes[1, 4]) * float(scales[1, 1])


def test_closed_forms():
    K, N = 16, 6
    rng = np.random.default_rng(4)
    w = rng.standard_normal((K, N)).astype(np.float16)
    wt = gemm.transpose(w)
    for k in (0, 7, 15):                       # a one-hot x picks row k of W
        x = np.zeros((1, K), np.float16); x[0, k] = 1
        assert np.array_equal(gemm.gemm_m1(x, wt)[0], w[k].astype(np.float64))
    d = np.zeros((K, K), np.float16)           # a diagonal W scales x
    np.fill_diagonal(d, np.arange(1, K + 1))
    x = rng.standard_normal((1, K)).astype(np.float16)
    assert np.array_equal(gemm.gemm_m1(x, gemm.transpose(d))[0],
                          x[0].astype(np.float64) * np.arange(1, K + 1))
    codes = rng.integers(-127, 128, (N, K)).astype(np.int8)  # one scale factors out
    y1 = gemm.gemm_m1(x, codes, np.full((N, K // 8), 0.5, np.float32), 8)
    y2 = gemm.gemm_m1(x, codes.astype(np.float16))
    assert np.allclose(y1, 0.5 * y2, rtol=0, atol=1e-12)


def test_abs_products_bound_the_sum():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 64)).astype(np.float16)
    codes = rng.integers(-127, 128, (10, 64)).astype(np.int8)
    s = rng.uniform(0.01, 0.1, (10, 2)).astype(np.float32)
    y = gemm.gemm_m1(x, codes, s, 32)
    a = gemm.abs_products(x, codes, s, 32)
    assert np.all(np.abs(y) <= a + 1e-12) and np.all(a >= 0)
    # equality when every product is non-negative
    assert np.allclose(gemm.gemm_m1(np.abs(x), np.abs(codes), s, 32),
                       gemm.abs_products(x, codes, s, 32), rtol=1e-15, atol=0)
