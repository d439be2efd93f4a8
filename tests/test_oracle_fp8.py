"""Pins for the oracle's e4m3fn codec (CPU only).

Independent references: the OCP spec points stored in tests/golden, torch's
float8_e4m3fn type (a library routine), and brute force over all codes.
"""
import os

import numpy as np
import pytest
import torch

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_spec_points.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                rows.append((int(c, 16), float(v)))
    return rows


def test_decode_spec_points():
    for code, val in _golden():
        got = fp8.decode(np.array([code]))[0]
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_decode_range():
    v = fp8.decode(np.arange(256))
    fin = v[~np.isnan(v)]
    assert fin.max() == 448.0 and fin.min() == -448.0
    assert np.min(np.abs(fin[fin != 0])) == 2.0 ** -9
    assert np.isnan(v).sum() == 2


def _all_fp16():
    x = np.arange(65536, dtype=np.uint16).view(np.float16)
    return x[np.isfinite(x)]


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -8, 0.010296, 3.7, 0.0078125])
def test_quantize_matches_torch_cast(scale):
    x = _all_fp16()
    y = x.astype(np.float32) / np.float32(scale)
    inr = np.abs(y) < 448.0   # torch's cast does not saturate; checked apart
    got = fp8.quantize(x, np.float32(scale))
    ref = torch.from_numpy(y[inr].astype(np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()
    assert np.array_equal(got[inr], ref)


def test_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(5)
    y = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * 50,
        rng.standard_normal(4000).astype(np.float32) * 0.01,
        rng.uniform(-460, 460, 2000).astype(np.float32),
    ])
    codes = fp8.encode(y)
    allc = np.arange(256)
    vals = fp8.decode(allc)
    finite = ~np.isnan(vals)
    fc, fv = allc[finite], vals[finite]
    for yi, ci in zip(y.astype(np.float64), codes):
        if abs(yi) >= 448:
            assert fp8.decode(ci) == np.copysign(448.0, yi)
            continue
        d = np.abs(fv - yi)
        best = d.min()
        cand = fc[d == best]
        # nearest value; on a tie the even mantissa; zero keeps y's sign
        assert abs(fp8.decode(ci) - yi) == best
        if len(set(fv[d == best])) > 1:
            assert ci % 2 == 0


def test_encode_ties_saturation_and_specials():
    cases = [
        (1.0625, 0x38),          # halfway 1.0 / 1.125 -> even (1.0)
        (1.1875, 0x3A),          # halfway 1.125 / 1.25 -> even (1.25)
        (2.0 ** -10, 0x00),      # half of the smallest subnormal -> 0
        (3 * 2.0 ** -10, 0x02),  # halfway 2^-9 / 2^-8 -> even
        (448.0, 0x7E), (449.0, 0x7E), (464.0, 0x7E), (1e6, 0x7E),
        (np.inf, 0x7E), (-1e6, 0xFE), (-np.inf, 0xFE), (0.0, 0x00),
        (-0.0, 0x80), (0.875 * 2.0 ** -6, 0x07), (2.0 ** -6, 0x08),
    ]
    for y, code in cases:
        assert fp8.encode(np.float32(y)) == code, (y, hex(int(fp8.encode(np.float32(y)))))
    assert fp8.encode(np.float32(np.nan)) == 0x7F


def test_roundtrip_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    v = fp8.decode(codes)
    fin = ~np.isnan(v)
    assert np.array_equal(fp8.encode(v[fin].astype(np.float32)), codes[fin])


def test_tabulated_quantize_and_decode_equal_the_direct_rules():
    """quantize() (a table over all fp16 inputs per scale) and decode() (a
    table over the 256 codes) give the bits of the direct definitions."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((50, 4, 64)) * 3).astype(np.float16)
    x[0, 0, :4] = [np.inf, -np.inf, np.nan, 0.0]
    for s in (np.float32(0.0123), np.array([0.01, 0.5, 2.0, 0.01], np.float32)[None, :, None]):
        assert np.array_equal(fp8.quantize(x, s), fp8.quantize_direct(x, s))
    c = rng.integers(0, 256, 5000)
    assert np.array_equal(fp8.decode(c), fp8.decode_closed_form(c), equal_nan=True)
