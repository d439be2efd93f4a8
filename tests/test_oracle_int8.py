"""Pins for the oracle's int8 cache codec and its use in append and decode
(CPU only).

The codec is checked against torch's own round-half-even and clamp (a
library routine) on every fp16 bit pattern, against hand-written tie and
saturation points, and by brute force against the nearest code; the paged
path against hand-gathered, hand-dequantised values fed to torch SDPA.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import int8
from tests.oracle_cases import contiguous_reference_sdpa, oracle_pools
from tests.test_oracle_attention import _tile_pos_k, _tile_pos_v
from workloads import make_case


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -8, 0.010296, 3.7, 1.0 / 127])
def test_quantize_matches_torch_on_every_fp16_pattern(scale):
    x = np.arange(65536, dtype=np.uint16).view(np.float16)
    got = int8.quantize(x, np.float32(scale))
    t = torch.from_numpy(x.astype(np.float32)) / torch.tensor(scale, dtype=torch.float32)
    t = torch.nan_to_num(t, nan=0.0)                    # NaN -> code 0 (inf stays)
    ref = torch.clamp(torch.round(t), -127, 127).to(torch.int8).numpy()
    assert got.dtype == np.int8
    assert np.array_equal(got, ref)


def test_ties_saturation_and_specials():
    y = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 125.5, 127.4, 127.5,
                  200.0, -200.0, np.inf, -np.inf, np.nan, -0.0, 0.49999997],
                 np.float32)
    exp = [0, 2, 2, 0, -2, -2, 126, 126, 127, 127, 127, -127, 127, -127, 0, 0, 0]
    assert int8.encode(y).tolist() == exp


def test_decode_every_code_and_round_trip():
    c = np.arange(-128, 128).astype(np.int8)
    assert np.array_equal(int8.decode(c), np.arange(-128, 128, dtype=np.float64))
    live = np.arange(-127, 128).astype(np.int8)
    assert np.array_equal(int8.encode(live.astype(np.float32)), live)
    assert not np.any(int8.encode(np.linspace(-1e4, 1e4, 20001, dtype=np.float32)) == -128)


def test_encode_is_the_nearest_code_by_brute_force():
    rng = np.random.default_rng(5)
    y = np.concatenate([rng.uniform(-130, 130, 4000), np.arange(-130, 130.5, 0.5)]
                       ).astype(np.float32)
    codes = np.arange(-127, 128)
    got = int8.encode(y).astype(np.int64)
    for yi, gi in zip(y.astype(np.float64), got):
        d = np.abs(codes - yi)
        best = codes[d == d.min()]
        if len(best) == 2:                       # a tie: the even code wins
            best = best[best % 2 == 0]
        assert gi == best[0], (yi, gi, best)


def test_int8_scales_bound_every_value():
    w = make_case(2, 4, 2, 32, 16, (40, 12), kv_dtype="int8", seed=27)
    ks, vs = w.kv_scales()
    K, V, _, _ = w.tokens()
    for X, s in ((K, ks), (V, vs)):
        y = X.astype(np.float32) / s[None, :, None]
        # amax / (amax / 127) may land one float32 ulp above 127: rounds to 127
        assert 126.5 <= np.abs(y).max() < 127.5
        codes = int8.quantize(X, s[None, :, None])
        assert codes.min() >= -127 and codes.max() <= 127
        assert np.abs(codes).max() == 127


def test_append_writes_int8_codes_at_the_header_offsets():
    w = make_case(3, 4, 2, 32, 16, (20, 1, 47), kv_dtype="int8", seed=28, extra_pages=2)
    bk, bv, ks, vs = oracle_pools(w, upto_last=True)
    kn, vn, pos = w.new_tokens()
    k2, v2 = oracle.kv_append(bk, bv, w.block_table, np.arange(3), pos, kn, vn,
                              "int8", ks, vs)
    P, H, bs, d = bk.shape
    kf, vf = k2.reshape(P, H, -1), v2.reshape(P, H, -1)
    touched_k = np.zeros(kf.shape, bool); touched_v = np.zeros(vf.shape, bool)
    for b in range(3):
        p, s = w.block_table[b, pos[b] // 16], pos[b] % 16
        ko = [_tile_pos_k(s, i, d, X=16) for i in range(d)]
        vo = [_tile_pos_v(s, i, d) for i in range(d)]
        touched_k[p, :, ko] = True; touched_v[p, :, vo] = True
        for h in range(2):
            rk = torch.clamp(torch.round(torch.from_numpy(kn[b, h].astype(np.float32))
                                         / float(ks[h])), -127, 127).to(torch.int8).numpy()
            rv = torch.clamp(torch.round(torch.from_numpy(vn[b, h].astype(np.float32))
                                         / float(vs[h])), -127, 127).to(torch.int8).numpy()
            assert np.array_equal(kf[p, h, ko], rk)
            assert np.array_equal(vf[p, h, vo], rv)
    assert np.array_equal(kf[~touched_k], bk.reshape(P, H, -1)[~touched_k])
    assert np.array_equal(vf[~touched_v], bv.reshape(P, H, -1)[~touched_v])
    # every slot the append did not touch and no token owns is still the marker
    full_k, _, _, _ = oracle_pools(w)
    assert np.array_equal(full_k, k2)


def test_int8_path_matches_sdpa_on_dequantised_values():
    w = make_case(2, 8, 2, 32, 16, (33, 7), kv_dtype="int8", seed=29)
    k, v, ks, vs = oracle_pools(w)
    out = oracle.decode(w.q, k, v, w.block_table, w.context_lens, w.scale, "int8", ks, vs)
    kf = k.reshape(k.shape[0], 2, -1); vf = v.reshape(v.shape[0], 2, -1)
    for b in range(2):
        L = int(w.context_lens[b])
        bt = w.block_table[b]
        Kd = np.zeros((2, L, 32)); Vd = np.zeros((2, L, 32))
        for t in range(L):
            p, s = bt[t // 16], t % 16
            for h in range(2):
                kc = [int(kf[p, h, _tile_pos_k(s, i, 32, X=16)]) for i in range(32)]
                vc = [int(vf[p, h, _tile_pos_v(s, i, 32)]) for i in range(32)]
                Kd[h, t] = np.array(kc, np.float64) * float(ks[h])
                Vd[h, t] = np.array(vc, np.float64) * float(vs[h])
        ref = contiguous_reference_sdpa(w.q[b].astype(np.float64), Kd, Vd, w.scale)
        assert np.max(np.abs(out[b] - ref)) < 1e-13


def test_int8_context_of_one_returns_the_dequantised_v():
    w = make_case(1, 4, 1, 64, 16, (1,), kv_dtype="int8", seed=30)
    k, v, ks, vs = oracle_pools(w)
    out = oracle.decode(w.q, k, v, w.block_table, w.context_lens, w.scale, "int8", ks, vs)
    _, V = w.token_kv(0)
    codes = int8.quantize(V[0, 0], vs[0])
    for j in range(4):
        assert np.array_equal(out[0, j], codes.astype(np.float64) * float(vs[0]))
