"""Pins for the oracle's split partials, their merge, and kv_append (CPU only)."""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import fp8
from tests.oracle_cases import oracle_pools
from tests.test_oracle_attention import _tile_pos_k, _tile_pos_v
from workloads import make_case


@pytest.mark.parametrize("L,bs", [(1, 16), (15, 16), (16, 16), (17, 16), (100, 16),
                                  (333, 32), (700, 64), (64, 64)])
def test_split_bounds_cover_context_once_and_are_page_aligned(L, bs):
    for S in range(1, 65):
        b = oracle.split_bounds(L, S, bs)
        assert len(b) == S
        covered = []
        for a, e in b:
            assert 0 <= a <= e <= L
            assert a % bs == 0 or a == L
            covered.extend(range(a, e))
        assert covered == list(range(L))


def test_merge_of_splits_equals_unsplit():
    w = make_case(3, 8, 2, 32, 16, (1, 77, 300), seed=21)
    k, v, ks, vs = oracle_pools(w)
    full = oracle.decode(w.q, k, v, w.block_table, w.context_lens, w.scale)
    for S in list(range(1, 20)) + [32, 63, 64]:
        o, lse = oracle.decode_partials(w.q, k, v, w.block_table, w.context_lens,
                                        w.scale, S)
        merged = oracle.merge_partials(o, lse)
        assert np.max(np.abs(merged - full)) < 1e-12, S
        # sequence of length 1 has one live split only
        assert np.sum(np.isfinite(lse[0, 0])) == 1


def test_one_split_is_identity_and_lse_is_logsumexp():
    w = make_case(2, 4, 2, 16, 16, (50, 9), seed=22)
    k, v, _, _ = oracle_pools(w)
    full = oracle.decode(w.q, k, v, w.block_table, w.context_lens, w.scale)
    o, lse = oracle.decode_partials(w.q, k, v, w.block_table, w.context_lens,
                                    w.scale, 1)
    assert np.max(np.abs(o[:, :, 0] - full)) < 1e-15
    # lse against scipy's logsumexp over scores gathered by hand
    for b in range(2):
        K, _ = w.token_kv(b)
        for j in range(4):
            s = w.scale * (K[:, j // 2, :].astype(np.float64) @ w.q[b, j].astype(np.float64))
            assert abs(lse[b, j, 0] - scipy.special.logsumexp(s)) < 1e-12


def test_split_partials_match_scipy_per_chunk():
    w = make_case(1, 2, 1, 16, 16, (90,), seed=23)
    k, v, _, _ = oracle_pools(w)
    S = 4
    o, lse = oracle.decode_partials(w.q, k, v, w.block_table, w.context_lens,
                                    w.scale, S)
    K, V = w.token_kv(0)
    for i, (a, e) in enumerate(oracle.split_bounds(90, S, 16)):
        for j in range(2):
            if e <= a:
                assert lse[0, j, i] == -np.inf and np.all(o[0, j, i] == 0)
                continue
            s = w.scale * (K[a:e, 0].astype(np.float64) @ w.q[0, j].astype(np.float64))
            p = scipy.special.softmax(s)
            assert np.max(np.abs(o[0, j, i] - p @ V[a:e, 0].astype(np.float64))) < 1e-14
            assert abs(lse[0, j, i] - scipy.special.logsumexp(s)) < 1e-12


def test_merge_handles_empty_and_all_empty():
    o = np.zeros((2, 3, 4)); lse = np.full((2, 3), -np.inf)
    o[0, 1] = [1, 2, 3, 4]; lse[0, 1] = 0.5
    m = oracle.merge_partials(o, lse)
    assert np.array_equal(m[0], [1, 2, 3, 4]) and np.array_equal(m[1], [0, 0, 0, 0])


def test_context_zero_all_splits_empty():
    w = make_case(2, 4, 1, 16, 16, (0, 3), seed=24)
    k, v, _, _ = oracle_pools(w)
    o, lse = oracle.decode_partials(w.q, k, v, w.block_table, w.context_lens,
                                    w.scale, 5)
    assert np.all(lse[0] == -np.inf) and np.all(o[0] == 0)
    assert np.all(oracle.merge_partials(o, lse)[0] == 0)


# -- kv_append ---------------------------------------------------------------

def _append_case(kv_dtype):
    w = make_case(3, 4, 2, 32, 16, (20, 1, 47), kv_dtype=kv_dtype, seed=25,
                  extra_pages=2)
    base_k, base_v, ks, vs = oracle_pools(w, upto_last=True)
    kn, vn, pos = w.new_tokens()
    k2, v2 = oracle.kv_append(base_k, base_v, w.block_table, np.arange(3), pos,
                              kn, vn, kv_dtype, ks, vs)
    return w, base_k, base_v, k2, v2, kn, vn, pos, ks, vs


def _bytes(a):
    return np.ascontiguousarray(a).view(np.uint8)


@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8_e4m3fn"])
def test_append_writes_target_slots_only(kv_dtype):
    w, bk, bv, k2, v2, kn, vn, pos, ks, vs = _append_case(kv_dtype)
    P, H, bs, d = bk.shape
    X = 8 if kv_dtype == "fp16" else 16
    bkf, bvf = bk.reshape(P, H, -1), bv.reshape(P, H, -1)
    k2f, v2f = k2.reshape(P, H, -1), v2.reshape(P, H, -1)
    tk = np.zeros(bkf.shape, bool); tv = np.zeros(bvf.shape, bool)
    for b in range(3):
        p = w.block_table[b, pos[b] // 16]; s = pos[b] % 16
        ko = [_tile_pos_k(s, i, d, X) for i in range(d)]
        vo = [_tile_pos_v(s, i, d) for i in range(d)]
        tk[p, :, ko] = True; tv[p, :, vo] = True
        for h in range(2):
            if kv_dtype == "fp16":
                assert np.array_equal(_bytes(k2f[p, h, ko]), _bytes(kn[b, h]))
                assert np.array_equal(_bytes(v2f[p, h, vo]), _bytes(vn[b, h]))
            else:   # torch's cast as the library reference; it does not
                    # saturate, so magnitudes >= 448 expect the +-448 code
                yk = kn[b, h].astype(np.float32) / np.float32(ks[h])
                yv = vn[b, h].astype(np.float32) / np.float32(vs[h])
                rk, rv = (np.where(np.abs(y) >= 448, np.where(y < 0, 0xFE, 0x7E),
                                   torch.from_numpy(np.clip(y, -447, 447)).to(
                                       torch.float8_e4m3fn).view(torch.uint8).numpy()
                                   ).astype(np.uint8) for y in (yk, yv))
                assert np.array_equal(k2f[p, h, ko], rk)
                assert np.array_equal(v2f[p, h, vo], rv)
    # everything else unchanged, byte for byte
    assert np.array_equal(_bytes(k2f[~tk]), _bytes(bkf[~tk]))
    assert np.array_equal(_bytes(v2f[~tv]), _bytes(bvf[~tv]))


def test_layout_offsets_are_a_bijection_of_the_tile():
    for bs in (16, 32, 64):
        for d in (64, 128):
            for X in (8, 16):
                ko = sorted(_tile_pos_k(t, i, d, X) for t in range(bs) for i in range(d))
                assert ko == list(range(bs * d))
            vo = sorted(_tile_pos_v(t, i, d) for t in range(bs) for i in range(d))
            assert vo == list(range(bs * d))
    # and the oracle's offsets agree with the hand-written ones
    t = np.arange(64)[:, None]; i = np.arange(128)[None, :]
    from oracle.paged import k_offset, v_offset
    assert np.array_equal(k_offset(t, i, 128, 8),
                          [[_tile_pos_k(a, b, 128, 8) for b in range(128)] for a in range(64)])
    assert np.array_equal(v_offset(t, i, 128),
                          [[_tile_pos_v(a, b, 128) for b in range(128)] for a in range(64)])


@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8_e4m3fn", "int8"])
def test_append_then_attend_equals_full_pool(kv_dtype):
    w, bk, bv, k2, v2, kn, vn, pos, ks, vs = _append_case(kv_dtype)
    fk, fv, _, _ = oracle_pools(w)
    assert np.array_equal(_bytes(fk), _bytes(k2)) and np.array_equal(_bytes(fv), _bytes(v2))


def test_fp8_scales_bound_every_value():
    w = make_case(2, 4, 2, 32, 16, (40, 12), kv_dtype="fp8_e4m3fn", seed=26)
    ks, vs = w.kv_scales()
    K, V, _, _ = w.tokens()
    yk = K.astype(np.float32) / ks[None, :, None]
    # amax / (amax/448) may land one float32 ulp above 448; anything below
    # 464 rounds to 448 by RNE, so saturation and rounding agree there
    assert 447.0 <= np.abs(yk).max() < 464.0
    codes = fp8.quantize(K, ks[None, :, None])
    assert not np.any(codes == 0x7F) and not np.any(codes == 0xFF)


def test_lse_of_matches_scipy_logsumexp_per_head():
    """oracle.attention.lse_of: ln sum_t exp(scale q.k_t) over the whole
    context of each (sequence, q head), on a group map where j // G and
    j % Hkv disagree (G = 3, Hkv = 2), a scale far from 1, an fp8 cache and
    an empty sequence (-inf). Scores are gathered by hand from the token
    stream, not from the pools."""
    for kv_dtype in ("fp16", "fp8_e4m3fn", "int8"):
        w = make_case(3, 6, 2, 32, 16, (70, 0, 5), kv_dtype=kv_dtype, seed=31,
                      scale=0.37)
        k, v, ks, vs = oracle_pools(w)
        got = oracle.attention.lse_of(w.q, k, v, w.block_table, w.context_lens,
                                      w.scale, kv_dtype, ks, vs)
        assert got.shape == (3, 6)
        assert np.all(got[1] == -np.inf)
        for b in (0, 2):
            K, _ = w.token_kv(b)
            for j in range(6):
                h = j // 3
                Kh = K[:, h, :].astype(np.float32)
                if kv_dtype == "fp8_e4m3fn":
                    Kh = fp8.decode(fp8.quantize(Kh, ks[h])) * np.float64(ks[h])
                elif kv_dtype == "int8":
                    from oracle import int8 as oi8
                    Kh = oi8.quantize(Kh, ks[h]).astype(np.float64) * np.float64(ks[h])
                s = 0.37 * (Kh.astype(np.float64) @ w.q[b, j].astype(np.float64))
                assert abs(got[b, j] - scipy.special.logsumexp(s)) < 1e-12, (kv_dtype, b, j)


def test_range_partial_matches_scipy_and_whole_context():
    """oracle.attention.range_partial over [a, e): scipy softmax-weighted V
    and logsumexp of hand-gathered scores; over [0, L) it is decode and
    lse_of; adjacent ranges merge to their union."""
    w = make_case(2, 6, 2, 32, 16, (150, 40), seed=32, scale=0.3)
    k, v, ks, vs = oracle_pools(w)
    full = oracle.decode(w.q, k, v, w.block_table, w.context_lens, w.scale)
    tot = oracle.attention.lse_of(w.q, k, v, w.block_table, w.context_lens, w.scale)
    K, V = w.token_kv(0)
    for h in range(2):
        for a, e in ((0, 32), (32, 150), (17, 18), (64, 64), (0, 150)):
            o, lse = oracle.attention.range_partial(w.q, k, v, w.block_table, 0, h, a, e,
                                                    w.scale)
            for g in range(3):
                j = h * 3 + g
                if e <= a:
                    assert lse[g] == -np.inf and np.all(o[g] == 0)
                    continue
                s = 0.3 * (K[a:e, h].astype(np.float64) @ w.q[0, j].astype(np.float64))
                p = scipy.special.softmax(s)
                assert np.max(np.abs(o[g] - p @ V[a:e, h].astype(np.float64))) < 1e-14
                assert abs(lse[g] - scipy.special.logsumexp(s)) < 1e-12
                if (a, e) == (0, 150):
                    assert np.max(np.abs(o[g] - full[0, j])) < 1e-14
                    assert abs(lse[g] - tot[0, j]) < 1e-12
        o1, l1 = oracle.attention.range_partial(w.q, k, v, w.block_table, 0, h, 0, 64, w.scale)
        o2, l2 = oracle.attention.range_partial(w.q, k, v, w.block_table, 0, h, 64, 150, w.scale)
        m = oracle.merge_partials(np.stack([o1, o2], 1), np.stack([l1, l2], 1))
        assert np.max(np.abs(m - full[0, h * 3:(h + 1) * 3])) < 1e-14


def test_inplace_append_equals_copying_append():
    w, bk, bv, k2, v2, kn, vn, pos, ks, vs = _append_case("fp8_e4m3fn")
    ik, iv = bk.copy(), bv.copy()
    rk, rv = oracle.kv_append(ik, iv, w.block_table, np.arange(3), pos, kn, vn,
                              "fp8_e4m3fn", ks, vs, inplace=True)
    assert np.shares_memory(rk, ik) and np.shares_memory(rv, iv)
    assert np.array_equal(ik, k2) and np.array_equal(iv, v2)
