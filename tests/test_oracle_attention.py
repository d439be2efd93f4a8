"""Pins for the oracle's decode attention (CPU only).

Each test checks the oracle against something other than itself: closed
forms, torch SDPA in float64 (library routine), mpmath brute force, or an
invariant stated on the pages (MQA = MHA with shared K/V; paged = contiguous).
"""
import math

import numpy as np
import pytest

import oracle
from tests.oracle_cases import contiguous_reference_sdpa, oracle_decode, oracle_pools
from workloads import make, make_case


# storage row of each slot of a 16-token K block, written out by hand: the
# second and third quads of slots trade places
_K_ROW = [0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15]


def _tile_pos_k(t, i, d, X=8):
    """Header layout, K: 16-token blocks, 16-byte chunks of X elements."""
    blk, r = divmod(t, 16)
    c, x = divmod(i, X)
    return ((blk * (d // X) + c) * 16 + _K_ROW[r]) * X + x


def _tile_pos_v(t, i, d):
    """Header layout, V: 16-token blocks, 16-dim groups, token octets."""
    blk, r = divmod(t, 16)
    jd, n = divmod(i, 16)
    o, e = divmod(r, 8)
    return (((blk * (d // 16) + jd) * 2 + o) * 16 + n) * 8 + e


def _scatter_by_hand(K, V, perm_pages, bs, num_pages):
    """Test-side page fill: K/V [Hkv, L, d] into pools, one value at a time.

    Token t goes to page perm_pages[t // bs], slot t % bs, at the position
    the library header documents for a (page, head) tile of bs * d values.
    """
    Hkv, L, d = K.shape
    kp = np.full((num_pages, Hkv, bs * d), np.nan)
    vp = np.full((num_pages, Hkv, bs * d), np.nan)
    for t in range(L):
        p, s = perm_pages[t // bs], t % bs
        for h in range(Hkv):
            for i in range(d):
                kp[p, h, _tile_pos_k(s, i, d)] = K[h, t, i]
                vp[p, h, _tile_pos_v(s, i, d)] = V[h, t, i]
    return kp.reshape(num_pages, Hkv, bs, d), vp.reshape(num_pages, Hkv, bs, d)


def _one_seq(q, K, V, scale, bs, rng, extra=3):
    """Run the oracle on one sequence scattered through a random page map."""
    Hkv, L, d = K.shape
    nblk = -(-L // bs)
    P = nblk + extra
    perm = rng.permutation(P)
    kp, vp = _scatter_by_hand(K, V, perm, bs, P)
    bt = np.full((1, nblk + 2), perm[-1], np.int32)   # unused -> a NaN page
    bt[0, :nblk] = perm[:nblk]
    return oracle.decode(q[None], kp, vp, bt, np.array([L]), scale)[0]


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


@pytest.mark.parametrize("Hq,Hkv,d,bs,L", [
    (4, 1, 64, 16, 17), (8, 2, 32, 16, 40), (6, 3, 16, 32, 70), (4, 4, 16, 64, 130),
])
def test_matches_torch_sdpa(Hq, Hkv, d, bs, L):
    rng = np.random.default_rng(L)
    q = _rand(rng, Hq, d); K = _rand(rng, Hkv, L, d); V = _rand(rng, Hkv, L, d)
    scale = 1 / math.sqrt(d) * 1.3
    got = _one_seq(q, K, V, scale, bs, rng)
    ref = contiguous_reference_sdpa(q, K, V, scale)
    assert np.max(np.abs(got - ref)) < 1e-13


def test_context_of_one_returns_v():
    rng = np.random.default_rng(1)
    q = _rand(rng, 4, 16); K = _rand(rng, 2, 1, 16); V = _rand(rng, 2, 1, 16)
    got = _one_seq(q, K, V, 0.3, 16, rng)
    assert np.array_equal(got, np.repeat(V[:, 0, :], 2, axis=0))


def test_constant_v_returns_constant():
    rng = np.random.default_rng(2)
    q = _rand(rng, 4, 16); K = _rand(rng, 1, 50, 16)
    c = _rand(rng, 16)
    V = np.broadcast_to(c, (1, 50, 16)).copy()
    got = _one_seq(q, K, V, 0.25, 16, rng)
    assert np.max(np.abs(got - c[None, :])) < 1e-14


def test_uniform_scores_give_mean_of_v():
    rng = np.random.default_rng(3)
    q = np.zeros((2, 16)); K = _rand(rng, 1, 37, 16); V = _rand(rng, 1, 37, 16)
    got = _one_seq(q, K, V, 0.25, 16, rng)
    assert np.max(np.abs(got - np.mean(V[0], axis=0)[None])) < 1e-14


def test_two_tokens_logistic_closed_form():
    rng = np.random.default_rng(4)
    q = _rand(rng, 1, 16); K = _rand(rng, 1, 2, 16); V = _rand(rng, 1, 2, 16)
    scale = 0.7
    s0 = scale * float(q[0] @ K[0, 0]); s1 = scale * float(q[0] @ K[0, 1])
    sig = 1.0 / (1.0 + math.exp(-(s0 - s1)))
    expect = sig * V[0, 0] + (1 - sig) * V[0, 1]
    got = _one_seq(q, K, V, scale, 16, rng)
    assert np.max(np.abs(got[0] - expect)) < 1e-15


def test_scale_invariance():
    rng = np.random.default_rng(6)
    q = _rand(rng, 4, 32); K = _rand(rng, 2, 90, 32); V = _rand(rng, 2, 90, 32)
    a = _one_seq(q, K, V, 0.2, 16, np.random.default_rng(9))
    b = _one_seq(q * 4.0, K, V, 0.05, 16, np.random.default_rng(9))
    assert np.max(np.abs(a - b)) < 1e-14


def test_mqa_equals_mha_with_replicated_kv():
    """MQA formula (shared K, V) = MHA formula with K_i = K, V_i = V for all i."""
    rng = np.random.default_rng(7)
    G, d, L = 4, 16, 45
    q = _rand(rng, 2 * G, d); K = _rand(rng, 2, L, d); V = _rand(rng, 2, L, d)
    gqa = _one_seq(q, K, V, 0.25, 16, np.random.default_rng(1))
    Krep = np.repeat(K, G, axis=0); Vrep = np.repeat(V, G, axis=0)
    mha = _one_seq(q, Krep, Vrep, 0.25, 16, np.random.default_rng(1))
    assert np.max(np.abs(gqa - mha)) < 1e-14   # BLAS order may differ
    # and a group's heads really use their own kv head (not j % Hkv)
    swapped = _one_seq(q, K[::-1].copy(), V[::-1].copy(), 0.25, 16,
                       np.random.default_rng(1))
    assert not np.allclose(gqa, swapped)


def test_paged_equals_contiguous_for_any_page_permutation():
    rng = np.random.default_rng(8)
    q = _rand(rng, 4, 16); K = _rand(rng, 2, 75, 16); V = _rand(rng, 2, 75, 16)
    outs = [_one_seq(q, K, V, 0.25, 16, np.random.default_rng(s)) for s in range(6)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    # contiguous: one page of 80 slots holding all 75 tokens in order
    kp, vp = _scatter_by_hand(K, V, [0], 80, 1)
    one = oracle.decode(q[None], kp, vp, np.zeros((1, 1), np.int32),
                        np.array([75]), 0.25)[0]
    assert np.max(np.abs(one - outs[0])) < 1e-14


def test_empty_context_gives_zeros():
    w = make_case(2, 4, 1, 16, 16, (0, 5), seed=3)
    out = oracle_decode(w)
    assert np.all(out[0] == 0) and np.all(np.isfinite(out))


def test_poisoned_slots_never_read():
    w = make("tiny_mqa")
    out = oracle_decode(w)
    assert np.all(np.isfinite(out))
    k, v, _, _ = oracle_pools(w)
    # 11 of the 16 pages are untouched and NaN; tail slots of last pages too
    assert np.isnan(k[w.poison_pages]).all() and np.isnan(v[w.poison_pages]).all()


def test_tiny_config_against_mpmath_brute_force():
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    w = make("tiny_mqa")
    out = oracle_decode(w)
    for b in range(2):
        K, V = w.token_kv(b)
        L = K.shape[0]
        for j in range(4):
            h = j // 4
            qj = [mpmath.mpf(float(x)) for x in w.q[b, j]]
            s = [mpmath.mpf(w.scale) * mpmath.fsum(qj[i] * mpmath.mpf(float(K[t, h, i]))
                                                   for i in range(64))
                 for t in range(L)]
            e = [mpmath.exp(x) for x in s]
            Z = mpmath.fsum(e)
            for i in range(64):
                ref = mpmath.fsum(e[t] * mpmath.mpf(float(V[t, h, i])) for t in range(L)) / Z
                assert abs(float(ref) - out[b, j, i]) < 1e-12


def test_fp8_path_matches_sdpa_on_dequantised_values():
    import torch
    w = make_case(2, 8, 2, 32, 16, (33, 7), kv_dtype="fp8_e4m3fn", seed=11)
    k, v, ks, vs = oracle_pools(w)
    out = oracle.decode(w.q, k, v, w.block_table, w.context_lens, w.scale,
                        "fp8_e4m3fn", ks, vs)
    for b in range(2):
        L = int(w.context_lens[b])
        bt = w.block_table[b]
        # dequantise with torch's float8 type, gathering by hand
        Kd = np.zeros((2, L, 32)); Vd = np.zeros((2, L, 32))
        kf = k.reshape(k.shape[0], 2, -1); vf = v.reshape(v.shape[0], 2, -1)
        for t in range(L):
            p, s = bt[t // 16], t % 16
            for h in range(2):
                kc = np.array([kf[p, h, _tile_pos_k(s, i, 32, X=16)] for i in range(32)], np.uint8)
                vc = np.array([vf[p, h, _tile_pos_v(s, i, 32)] for i in range(32)], np.uint8)
                Kd[h, t] = torch.from_numpy(kc).view(torch.float8_e4m3fn).to(torch.float64).numpy() * float(ks[h])
                Vd[h, t] = torch.from_numpy(vc).view(torch.float8_e4m3fn).to(torch.float64).numpy() * float(vs[h])
        ref = contiguous_reference_sdpa(w.q[b].astype(np.float64), Kd, Vd, w.scale)
        assert np.max(np.abs(out[b] - ref)) < 1e-13
