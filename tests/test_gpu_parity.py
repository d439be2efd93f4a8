"""GPU parity: the HIP library against the fp64 CPU oracle (needs an MI355X).

Both sides get the same seeded inputs from `workloads`; the oracle builds
its pools with its own append, the GPU with the library's kv_append, and no
expected value comes from the GPU. Tolerances are those fixed for the path:
max-abs 2e-3 for fp16 KV and 3e-2 for fp8 KV (fp32 accumulation); int8 KV,
the other one-byte cache, runs the same arithmetic on exactly representable
codes and is held to the one-byte bound, 3e-2. Cache append and
block-table indexing are bit-exact.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
from oracle import int8 as oi8
from oracle.paged import k_offset, v_offset
from tests.oracle_cases import oracle_pools
from workloads import CONFIGS, make, make_case
from workloads.device import DeviceWorkload, remap_pages

pytestmark = pytest.mark.gpu

TOL = {"fp16": 2e-3, "fp8_e4m3fn": 3e-2, "int8": 3e-2}
KV_ALL = ["fp16", "fp8_e4m3fn", "int8"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mqa_gqa_amd as pa
    pa.load()          # must load on a GPU machine: no fallback exists
    yield


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def pa_mod():
    import paged_mqa_gqa_amd as pa
    return pa


def gpu_decode(dw, num_splits=1, merged=False):
    pa = pa_mod()
    if merged:
        ws = pa.splitk_workspace(dw.q, dw.k_pages, dw.block_table, num_splits)
        out = pa.paged_decode_attn_splitk_merged(dw.q, dw.k_pages, dw.v_pages,
                                                 dw.block_table, dw.context_lens,
                                                 dw.scale, num_splits, ws,
                                                 dw.k_scale, dw.v_scale)
    elif num_splits == 1:
        out = pa.paged_decode_attn(dw.q, dw.k_pages, dw.v_pages, dw.block_table,
                                   dw.context_lens, dw.scale, dw.k_scale, dw.v_scale)
    else:
        ws = pa.paged_decode_attn_splitk(dw.q, dw.k_pages, dw.v_pages, dw.block_table,
                                         dw.context_lens, dw.scale, num_splits,
                                         dw.k_scale, dw.v_scale)
        out = pa.paged_decode_attn_splitk_reduce(dw.q, dw.k_pages, dw.block_table,
                                                 dw.context_lens, num_splits, ws)
    torch.cuda.synchronize()
    return out


def oracle_out(w, seqs=None):
    if seqs is None:
        k, v, ks, vs = oracle_pools(w)
        return oracle.decode(w.q, k, v, w.block_table, w.context_lens, w.scale,
                             w.cfg.kv_dtype, ks, vs)
    sub = remap_pages(w, seqs)
    k, v, ks, vs = oracle_pools(sub, seqs=seqs)
    return oracle.decode(sub.q, k, v, sub.block_table, sub.context_lens, sub.scale,
                         sub.cfg.kv_dtype, ks, vs, seqs=seqs)


def max_err(gpu_out, ref, seqs=None):
    g = gpu_out.float().cpu().numpy().astype(np.float64)
    if seqs is not None:
        g, ref = g[list(seqs)], ref[list(seqs)]
    assert np.all(np.isfinite(g)), "non-finite output"
    return float(np.max(np.abs(g - ref))) if g.size else 0.0


# -- cache append ----------------------------------------------------------

APPEND_CASES = [
    dict(num_seqs=3, num_q_heads=4, num_kv_heads=2, head_dim=128, block_size=16, lens=(20, 1, 47)),
    dict(num_seqs=2, num_q_heads=8, num_kv_heads=4, head_dim=64, block_size=32, lens=(33, 90)),
    dict(num_seqs=4, num_q_heads=8, num_kv_heads=8, head_dim=128, block_size=64, lens=(64, 65, 1, 200)),
]


@pytest.mark.parametrize("kv_dtype", KV_ALL)
@pytest.mark.parametrize("case", range(len(APPEND_CASES)))
def test_kv_append_bit_exact(case, kv_dtype):
    c = APPEND_CASES[case]
    say("kv_append", kv_dtype, c)
    w = make_case(**c, kv_dtype=kv_dtype, seed=31 + case, extra_pages=3)
    dw = DeviceWorkload(w, upto_last=True)       # library fills all but the last token
    pa = pa_mod()
    pa.kv_append(dw.new_k, dw.new_v, dw.k_pages, dw.v_pages, dw.block_table,
                 dw.positions, k_scale=dw.k_scale, v_scale=dw.v_scale)
    torch.cuda.synchronize()
    ok, ov, _, _ = oracle_pools(w)
    gk = dw.k_pages.cpu().numpy().view(np.uint8)
    gv = dw.v_pages.cpu().numpy().view(np.uint8)
    assert np.array_equal(gk, np.ascontiguousarray(ok).view(np.uint8))
    assert np.array_equal(gv, np.ascontiguousarray(ov).view(np.uint8))


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -8, 0.010296, 3.7])
def test_kv_append_fp8_encodes_every_fp16_pattern(scale):
    """All 65536 fp16 bit patterns (incl. inf/NaN) through the device encoder."""
    say("fp8 encode exhaustive", scale)
    pa = pa_mod()
    vals = np.arange(65536, dtype=np.uint16).view(np.float16)
    T, H, D, bs = 512, 1, 128, 16
    x = vals.reshape(T, H, D)
    bt = np.arange(T // bs, dtype=np.int32)[None, :]
    P = T // bs
    kp = torch.zeros((P, H, bs, D), dtype=torch.uint8, device="cuda")
    vp = torch.zeros((P, H, bs, D), dtype=torch.uint8, device="cuda")
    s = torch.tensor([scale], dtype=torch.float32, device="cuda")
    xt = torch.from_numpy(x.copy()).cuda()
    pa.kv_append(xt, xt, kp, vp, torch.from_numpy(bt).cuda(),
                 torch.arange(T, dtype=torch.int32, device="cuda"),
                 seq_ids=torch.zeros(T, dtype=torch.int32, device="cuda"),
                 k_scale=s, v_scale=s)
    torch.cuda.synchronize()
    ref = ofp8.quantize(x, np.float32(scale))[:, 0, :]     # [T, D]
    t = np.arange(T)[:, None]; i = np.arange(D)[None, :]
    kf = kp.cpu().numpy().reshape(P, bs * D); vf = vp.cpu().numpy().reshape(P, bs * D)
    got_k = kf[t // bs, k_offset(t % bs, i, D, 16)]
    got_v = vf[t // bs, v_offset(t % bs, i, D)]
    assert np.array_equal(got_k, ref)
    assert np.array_equal(got_v, ref)


def test_fp8_decode_of_every_code_via_single_token_attention():
    """L = 1 returns V exactly: out = fp16(decode(code) * v_scale) for every code."""
    say("fp8 decode exhaustive")
    pa = pa_mod()
    H, D, bs = 2, 128, 16
    codes = np.arange(256, dtype=np.uint8).reshape(H, D)
    vp = np.zeros((1, H, bs * D), np.uint8)
    vp[0, :, v_offset(0, np.arange(D), D)] = codes.T        # token 0 of page 0
    vp = vp.reshape(1, H, bs, D)
    kp = np.zeros((1, H, bs, D), np.uint8)
    vscale = np.array([0.75, 0.0103], np.float32)
    out = pa.paged_decode_attn(
        torch.zeros((1, H, D), dtype=torch.float16, device="cuda"),
        torch.from_numpy(kp).cuda(), torch.from_numpy(vp).cuda(),
        torch.zeros((1, 1), dtype=torch.int32, device="cuda"),
        torch.ones(1, dtype=torch.int32, device="cuda"), 0.1,
        torch.ones(H, dtype=torch.float32, device="cuda"),
        torch.from_numpy(vscale).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy()[0].astype(np.float64)
    exp = (ofp8.decode(codes) * vscale[:, None].astype(np.float64)).astype(np.float16).astype(np.float64)
    fin = np.isfinite(exp)                      # 0x7F / 0xFF are NaN codes, never stored
    assert fin.sum() == 254
    # the device scales in fp32 and then rounds to fp16: at most 1 fp16 ulp apart
    ulp = np.spacing(np.abs(exp[fin]).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(got[fin] - exp[fin]) <= ulp)


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -8, 0.010296, 3.7, 1.0 / 127])
def test_kv_append_int8_encodes_every_fp16_pattern(scale):
    """All 65536 fp16 bit patterns (inf and NaN included) through the device's
    int8 encoder, against the oracle's codec."""
    say("int8 encode exhaustive", scale)
    pa = pa_mod()
    vals = np.arange(65536, dtype=np.uint16).view(np.float16)
    T, H, D, bs = 512, 1, 128, 16
    x = vals.reshape(T, H, D)
    P = T // bs
    bt = torch.arange(P, dtype=torch.int32, device="cuda")[None, :]
    kp = torch.zeros((P, H, bs, D), dtype=torch.int8, device="cuda")
    vp = torch.zeros((P, H, bs, D), dtype=torch.int8, device="cuda")
    s = torch.tensor([scale], dtype=torch.float32, device="cuda")
    xt = torch.from_numpy(x.copy()).cuda()
    pa.kv_append(xt, xt, kp, vp, bt, torch.arange(T, dtype=torch.int32, device="cuda"),
                 seq_ids=torch.zeros(T, dtype=torch.int32, device="cuda"),
                 k_scale=s, v_scale=s)
    torch.cuda.synchronize()
    ref = oi8.quantize(x, np.float32(scale))[:, 0, :]
    t = np.arange(T)[:, None]; i = np.arange(D)[None, :]
    kf = kp.cpu().numpy().reshape(P, bs * D); vf = vp.cpu().numpy().reshape(P, bs * D)
    assert np.array_equal(kf[t // bs, k_offset(t % bs, i, D, 16)], ref)
    assert np.array_equal(vf[t // bs, v_offset(t % bs, i, D)], ref)


def test_int8_decode_of_every_code_via_single_token_attention():
    """L = 1 returns V: out = fp16(code * v_scale) for all 256 codes (the
    device expands each code to fp16 exactly and scales in fp32)."""
    say("int8 decode exhaustive")
    pa = pa_mod()
    H, D, bs = 2, 128, 16
    codes = (np.arange(256) - 128).astype(np.int8).reshape(H, D)
    vp = np.zeros((1, H, bs * D), np.int8)
    vp[0, :, v_offset(0, np.arange(D), D)] = codes.T
    vp = vp.reshape(1, H, bs, D)
    kp = np.zeros((1, H, bs, D), np.int8)
    vscale = np.array([0.75, 0.0103], np.float32)
    out = pa.paged_decode_attn(
        torch.zeros((1, H, D), dtype=torch.float16, device="cuda"),
        torch.from_numpy(kp).cuda(), torch.from_numpy(vp).cuda(),
        torch.zeros((1, 1), dtype=torch.int32, device="cuda"),
        torch.ones(1, dtype=torch.int32, device="cuda"), 0.1,
        torch.ones(H, dtype=torch.float32, device="cuda"),
        torch.from_numpy(vscale).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy()[0].astype(np.float64)
    exact = codes.astype(np.float64) * vscale[:, None].astype(np.float64)
    exp = exact.astype(np.float16).astype(np.float64)
    ulp = np.spacing(np.abs(exp).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(got - exp) <= ulp)


# -- attention parity ------------------------------------------------------

SWEEP = [
    # (Hq, Hkv, d, bs, lens)
    (4, 1, 64, 16, (17, 40)),
    (4, 4, 128, 16, (1, 2, 15, 16, 17, 31, 32, 33)),
    (8, 2, 128, 32, (100, 300, 64, 65)),
    (32, 8, 128, 16, (700, 1, 513)),
    (16, 1, 128, 64, (1000, 63, 64, 129)),
    (20, 1, 64, 16, (90, 33)),
    (48, 2, 128, 32, (257, 12)),
    (96, 1, 128, 32, (600, 31, 1)),
    (128, 1, 64, 16, (77, 300)),
    (2, 1, 64, 64, (5000,)),
    (8, 8, 64, 16, (0, 5, 0)),
]


@pytest.mark.parametrize("kv_dtype", KV_ALL)
@pytest.mark.parametrize("case", range(len(SWEEP)))
def test_decode_parity_sweep(case, kv_dtype):
    Hq, Hkv, d, bs, lens = SWEEP[case]
    say("decode", kv_dtype, SWEEP[case])
    w = make_case(len(lens), Hq, Hkv, d, bs, lens, kv_dtype=kv_dtype,
                  seed=100 + case, extra_pages=2)
    dw = DeviceWorkload(w)
    ref = oracle_out(w)
    err = max_err(gpu_decode(dw), ref)
    assert err <= TOL[kv_dtype], err


@pytest.mark.parametrize("kv_dtype", KV_ALL)
@pytest.mark.parametrize("case", range(len(SWEEP)))
def test_merged_split_parity_sweep(case, kv_dtype):
    """Split pass with the in-kernel merge, same sweep and bounds."""
    Hq, Hkv, d, bs, lens = SWEEP[case]
    say("merged", kv_dtype, SWEEP[case])
    w = make_case(len(lens), Hq, Hkv, d, bs, lens, kv_dtype=kv_dtype,
                  seed=100 + case, extra_pages=2)
    dw = DeviceWorkload(w)
    ref = oracle_out(w)
    for S in (2, 5, 64):
        err = max_err(gpu_decode(dw, S, merged=True), ref)
        assert err <= TOL[kv_dtype], (S, err)


def test_merged_counters_return_to_zero_across_calls():
    """One workspace serves merged calls whose batch and split count shrink
    and grow in turn (B 4 -> 2 -> 9 -> 4 -> 1, S 16 -> 64 -> 3 -> 16 -> 2):
    every result matches the oracle and the arrival counters are zero after
    each call. Each call writes partials over what the previous call left
    in the workspace."""
    say("merged reuse")
    pa = pa_mod()
    cases = [
        (make_case(4, 32, 8, 128, 16, (3000, 0, 700, 64), seed=303), 16),
        (make_case(2, 32, 8, 128, 16, (2500, 900), seed=304), 64),
        (make_case(9, 16, 4, 128, 16, (1, 40, 777, 1200, 0, 33, 3000, 64, 65), seed=309), 3),
        (make_case(4, 32, 8, 128, 16, (3000, 0, 700, 64), seed=303), 16),
        (make_case(1, 8, 1, 64, 32, (4000,), seed=310), 2),
    ]
    need = 0
    for w, S in cases:
        dw = DeviceWorkload(w)
        need = max(need, pa.splitk_workspace_size(
            pa.dims(w.cfg.num_seqs, w.cfg.num_q_heads, dw.k_pages, dw.block_table), S))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for w, S in cases:
        dw = DeviceWorkload(w)
        out = pa.paged_decode_attn_splitk_merged(dw.q, dw.k_pages, dw.v_pages,
                                                 dw.block_table, dw.context_lens,
                                                 dw.scale, S, ws)
        torch.cuda.synchronize()
        assert max_err(out, oracle_out(w)) <= TOL["fp16"], (w.cfg.num_seqs, S)
        assert int(pa.sem_view(ws).abs().sum()) == 0


def _range_end(lse_gpu, q, k, v, bt, b, h, a, L, scale, kv_dtype, ks, vs):
    """The end e of the token range [a, e) (e a multiple of the 32-token tile,
    or L) whose oracle lse matches the GPU partial's lse_gpu [G] best, and
    the oracle partial (o [G, d], lse [G]) over that range."""
    best = None
    for e in list(range(a + 32, L, 32)) + [L]:
        o, lse = oracle.attention.range_partial(q, k, v, bt, b, h, a, e, scale,
                                                kv_dtype, ks, vs)
        d = float(np.max(np.abs(lse - lse_gpu)))
        if best is None or d < best[0]:
            best = (d, e, o, lse)
    return best


@pytest.mark.parametrize("kv_dtype", KV_ALL)
@pytest.mark.parametrize("S", [1, 2, 3, 7, 16, 64])
def test_split_pass_partials_and_merge(S, kv_dtype):
    """The split pass's partials, one by one: partial i of a (sequence, kv
    head) covers the tokens [a_i, a_{i+1}) that follow partial i-1's, with
    a_0 = 0 and the last ending at L. Each range's end is found as the
    32-token boundary where the oracle's lse over [a_i, e) matches the
    partial's lse (to 1e-4), and its o is then compared with the oracle's
    partial over that range. The merge equals the oracle's full result."""
    say("split pass", kv_dtype, S)
    pa = pa_mod()
    lens = (1, 40, 333, 1000, 0, 4100)
    B, Hq, Hkv, D = len(lens), 8, 2, 128
    w = make_case(B, Hq, Hkv, D, 16, lens, kv_dtype=kv_dtype, seed=200 + S)
    dw = DeviceWorkload(w)
    ws = pa.paged_decode_attn_splitk(dw.q, dw.k_pages, dw.v_pages, dw.block_table,
                                     dw.context_lens, dw.scale, S, dw.k_scale, dw.v_scale)
    out = pa.paged_decode_attn_splitk_reduce(dw.q, dw.k_pages, dw.block_table,
                                             dw.context_lens, S, ws)
    torch.cuda.synchronize()
    o_g, lse_g, cnt = (x.cpu().numpy() for x in pa.split_views(ws, B, Hq, Hkv, S, D))
    k, v, ks, vs = oracle_pools(w)
    full = oracle.decode(w.q, k, v, w.block_table, w.context_lens, w.scale,
                         kv_dtype, ks, vs)
    total = oracle.attention.lse_of(w.q, k, v, w.block_table, w.context_lens, w.scale,
                                    kv_dtype, ks, vs)
    G = Hq // Hkv
    for b in range(B):
        L = lens[b]
        if L == 0:
            continue
        for h in range(Hkv):
            n = int(cnt[b, h])
            assert 1 <= n <= S
            if S == 1:
                assert n == 1
            a = 0
            for i in range(n):
                lse_i = lse_g[b, h * G:(h + 1) * G, i].astype(np.float64)
                assert np.all(np.isfinite(lse_i))
                if i == n - 1:      # the last range ends at L
                    o_r, lse_r = oracle.attention.range_partial(
                        w.q, k, v, w.block_table, b, h, a, L, w.scale, kv_dtype, ks, vs)
                    e, dl = L, float(np.max(np.abs(lse_r - lse_i)))
                else:
                    dl, e, o_r, lse_r = _range_end(lse_i, w.q, k, v, w.block_table, b, h, a,
                                                   L, w.scale, kv_dtype, ks, vs)
                assert dl <= 1e-4, (b, h, i, a, e, dl)
                assert e > a and (e == L or e % 32 == 0), (b, h, i, a, e)
                err = float(np.max(np.abs(o_g[b, h * G:(h + 1) * G, i] - o_r)))
                assert err <= TOL[kv_dtype], (b, h, i, a, e, err)
                a = e
            assert a == L, (b, h, a, L)
            # merging the partials in fp64 reproduces the oracle
            for j in range(h * G, (h + 1) * G):
                lse = lse_g[b, j, :n].astype(np.float64)
                assert abs(np.exp(lse - total[b, j]).sum() - 1.0) <= 2e-3
                wts = np.exp(lse - lse.max())
                merged = (wts[:, None] * o_g[b, j, :n]).sum(0) / wts.sum()
                assert np.max(np.abs(merged - full[b, j])) <= TOL[kv_dtype]
    assert max_err(out, full) <= TOL[kv_dtype]


@pytest.mark.parametrize("S,D", [(1, 64), (2, 64), (5, 64), (64, 64), (100, 64), (17, 128)])
def test_reduce_kernel_matches_oracle_merge(S, D):
    """The merge kernel alone, on partials computed by the oracle (page-aligned
    equal chunks), placed in the documented workspace layout. Empty chunks
    (lse = -inf) get NaN output rows, which must never reach the result;
    S = 100 spans two 64-lane chunks of partials."""
    say("reduce", S, D)
    pa = pa_mod()
    lens = (0, 1, 100, 777, 3000)
    B, Hq, Hkv = len(lens), 12, 3
    w = make_case(B, Hq, Hkv, D, 16, lens, seed=250 + S)
    k, v, _, _ = oracle_pools(w)
    o_r, lse_r = oracle.decode_partials(w.q, k, v, w.block_table, w.context_lens,
                                        w.scale, S)
    ref = oracle.merge_partials(o_r, lse_r)
    d = pa.PaDims(B, Hq, Hkv, D, 16, w.num_pages, w.block_table.shape[1], pa.KV_FP16)
    nbytes = pa.splitk_workspace_size(d, S)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    o_v, lse_v, cnt_v = pa.split_views(ws, B, Hq, Hkv, S, D)
    o_poisoned = o_r.astype(np.float32)
    o_poisoned[np.isneginf(lse_r)] = np.nan
    assert np.isnan(o_poisoned).any()
    o_v.copy_(torch.from_numpy(o_poisoned))
    lse_v.copy_(torch.from_numpy(lse_r.astype(np.float32)))
    cnt_v.fill_(S)
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    kp = torch.zeros((w.num_pages, Hkv, 16, D), dtype=torch.float16, device="cuda")
    bt = torch.from_numpy(w.block_table).cuda()
    out = pa.paged_decode_attn_splitk_reduce(torch.empty((B, Hq, D), dtype=torch.float16,
                                                         device="cuda"),
                                             kp, bt, lens_t, S, ws)
    torch.cuda.synchronize()
    assert max_err(out, ref) <= 2e-3


@pytest.mark.parametrize("Hq", [8, 32], ids=["merge-in-kernel", "reduce-kernel"])
def test_max_splits_one_long_sequence(Hq):
    """The largest split count (1024): one 40000-token sequence on one kv
    head is 1250 tiles, so the 1024 workers cut it into 1024 partials. With
    8 q heads the last worker to arrive merges all of them; with 32 the
    reduce kernel does, over 16 chunks of 64 partials."""
    say("max splits", Hq)
    w = make_case(1, Hq, 1, 128, 16, (40000,), seed=308)
    dw = DeviceWorkload(w)
    err = max_err(gpu_decode(dw, 1024, merged=True), oracle_out(w))
    assert err <= TOL["fp16"], err


def test_output_bitwise_invariant_under_page_permutation():
    say("page permutation")
    lens = (300, 77, 1000)
    outs = []
    for seed_pages in range(3):
        w = make_case(3, 16, 2, 128, 16, lens, seed=300)
        # re-draw only the page map: permute physical pages of the same tokens
        rng = np.random.default_rng(seed_pages)
        perm = rng.permutation(w.num_pages)
        w.block_table = perm[w.block_table].astype(np.int32)
        dw = DeviceWorkload(w)
        outs.append(gpu_decode(dw).cpu())
        outs.append(gpu_decode(dw, 5).cpu())
    for o in outs[2::2]:
        assert torch.equal(o, outs[0])
    for o in outs[3::2]:
        assert torch.equal(o, outs[1])


def test_repeated_calls_are_deterministic():
    say("determinism")
    w = make_case(4, 32, 8, 128, 16, (2000, 1, 640, 333), seed=301)
    dw = DeviceWorkload(w)
    a = [gpu_decode(dw).cpu() for _ in range(3)] + [gpu_decode(dw, 4).cpu() for _ in range(3)]
    assert all(torch.equal(a[0], x) for x in a[1:3])
    assert all(torch.equal(a[3], x) for x in a[4:6])
    # the in-kernel merge: whichever worker arrives last, the same bits
    m = [gpu_decode(dw, S, merged=True).cpu() for S in (4, 4, 4, 4, 4, 9, 9, 9, 9, 9)]
    assert all(torch.equal(m[0], x) for x in m[1:5])
    assert all(torch.equal(m[5], x) for x in m[6:])


def test_decode_step_append_then_attend():
    """One decode step as the hot path runs it: append the new token, attend."""
    say("append+attend step")
    for kv_dtype in KV_ALL:
        w = make_case(5, 16, 2, 128, 16, (1, 16, 17, 500, 64), kv_dtype=kv_dtype, seed=302)
        dw = DeviceWorkload(w, upto_last=True)
        pa = pa_mod()
        pa.kv_append(dw.new_k, dw.new_v, dw.k_pages, dw.v_pages, dw.block_table,
                     dw.positions, k_scale=dw.k_scale, v_scale=dw.v_scale)
        assert max_err(gpu_decode(dw, 3), oracle_out(w)) <= TOL[kv_dtype]


@pytest.mark.parametrize("shape", [(32, 8, 8), (48, 1, 8), (16, 2, 1)],
                         ids=["merged-in-kernel", "split+reduce", "single-pass"])
def test_graph_replay_matches_eager(shape):
    """The decode step (kv_append + attention) captured as a HIP graph gives,
    on every replay, the bits of the eager step, with other eager library
    work and synchronisations between the replays."""
    Hq, Hkv, S = shape
    say("graph replay", shape)
    pa = pa_mod()
    w = make_case(6, Hq, Hkv, 128, 16, (1500, 1, 700, 64, 2100, 333), seed=303)
    dw = DeviceWorkload(w, upto_last=True)
    ws = pa.splitk_workspace(dw.q, dw.k_pages, dw.block_table, S)
    out = torch.empty_like(dw.q)
    stream = torch.cuda.Stream()

    def step():
        pa.kv_append(dw.new_k, dw.new_v, dw.k_pages, dw.v_pages, dw.block_table,
                     dw.positions, stream=stream)
        pa.paged_decode_attn_splitk_merged(dw.q, dw.k_pages, dw.v_pages, dw.block_table,
                                           dw.context_lens, dw.scale, S, ws, out=out,
                                           stream=stream)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    ref = out.clone()
    assert max_err(ref, oracle_out(w)) <= TOL["fp16"]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        other = gpu_decode(dw, 3)          # eager library work in between
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
        assert torch.isfinite(other.float()).all()


@pytest.mark.parametrize("kv_dtype", KV_ALL)
@pytest.mark.parametrize("shape", [(32, 8, 16, 8), (48, 1, 32, 8), (16, 2, 16, 1),
                                   (8, 2, 64, 3)],
                         ids=["merged-in-kernel", "split+reduce", "single-pass", "bs64"])
def test_fused_step_matches_append_then_merged(shape, kv_dtype):
    """paged_decode_step gives the bits of kv_append followed by the merged
    call: the same output and the same cache bytes (empty and one-token
    contexts included)."""
    Hq, Hkv, bs, S = shape
    say("fused step", shape, kv_dtype)
    pa = pa_mod()
    lens = (1500, 1, 0, 700, 64, 2100, 333, 2)
    w = make_case(len(lens), Hq, Hkv, 128, bs, lens, kv_dtype=kv_dtype, seed=304)
    a = DeviceWorkload(w, upto_last=True)
    b = DeviceWorkload(w, upto_last=True)
    ws_a = pa.splitk_workspace(a.q, a.k_pages, a.block_table, S)
    ws_b = pa.splitk_workspace(b.q, b.k_pages, b.block_table, S)
    pa.kv_append(a.new_k, a.new_v, a.k_pages, a.v_pages, a.block_table, a.positions,
                 k_scale=a.k_scale, v_scale=a.v_scale)
    ref = pa.paged_decode_attn_splitk_merged(a.q, a.k_pages, a.v_pages, a.block_table,
                                             a.context_lens, a.scale, S, ws_a,
                                             a.k_scale, a.v_scale)
    out = pa.paged_decode_step(b.q, b.new_k, b.new_v, b.positions, b.k_pages, b.v_pages,
                               b.block_table, b.context_lens, b.scale, S, ws_b,
                               b.k_scale, b.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(a.k_pages.view(torch.uint8), b.k_pages.view(torch.uint8))
    assert torch.equal(a.v_pages.view(torch.uint8), b.v_pages.view(torch.uint8))
    assert torch.equal(out, ref)
    assert max_err(out, oracle_out(w)) <= TOL[kv_dtype]


def _short_lens(n):
    cycle = (0, 1, 3, 16, 31, 32, 33, 2, 7, 0, 20)
    return tuple(cycle[i % len(cycle)] for i in range(n))


@pytest.mark.parametrize("kv_dtype", KV_ALL)
@pytest.mark.parametrize("case", ["share-spans-many-pairs", "append-launched-apart"])
def test_decode_step_many_pairs(case, kv_dtype):
    """paged_decode_step with many short sequences (empty ones among them)
    gives the bits of kv_append followed by the merged call.
    share-spans-many-pairs: one long sequence and 300 short ones with two
    splits, so each worker's share holds the long pair's 100 tiles or about
    that many short pairs: the in-kernel append walks tens of pairs.
    append-launched-apart: 2400 (sequence, kv head) pairs, above the count
    where the step issues the append as a launch of its own."""
    say("decode step, many pairs", case, kv_dtype)
    pa = pa_mod()
    if case == "share-spans-many-pairs":
        lens, Hq, Hkv, S = (3200,) + _short_lens(300), 8, 2, 2
    else:
        lens, Hq, Hkv, S = _short_lens(300), 32, 8, 16
    w = make_case(len(lens), Hq, Hkv, 128, 16, lens, kv_dtype=kv_dtype, seed=307)
    a = DeviceWorkload(w, upto_last=True)
    b = DeviceWorkload(w, upto_last=True)
    ws_a = pa.splitk_workspace(a.q, a.k_pages, a.block_table, S)
    ws_b = pa.splitk_workspace(b.q, b.k_pages, b.block_table, S)
    pa.kv_append(a.new_k, a.new_v, a.k_pages, a.v_pages, a.block_table, a.positions,
                 k_scale=a.k_scale, v_scale=a.v_scale)
    ref = pa.paged_decode_attn_splitk_merged(a.q, a.k_pages, a.v_pages, a.block_table,
                                             a.context_lens, a.scale, S, ws_a,
                                             a.k_scale, a.v_scale)
    out = pa.paged_decode_step(b.q, b.new_k, b.new_v, b.positions, b.k_pages, b.v_pages,
                               b.block_table, b.context_lens, b.scale, S, ws_b,
                               b.k_scale, b.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(a.k_pages.view(torch.uint8), b.k_pages.view(torch.uint8))
    assert torch.equal(a.v_pages.view(torch.uint8), b.v_pages.view(torch.uint8))
    assert torch.equal(out, ref)
    assert max_err(out, oracle_out(w)) <= TOL[kv_dtype]


@pytest.mark.parametrize("kv_dtype", KV_ALL)
@pytest.mark.parametrize("scale", [2.0, 4.0])
def test_wide_score_range_exercises_the_rescale(scale, kv_dtype):
    """Scores spread over tens of log2 units (softmax scale far above
    1/sqrt(d)), so the running reference max of a head is bumped again and
    again inside a segment: the accumulator rescale path, on every schedule."""
    say("score range", scale, kv_dtype)
    w = make_case(5, 32, 4, 128, 16, (3000, 97, 1, 640, 1500), kv_dtype=kv_dtype,
                  seed=305, scale=scale)
    dw = DeviceWorkload(w)
    ref = oracle_out(w)
    for S, merged in ((1, False), (6, False), (6, True), (33, True)):
        err = max_err(gpu_decode(dw, S, merged=merged), ref)
        assert err <= TOL[kv_dtype], (S, merged, err)
    w2 = make_case(3, 96, 1, 128, 32, (2500, 33, 900), kv_dtype=kv_dtype, seed=306,
                   scale=scale)                       # two-wave workers, reduce kernel
    dw2 = DeviceWorkload(w2)
    assert max_err(gpu_decode(dw2, 5, merged=True), oracle_out(w2)) <= TOL[kv_dtype]


# -- full-size workloads, every sequence ------------------------------------

def _oracle_seq(w, b, new_tokens):
    """Oracle output [Hq, d] of sequence b of w after its decode-step append,
    built on a compact pool holding that sequence alone: the oracle appends
    tokens 0..L-2, then the step's token (new_tokens = w.new_tokens()) at
    position L-1 with its own kv_append, then attends."""
    cfg = w.cfg
    sub = remap_pages(w, [b])
    ks, vs = w.kv_scales()
    kp, vp = oracle.empty_pools(sub.num_pages, cfg.num_kv_heads, cfg.block_size,
                                cfg.head_dim, cfg.kv_dtype)
    K, V, sid, pos = sub.tokens([b], upto_last=True)
    if len(sid):
        kp, vp = oracle.kv_append(kp, vp, sub.block_table, sid, pos, K, V, cfg.kv_dtype,
                                  ks, vs)
    nk, nv, npos = new_tokens
    if npos[b] >= 0:
        kp, vp = oracle.kv_append(kp, vp, sub.block_table, [b], npos[b:b + 1],
                                  nk[b:b + 1], nv[b:b + 1], cfg.kv_dtype, ks, vs)
    return oracle.decode(sub.q, kp, vp, sub.block_table, sub.context_lens, sub.scale,
                         cfg.kv_dtype, ks, vs, seqs=[b])[b]


def _appended_rows(w, dw, b):
    """The new token's K and V rows of sequence b as the GPU pool holds them
    (bytes [Hkv, d] each), read at the header's layout offsets."""
    cfg = w.cfg
    p = int(w.context_lens[b]) - 1
    page = int(w.block_table[b, p // cfg.block_size])
    slot = p % cfg.block_size
    X = 8 if cfg.kv_dtype == "fp16" else 16
    i = np.arange(cfg.head_dim)
    ko = torch.from_numpy(k_offset(slot, i, cfg.head_dim, X)).cuda()
    vo = torch.from_numpy(v_offset(slot, i, cfg.head_dim)).cuda()
    kt = dw.k_pages[page].reshape(cfg.num_kv_heads, -1)
    vt = dw.v_pages[page].reshape(cfg.num_kv_heads, -1)
    return kt[:, ko].cpu().numpy(), vt[:, vo].cpu().numpy()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_mqa", "gqa_llama", "wide_mqa", "long_splitk",
                                  "mixed_fp8", "mixed_int8"])
def test_full_size_workload(name):
    """Each workload at its full size through the call the benchmark times:
    paged_decode_step (the new token appended inside the attention kernel up
    to 1536 (sequence, kv head) pairs, by a launch of its own above), with
    the workload's split count. Every sequence's output is compared with the
    oracle's, element by element, and every appended K/V row with the
    oracle's append, byte for byte."""
    say("full", name)
    pa = pa_mod()
    w = make(name, cache_tokens=True)
    cfg = w.cfg
    dw = DeviceWorkload(w, upto_last=True)
    S = cfg.num_splits
    ws = pa.splitk_workspace(dw.q, dw.k_pages, dw.block_table, S)
    out = pa.paged_decode_step(dw.q, dw.new_k, dw.new_v, dw.positions, dw.k_pages,
                               dw.v_pages, dw.block_table, dw.context_lens, dw.scale, S,
                               ws, dw.k_scale, dw.v_scale)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g))
    ks, vs = w.kv_scales()
    new_tokens = w.new_tokens()
    nk, nv, _ = new_tokens
    worst = 0.0
    for b in range(cfg.num_seqs):
        if w.context_lens[b] == 0:
            assert np.all(g[b] == 0)
            continue
        ref = _oracle_seq(w, b, new_tokens)
        err = float(np.max(np.abs(g[b] - ref)))
        worst = max(worst, err)
        assert err <= TOL[cfg.kv_dtype], (name, b, err)
        gk, gv = _appended_rows(w, dw, b)
        if cfg.kv_dtype == "fp16":
            ek, ev = nk[b].view(np.uint16), nv[b].view(np.uint16)
            gk, gv = gk.view(np.uint16), gv.view(np.uint16)
        else:
            codec = ofp8 if cfg.kv_dtype == "fp8_e4m3fn" else oi8
            ek = codec.quantize(nk[b], ks[:, None])
            ev = codec.quantize(nv[b], vs[:, None])
            gk, gv = gk.view(ek.dtype), gv.view(ev.dtype)
        assert np.array_equal(gk, ek), (name, b)
        assert np.array_equal(gv, ev), (name, b)
    say("full", name, "max err over all", cfg.num_seqs, "sequences", worst)
