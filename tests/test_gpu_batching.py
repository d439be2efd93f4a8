"""Continuous batching over a preallocated paged cache (needs an MI355X).

The mixed continuous batch (256 slots, 64 q / 8 kv heads, head_dim 128,
pages of 16 tokens, log-normal prompt lengths with median 1024, fp8 e4m3fn
cache with per-head scales) runs as a live loop: the pool is allocated once,
sized by the KV formula for the tokens it must hold; the page manager admits
sequences (prefill: their prompt appended with kv_append through the
manager's block table), releases finished ones, and before each step gives
every live sequence the page of its next token. Each step is one
paged_decode_step over the fixed 256-slot batch, free slots taking part as
empty sequences. The oracle mirrors every append on its own pools through
the same block table; after every step each live sequence's output is
compared with the oracle's and free slots must be zero; after the last step
the whole cache is compared byte for byte.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_mqa_gqa_amd as pa
from workloads import CONFIGS, Workload, arrivals

pytestmark = pytest.mark.gpu

TOL = {"fp16": 2e-3, "fp8_e4m3fn": 3e-2, "int8": 3e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load()
    yield


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixed_fp8", "mixed_int8"])
def test_continuous_batching_loop(name):
    cfg = CONFIGS[name]
    steps, first_live, joins, leaves = 6, 232, 5, 6
    w = Workload(cfg, cache_tokens=True)
    B, Hq, Hkv, d, bs = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, \
        cfg.block_size
    kv = cfg.kv_dtype
    kvd = {"fp16": pa.KV_FP16, "fp8_e4m3fn": pa.KV_FP8_E4M3FN, "int8": pa.KV_INT8}[kv]
    ks, vs = w.kv_scales()
    arrivals_by_step = [arrivals(cfg, joins, tag=t) for t in range(steps)]
    # pool sized by the KV formula for every token the run can hold (plus a
    # page of slack per slot), allocated once
    tokens = int(w.context_lens[:first_live].sum()) + sum(int(a[0].sum()) for a in
                                                           arrivals_by_step)
    tokens += B * (steps + bs)
    P = int(pa.kv_pages_for_budget(pa.kv_bytes_per_sequence(1, Hkv, d, tokens, kvd),
                                   1, Hkv, d, bs, kvd))
    assert pa.kv_pool_bytes(P, Hkv, d, bs, kvd) <= pa.kv_bytes_per_sequence(1, Hkv, d,
                                                                            tokens, kvd)
    max_blocks = cfg.max_blocks + 1
    say("batching", name, "pages", P, "pool MB", pa.kv_pool_bytes(P, Hkv, d, bs, kvd) / 1e6)
    m = pa.KvPageManager(P, bs, B, max_blocks)
    okp, ovp = oracle.empty_pools(P, Hkv, bs, d, kv)
    kp = torch.from_numpy(okp).cuda()
    vp = torch.from_numpy(ovp).cuda()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    k_scale, v_scale = dev(ks), dev(vs)
    rng = np.random.default_rng(600)

    def prefill(slot, K, V):
        """The prompt of a newly admitted slot, appended on both sides."""
        T = K.shape[0]
        if T == 0:
            return
        bt = m.block_table()
        sid = np.full(T, slot, np.int32)
        pos = np.arange(T, dtype=np.int32)
        pa.kv_append(dev(K), dev(V), kp, vp, dev(bt), dev(pos), seq_ids=dev(sid),
                     k_scale=k_scale, v_scale=v_scale)
        oracle.kv_append(okp, ovp, bt, sid, pos, K, V, kv, ks, vs, inplace=True)

    for b in range(first_live):
        slot = m.admit(int(w.context_lens[b]))
        assert slot == b
        K, V = w.token_kv(b)
        prefill(slot, K, V)
    torch.cuda.synchronize()

    S = cfg.num_splits
    out = torch.empty((B, Hq, d), dtype=torch.float16, device="cuda")
    ws = None
    for t in range(steps):
        if t > 0:                                   # finished sequences leave
            live = [s for s in range(B) if m.length(s) >= 0]
            for s in rng.choice(live, leaves, replace=False):
                m.release(int(s))
        lens_new, prompts = arrivals_by_step[t]     # new sequences join
        for L, (K, V) in zip(lens_new, prompts):
            slot = m.admit(int(L))
            prefill(slot, K, V)
        bt, lens, pos = m.plan_step()
        live = [s for s in range(B) if lens[s] > 0]
        q, nk, nv = w.step_inputs(t + 1)
        bt_d = dev(bt)
        if ws is None:
            ws = pa.splitk_workspace(dev(q), kp, bt_d, S)
        pa.paged_decode_step(dev(q), dev(nk), dev(nv), dev(pos), kp, vp, bt_d, dev(lens),
                             w.scale, S, ws, k_scale, v_scale, out=out)
        torch.cuda.synchronize()
        oracle.kv_append(okp, ovp, bt, live, pos[live], nk[live], nv[live], kv, ks, vs,
                         inplace=True)
        ref = oracle.decode(q, okp, ovp, bt, lens, w.scale, kv, ks, vs, seqs=live)
        got = out.float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got))
        err = float(np.max(np.abs(got[live] - ref[live])))
        free = [s for s in range(B) if lens[s] == 0]
        say("batching", name, "step", t, "live", len(live), "free", len(free),
            "free pages", m.free_pages, "max err", err)
        assert err <= TOL[kv], (t, err)
        assert np.all(got[free] == 0)
    assert np.array_equal(kp.cpu().numpy().view(np.uint8), okp.view(np.uint8))
    assert np.array_equal(vp.cpu().numpy().view(np.uint8), ovp.view(np.uint8))
