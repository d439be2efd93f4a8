"""Decode steps replayed from one captured graph, step values on the device
(needs an MI355X).

One graph holds a whole decode step: paged_decode_step (append of every
live sequence's new token + attention) followed by paged_decode_advance,
which moves each live slot's append position and context length on by one
token in device memory. The pool has room for the steps ahead: the page
manager reserves each sequence's pages for ten more tokens before capture.
The host writes only the next step's q and new K/V rows into the fixed
input buffers before each replay (in a model they come from the preceding
projection). After every replay the output is compared with the oracle,
which appends the same tokens with its own kv_append and attends over one
more token each step; after the last, the whole cache is compared with the
oracle's byte for byte, and the step values with their expected values.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_mqa_gqa_amd as pa
from workloads import make_case

pytestmark = pytest.mark.gpu

TOL = {"fp16": 2e-3, "fp8_e4m3fn": 3e-2, "int8": 3e-2}
STEPS = 10


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load()
    yield


@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8_e4m3fn", "int8"])
@pytest.mark.parametrize("shape", [(32, 8, 8), (48, 1, 6), (16, 2, 1)],
                         ids=["merge-in-kernel", "split+reduce", "single-pass"])
def test_graph_replays_advance_step_values_on_device(shape, kv_dtype):
    Hq, Hkv, S = shape
    print("[case] graph steps", shape, kv_dtype, file=sys.stderr, flush=True)
    lens = (1500, 1, 0, 700, 15, 2100, 333, 31)          # slot 2 is free
    B, d, bs = len(lens), 128, 16
    w = make_case(B, Hq, Hkv, d, bs, lens, kv_dtype=kv_dtype, seed=500)
    cfg = w.cfg
    ks, vs = w.kv_scales()
    max_blocks = -(-(max(lens) + STEPS) // bs)
    P = sum(-(-(L + STEPS) // bs) for L in lens) + 4
    # pages: every live slot holds its first L - 1 tokens and room for STEPS more
    m = pa.KvPageManager(P, bs, B, max_blocks)
    for L in lens:
        assert m.admit(max(L - 1, 0)) >= 0
    m.release(2)
    m.reserve_ahead(STEPS)
    bt = m.block_table()

    # the cache before the first step: tokens 0..L-2 of every live slot
    # both pools start as the never-written marker (NaN codes, int8 -128)
    okp, ovp = oracle.empty_pools(P, Hkv, bs, d, kv_dtype)
    kp = torch.from_numpy(okp.copy()).cuda()
    vp = torch.from_numpy(ovp.copy()).cuda()
    K, V, sid, pos0 = w.tokens([b for b in range(B) if b != 2], upto_last=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    k_scale = dev(ks) if kv_dtype != "fp16" else None
    v_scale = dev(vs) if kv_dtype != "fp16" else None
    bt_d = dev(bt)
    pa.kv_append(dev(K), dev(V), kp, vp, bt_d, dev(pos0), seq_ids=dev(sid),
                 k_scale=k_scale, v_scale=v_scale)
    oracle.kv_append(okp, ovp, bt, sid, pos0, K, V, kv_dtype, ks, vs, inplace=True)

    # fixed device buffers of the step values and inputs
    lens0 = np.array([0 if b == 2 else L for b, L in enumerate(lens)], np.int32)
    pos_first = np.where(lens0 > 0, lens0 - 1, -1).astype(np.int32)
    lens_d, pos_d = dev(lens0), dev(pos_first)
    q_buf = torch.zeros((B, Hq, d), dtype=torch.float16, device="cuda")
    kn_buf = torch.zeros((B, Hkv, d), dtype=torch.float16, device="cuda")
    vn_buf = torch.zeros_like(kn_buf)
    out = torch.zeros_like(q_buf)
    ws = torch.zeros(max(pa.splitk_workspace_size(pa.dims(B, Hq, kp, bt_d), S), 1),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()

    def step():
        pa.paged_decode_step(q_buf, kn_buf, vn_buf, pos_d, kp, vp, bt_d, lens_d, w.scale, S,
                             ws, k_scale, v_scale, out=out, stream=stream)
        pa.paged_decode_advance(lens_d, pos_d, kp, bt_d, stream=stream)

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()

    cur_lens = lens0.copy()
    for t in range(STEPS):
        # the step's inputs: the workload's own last token first, then later ones
        if t == 0:
            q = w.q
            nk, nv, _ = w.new_tokens()
        else:
            q, nk, nv = w.step_inputs(t)
        with torch.cuda.stream(stream):
            q_buf.copy_(torch.from_numpy(q))
            kn_buf.copy_(torch.from_numpy(nk))
            vn_buf.copy_(torch.from_numpy(nv))
            out.zero_()
            g.replay()
        torch.cuda.synchronize()
        live = [b for b in range(B) if cur_lens[b] > 0]
        p = cur_lens[live] - 1
        oracle.kv_append(okp, ovp, bt, live, p, nk[live], nv[live], kv_dtype, ks, vs,
                         inplace=True)
        ref = oracle.decode(q, okp, ovp, bt, cur_lens, w.scale, kv_dtype, ks, vs, seqs=live)
        got = out.float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got))
        err = float(np.max(np.abs(got - ref)))
        assert err <= TOL[kv_dtype], (t, err)
        assert np.all(got[2] == 0)
        cur_lens[live] += 1
    assert np.array_equal(lens_d.cpu().numpy(), cur_lens)
    assert np.array_equal(pos_d.cpu().numpy(), np.where(cur_lens > 0, cur_lens - 1, -1))
    assert np.array_equal(kp.cpu().numpy().view(np.uint8), okp.view(np.uint8))
    assert np.array_equal(vp.cpu().numpy().view(np.uint8), ovp.view(np.uint8))
    m.commit_steps(STEPS)
    assert [m.length(b) for b in range(B)] == [int(L) - 1 if L > 0 else -1 for L in cur_lens]


def test_advance_stops_at_the_block_table_capacity():
    """A slot whose next position would leave its block table row stops
    appending (position -1) and keeps its length; free slots stay as they are."""
    lens = torch.tensor([31, 5, 0, 32], dtype=torch.int32, device="cuda")
    pos = torch.tensor([30, 4, -1, 31], dtype=torch.int32, device="cuda")
    kp = torch.zeros((4, 1, 16, 64), dtype=torch.float16, device="cuda")
    bt = torch.zeros((4, 2), dtype=torch.int32, device="cuda")       # capacity 32
    pa.paged_decode_advance(lens, pos, kp, bt)
    torch.cuda.synchronize()
    assert lens.tolist() == [32, 6, 0, 32]
    assert pos.tolist() == [31, 5, -1, -1]
