"""Seeded random-shape parity sweep (needs an MI355X).

hypothesis draws shapes deterministically (derandomize=True, no example
database, no shrinking: a failing draw is reported once, never re-run over
and over on the GPU). Each draw runs through the single pass, the split pass
plus the reduce kernel, the merged call and paged_decode_step, and every
result is compared with the oracle element by element; the step's cache
bytes are compared with kv_append followed by the merged call. The first
failing draw stops the run.

Drawn: B <= 8 sequences with lengths in [0, 5000], group size G in [1, 128]
over 1, 2, 4 or 8 kv heads (at most 256 q heads), head_dim 64 or 128, page
size 16, 32 or 64, S in [1, 64] splits, fp16 / fp8 e4m3fn / int8 caches.
"""
import sys

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, Phase, given, settings
from hypothesis import strategies as st

import oracle
from tests.oracle_cases import oracle_pools
from workloads import make_case
from workloads.device import DeviceWorkload

pytestmark = pytest.mark.gpu

TOL = {"fp16": 2e-3, "fp8_e4m3fn": 3e-2, "int8": 3e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mqa_gqa_amd as pa
    pa.load()
    yield


@st.composite
def shapes(draw):
    Hkv = draw(st.sampled_from([1, 2, 4, 8]))
    G = draw(st.integers(1, min(128, 256 // Hkv)))
    B = draw(st.integers(1, 8))
    # mostly short contexts, some long ones, some empty
    lens = tuple(draw(st.lists(st.one_of(st.integers(0, 80), st.integers(0, 5000)),
                               min_size=B, max_size=B)))
    return dict(B=B, Hq=G * Hkv, Hkv=Hkv, d=draw(st.sampled_from([64, 128])),
                bs=draw(st.sampled_from([16, 32, 64])), lens=lens,
                S=draw(st.integers(1, 64)),
                kv=draw(st.sampled_from(["fp16", "fp8_e4m3fn", "int8"])),
                seed=draw(st.integers(0, 2 ** 20)))


def _err(out, ref):
    g = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), "non-finite output"
    return float(np.max(np.abs(g - ref))) if g.size else 0.0


@settings(derandomize=True, max_examples=100, deadline=None, database=None,
          phases=[Phase.explicit, Phase.generate], report_multiple_bugs=False,
          suppress_health_check=list(HealthCheck))
@given(shapes())
def test_random_shapes_all_paths(c):
    import paged_mqa_gqa_amd as pa
    print("[case] sweep", c, file=sys.stderr, flush=True)
    w = make_case(c["B"], c["Hq"], c["Hkv"], c["d"], c["bs"], c["lens"], kv_dtype=c["kv"],
                  seed=c["seed"], extra_pages=1)
    k, v, ks, vs = oracle_pools(w)
    ref = oracle.decode(w.q, k, v, w.block_table, w.context_lens, w.scale, c["kv"], ks, vs)
    tol = TOL[c["kv"]]
    S = c["S"]

    dw = DeviceWorkload(w)
    one = pa.paged_decode_attn(dw.q, dw.k_pages, dw.v_pages, dw.block_table,
                               dw.context_lens, dw.scale, dw.k_scale, dw.v_scale)
    ws = pa.paged_decode_attn_splitk(dw.q, dw.k_pages, dw.v_pages, dw.block_table,
                                     dw.context_lens, dw.scale, S, dw.k_scale, dw.v_scale)
    two = pa.paged_decode_attn_splitk_reduce(dw.q, dw.k_pages, dw.block_table,
                                             dw.context_lens, S, ws)
    ws_m = pa.splitk_workspace(dw.q, dw.k_pages, dw.block_table, S)
    merged = pa.paged_decode_attn_splitk_merged(dw.q, dw.k_pages, dw.v_pages,
                                                dw.block_table, dw.context_lens, dw.scale,
                                                S, ws_m, dw.k_scale, dw.v_scale)
    torch.cuda.synchronize()
    for name, out in (("single", one), ("split+reduce", two), ("merged", merged)):
        err = _err(out, ref)
        assert err <= tol, (name, c, err)

    # the decode step: append of each sequence's last token fused with the
    # attention, against kv_append + the merged call on a second copy
    a = DeviceWorkload(w, upto_last=True)
    b = DeviceWorkload(w, upto_last=True)
    ws_a = pa.splitk_workspace(a.q, a.k_pages, a.block_table, S)
    ws_b = pa.splitk_workspace(b.q, b.k_pages, b.block_table, S)
    pa.kv_append(a.new_k, a.new_v, a.k_pages, a.v_pages, a.block_table, a.positions,
                 k_scale=a.k_scale, v_scale=a.v_scale)
    ref_m = pa.paged_decode_attn_splitk_merged(a.q, a.k_pages, a.v_pages, a.block_table,
                                               a.context_lens, a.scale, S, ws_a,
                                               a.k_scale, a.v_scale)
    step = pa.paged_decode_step(b.q, b.new_k, b.new_v, b.positions, b.k_pages, b.v_pages,
                                b.block_table, b.context_lens, b.scale, S, ws_b,
                                b.k_scale, b.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(a.k_pages.view(torch.uint8), b.k_pages.view(torch.uint8)), c
    assert torch.equal(a.v_pages.view(torch.uint8), b.v_pages.view(torch.uint8)), c
    assert torch.equal(step, ref_m), c
    err = _err(step, ref)
    assert err <= tol, ("step", c, err)
