"""paged_decode_step_static (the entry point that allocates nothing) against
paged_decode_step with a caller workspace, through the C ABI (needs an
MI355X).

Two calls in a row on the library's static scratch, the second on a
smaller batch with fewer splits: each gives the bits (output and cache
bytes) of paged_decode_step on an identical copy of the inputs, and is
within the path's tolerance of the oracle. Both the in-kernel merge (up to
16 q heads per kv head) and the split + reduce route (wider groups) use the
scratch.
"""
import sys

import numpy as np
import pytest
import torch

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


def _lens(rng, n, hi):
    return tuple(int(x) for x in rng.integers(0, hi, n))


CASES = {
    # (Hq, Hkv, kv dtype): first call (B, max len, S), second call (B, max len, S)
    "merge-in-kernel": (32, 8, "fp16", (32, 4096, 32), (5, 900, 8)),
    "split+reduce": (48, 1, "fp16", (12, 3000, 16), (3, 700, 4)),
    "fp8": (64, 8, "fp8_e4m3fn", (24, 3000, 16), (7, 2000, 3)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_static_step_matches_workspace_step_twice(case):
    import paged_mqa_gqa_amd as pa
    Hq, Hkv, kv, first, second = CASES[case]
    rng = np.random.default_rng(400 + len(case))
    for call, (B, hi, S) in enumerate((first, second)):
        print("[case] static step", case, "call", call, (B, hi, S), file=sys.stderr, flush=True)
        lens = _lens(rng, B, hi)
        w = make_case(B, Hq, Hkv, 128, 16, lens, kv_dtype=kv, seed=410 + call)
        a = DeviceWorkload(w, upto_last=True)
        b = DeviceWorkload(w, upto_last=True)
        d = pa.dims(B, Hq, a.k_pages, a.block_table)
        assert pa.splitk_workspace_size(d, S) <= pa.STATIC_SCRATCH_BYTES
        ws = pa.splitk_workspace(a.q, a.k_pages, a.block_table, S)
        ref = pa.paged_decode_step(a.q, a.new_k, a.new_v, a.positions, a.k_pages, a.v_pages,
                                   a.block_table, a.context_lens, a.scale, S, ws,
                                   a.k_scale, a.v_scale)
        out = pa.paged_decode_step_static(b.q, b.new_k, b.new_v, b.positions, b.k_pages,
                                          b.v_pages, b.block_table, b.context_lens, b.scale,
                                          S, b.k_scale, b.v_scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (case, call)
        assert torch.equal(a.k_pages.view(torch.uint8), b.k_pages.view(torch.uint8))
        assert torch.equal(a.v_pages.view(torch.uint8), b.v_pages.view(torch.uint8))
        k, v, ks, vs = oracle_pools(w)
        exp = oracle.decode(w.q, k, v, w.block_table, w.context_lens, w.scale, kv, ks, vs)
        got = out.float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got))
        err = float(np.max(np.abs(got - exp)))
        assert err <= TOL[kv], (case, call, err)


def test_static_step_rejects_a_request_beyond_the_scratch():
    import paged_mqa_gqa_amd as pa
    w = make_case(2, 64, 8, 128, 16, (10, 20), seed=420)
    dw = DeviceWorkload(w, upto_last=True)
    # 2 x 64 x 1024 splits x 129 floats: 67 MB of partials > 32 MiB
    with pytest.raises(pa.PagedAttnError) as e:
        pa.paged_decode_step_static(dw.q, dw.new_k, dw.new_v, dw.positions, dw.k_pages,
                                    dw.v_pages, dw.block_table, dw.context_lens, dw.scale,
                                    1024)
    assert e.value.status == -7
