"""The decode projection (M == 1 GEMM over transposed weights) and the
load-time transpose against the oracle (needs an MI355X).

The weight is drawn [K, N] as a model stores it; the library builds the
[N, K] copy (transpose_weights, compared with the oracle's transpose byte
for byte) and multiplies. The tolerance is derived from the arithmetic: y
is summed in fp32 (each lane adds its share of k in sequence, at most K/64
terms, then 6 levels across the wave, plus one group-scale product for int8
weights; every fp16 x fp16 or fp16 x int8 product is exact in fp32) and
rounded once to fp16, so per element

  |y - y_ref| <= 2^-11 |y_ref| + 2^-24 (K/32 + 32) sum_k |x_k W_kn| + 2^-24

(half an fp16 ulp, the summation bound with a margin of two, the subnormal
floor).
"""
import sys

import numpy as np
import pytest
import torch

from oracle import gemm
from workloads import GEMM_CONFIGS, GemmConfig, make_gemm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mqa_gqa_amd as pa
    pa.load()
    yield


CASES = list(GEMM_CONFIGS.values()) + [
    GemmConfig("m2_fp16", 2, 512, 1000, "fp16", seed=2101),
    GemmConfig("m3_int8_g64", 3, 1024, 777, "int8", 64, seed=2102),
    GemmConfig("m4_k8192", 4, 8192, 50, "fp16", seed=2103),
    GemmConfig("tiny_int8_g16", 1, 16, 1, "int8", 16, seed=2104),
    GemmConfig("k_tail_fp16", 1, 520, 9, "fp16", seed=2105),      # 65 chunks of 8
    GemmConfig("k16384_int8", 2, 16384, 300, "int8", 128, seed=2106),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_gemm_m1_against_oracle(cfg):
    import paged_mqa_gqa_amd as pa
    print("[case] gemm", cfg, file=sys.stderr, flush=True)
    x, w, s = make_gemm(cfg)
    xd = torch.from_numpy(x).cuda()
    wd = torch.from_numpy(w).cuda()
    wt = pa.transpose_weights(wd)
    st = pa.transpose_weights(torch.from_numpy(s).cuda()) if s is not None else None
    y = pa.gemm_m1_transposed(xd, wt, st, cfg.group)
    torch.cuda.synchronize()
    # the load-time transposes, bit for bit
    wt_ref = gemm.transpose(w)
    assert np.array_equal(wt.cpu().numpy().view(np.uint8), wt_ref.view(np.uint8))
    st_ref = gemm.transpose(s) if s is not None else None
    if s is not None:
        assert np.array_equal(st.cpu().numpy().view(np.uint32), st_ref.view(np.uint32))
    ref = gemm.gemm_m1(x, wt_ref, st_ref, cfg.group)
    absp = gemm.abs_products(x, wt_ref, st_ref, cfg.group)
    got = y.float().cpu().numpy().astype(np.float64)
    assert got.shape == (cfg.M, cfg.N) and np.all(np.isfinite(got))
    tol = 2.0 ** -11 * np.abs(ref) + 2.0 ** -24 * (cfg.K / 32 + 32) * absp + 2.0 ** -24
    bad = np.abs(got - ref) > tol
    print("[case] gemm", cfg.name, "max err", float(np.max(np.abs(got - ref))),
          "max err/tol", float(np.max(np.abs(got - ref) / tol)), file=sys.stderr, flush=True)
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:5])


@pytest.mark.parametrize("shape,dtype", [((33, 70), torch.int8), ((64, 64), torch.float16),
                                         ((4096, 130), torch.float16),
                                         ((7, 4864), torch.float32), ((1, 1), torch.int8)])
def test_transpose_weights_bit_exact(shape, dtype):
    """Random bytes (NaN and inf patterns included) moved bit for bit."""
    import paged_mqa_gqa_amd as pa
    elem = {torch.int8: 1, torch.float16: 2, torch.float32: 4}[dtype]
    raw = np.random.default_rng(9).integers(0, 256, shape[0] * shape[1] * elem, dtype=np.uint8)
    t = torch.from_numpy(raw).view(dtype).reshape(shape)
    out = pa.transpose_weights(t.cuda())
    torch.cuda.synchronize()
    assert out.shape == (shape[1], shape[0])
    assert torch.equal(out.cpu().view(torch.uint8), t.T.contiguous().view(torch.uint8))
