"""CPU oracle for paged MQA/GQA decode attention (test infrastructure only).

This package is a plain, slow, fp64 statement of what the decode path
computes. It exists to check the HIP library and nothing else: only the test
suite, the smoke check of the package entry file and the CPU-baseline leg of
the benchmark may import it. The library and its Python binding never do, and
this package imports nothing from them.

Contents
  fp8        e4m3fn decode/encode from the OCP 8-bit floating point format
  int8       symmetric int8 codes with a per-head scale
  paged      cache append (scatter) and block-table gather
  attention  single-token decode attention, split partials and their merge
  gemm       the M == 1 decode projection over transposed (fp16 or int8) weights

Sources, by page title and section:
  * "TensorRT对Multi-Query Attention的专项优化支持" (r-odyssey.com/news/246352):
    the MHA and MQA formulas (every query head keeps its own projection, the
    K/V projection is shared), decode re-reading every cached K/V for each
    new token, and the paragraph on fixed-length KV pages.
  * "优化" on tiny-llm (open-infra-ai.github.io/tiny-llm/performance/optimization):
    roadmap table, row 分页 KV (block table + scatter/gather, checked token by
    token against contiguous KV) and row FlashDecoding (long-context decode
    attention, named only); section 3 (GQA: kv heads may differ from q heads);
    section 4 (the M == 1 GEMM over transposed weights) and section 1 (int8
    weights with group-wise scales).
  * zyxy.net tag page "tensorrt", FMHA abstract: attention as projections,
    scores, softmax, weighted sum.

Parity status: every function here is pinned by tests/test_oracle_*.py
against closed forms, library routines (torch SDPA in float64, torch's
float8_e4m3fn cast, torch's round-half-even and clamp, scipy logsumexp),
mpmath brute force and invariants.
"""
from . import fp8, int8, paged, attention, gemm  # noqa: F401
from .attention import decode, decode_partials, merge_partials, split_bounds  # noqa: F401
from .paged import kv_append, gather, empty_pools  # noqa: F401
