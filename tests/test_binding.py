"""The Python binding rejects mismatched tensors before any launch (CPU only).

Every call here uses CPU tensors. A call whose shapes and dtypes are all
right gets as far as the device check ("must be a GPU tensor") and stops
there; a call with one wrong shape, dtype or length stops earlier, at a
message naming that argument. Either way no pointer reaches the library.
"""
import pytest
import torch

import paged_mqa_gqa_amd as pa

B, HQ, HKV, D, BS, P, MB = 3, 8, 2, 128, 16, 20, 4


def _args(kv="fp16"):
    pool_dtype = {"fp16": torch.float16, "fp8": torch.uint8, "int8": torch.int8}[kv]
    a = dict(q=torch.zeros(B, HQ, D, dtype=torch.float16),
             k_new=torch.zeros(B, HKV, D, dtype=torch.float16),
             v_new=torch.zeros(B, HKV, D, dtype=torch.float16),
             positions=torch.zeros(B, dtype=torch.int32),
             k_pages=torch.zeros(P, HKV, BS, D, dtype=pool_dtype),
             v_pages=torch.zeros(P, HKV, BS, D, dtype=pool_dtype),
             block_table=torch.zeros(B, MB, dtype=torch.int32),
             context_lens=torch.ones(B, dtype=torch.int32),
             scale=0.1, num_splits=4,
             workspace=torch.zeros(1 << 16, dtype=torch.uint8),
             k_scale=None, v_scale=None, out=torch.zeros(B, HQ, D, dtype=torch.float16))
    if kv != "fp16":
        a["k_scale"] = torch.ones(HKV, dtype=torch.float32)
        a["v_scale"] = torch.ones(HKV, dtype=torch.float32)
    return a


def _step(**a):
    return pa.paged_decode_step(**a)


@pytest.mark.parametrize("kv", ["fp16", "fp8", "int8"])
def test_well_formed_call_reaches_the_device_check(kv):
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        _step(**_args(kv))


BAD = {
    "out rows": ("out", torch.zeros(B - 1, HQ, D, dtype=torch.float16), "out"),
    "out head_dim": ("out", torch.zeros(B, HQ, D // 2, dtype=torch.float16), "out"),
    "out dtype": ("out", torch.zeros(B, HQ, D, dtype=torch.float32), "out"),
    "k_new heads": ("k_new", torch.zeros(B, HKV + 1, D, dtype=torch.float16), "k_new"),
    "k_new rows": ("k_new", torch.zeros(B - 1, HKV, D, dtype=torch.float16), "k_new"),
    "v_new dims": ("v_new", torch.zeros(B, HKV, 64, dtype=torch.float16), "v_new"),
    "positions length": ("positions", torch.zeros(B + 1, dtype=torch.int32), "positions"),
    "positions dtype": ("positions", torch.zeros(B, dtype=torch.int64), "positions"),
    "context_lens length": ("context_lens", torch.ones(B - 1, dtype=torch.int32),
                            "context_lens"),
    "block_table rows": ("block_table", torch.zeros(B + 2, MB, dtype=torch.int32),
                         "block_table"),
    "q head_dim": ("q", torch.zeros(B, HQ, 64, dtype=torch.float16), "head_dim"),
    "v_pages shape": ("v_pages", torch.zeros(P + 1, HKV, BS, D, dtype=torch.float16),
                      "v_pages"),
    "v_pages dtype": ("v_pages", torch.zeros(P, HKV, BS, D, dtype=torch.uint8), "v_pages"),
    "workspace missing": ("workspace", None, "workspace"),
}


@pytest.mark.parametrize("case", list(BAD))
def test_mismatch_raises_before_any_launch(case):
    key, value, name = BAD[case]
    a = _args()
    a[key] = value
    with pytest.raises((ValueError, TypeError), match=name):
        _step(**a)


@pytest.mark.parametrize("kv", ["fp8", "int8"])
@pytest.mark.parametrize("which", ["k_scale", "v_scale"])
def test_scale_length_and_presence(kv, which):
    a = _args(kv)
    a[which] = torch.ones(HKV + 1, dtype=torch.float32)
    with pytest.raises(ValueError, match=which):
        _step(**a)
    a[which] = None
    with pytest.raises(ValueError, match=which):
        _step(**a)


def test_attention_calls_check_out_and_lens():
    a = _args()
    common = dict(q=a["q"], k_pages=a["k_pages"], v_pages=a["v_pages"],
                  block_table=a["block_table"], context_lens=a["context_lens"], scale=0.1)
    bad_out = torch.zeros(B, HQ + 1, D, dtype=torch.float16)
    with pytest.raises(ValueError, match="out"):
        pa.paged_decode_attn(**common, out=bad_out)
    with pytest.raises(ValueError, match="out"):
        pa.paged_decode_attn_splitk_merged(**common, num_splits=4, workspace=a["workspace"],
                                           out=bad_out)
    with pytest.raises(ValueError, match="out"):
        pa.paged_decode_attn_splitk_reduce(a["q"], a["k_pages"], a["block_table"],
                                           a["context_lens"], 4, a["workspace"], out=bad_out)
    with pytest.raises(ValueError, match="context_lens"):
        pa.paged_decode_attn_splitk_reduce(a["q"], a["k_pages"], a["block_table"],
                                           torch.ones(B + 1, dtype=torch.int32), 4,
                                           a["workspace"])
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        pa.paged_decode_attn(**common, out=a["out"])


def test_kv_append_checks_rows_and_lengths():
    a = _args()
    T = 5
    kn = torch.zeros(T, HKV, D, dtype=torch.float16)
    pos = torch.zeros(T, dtype=torch.int32)
    sid = torch.zeros(T, dtype=torch.int32)
    call = lambda **kw: pa.kv_append(**{**dict(
        k_new=kn, v_new=kn, k_pages=a["k_pages"], v_pages=a["v_pages"],
        block_table=a["block_table"], positions=pos, seq_ids=sid), **kw})
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        call()
    with pytest.raises(ValueError, match="k_new"):
        call(k_new=torch.zeros(T, HKV + 1, D, dtype=torch.float16))
    with pytest.raises(ValueError, match="v_new"):
        call(v_new=torch.zeros(T + 1, HKV, D, dtype=torch.float16))
    with pytest.raises(ValueError, match="positions"):
        call(positions=torch.zeros(T - 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="seq_ids"):
        call(seq_ids=torch.zeros(T + 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="num_seqs"):
        call(num_seqs=B + 1)
