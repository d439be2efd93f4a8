"""C ABI checks that need no GPU: symbols, status strings, host validation.

Every call here fails validation on the host, which happens before anything
touches a device, so no GPU is needed. Pointers are dummy non-null values
that the library must never dereference on these paths.
"""
import ctypes
import os
import re
import subprocess

import pytest

import paged_mqa_gqa_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h)
           for h in ("paged_attn.h", "paged_kv_manager.h", "decode_gemm.h")]

pytestmark = pytest.mark.skipif(not os.path.exists(pa.library_path()),
                                reason="library not built")

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def _declared():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, re.M))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["kv_append", "paged_decode_attn", "paged_decode_attn_splitk",
              "paged_decode_attn_splitk_reduce", "paged_decode_attn_splitk_merged",
              "paged_decode_step", "paged_decode_attn_splitk_workspace_size",
              "paged_decode_attn_suggest_splits", "paged_decode_step_fuses_append",
              "paged_decode_step_static", "paged_decode_advance",
              "pa_status_string", "pa_version", "pa_kvm_create", "pa_kvm_plan_step",
              "pa_kvm_admit", "pa_kvm_release", "pa_kvm_reserve_ahead",
              "pa_kv_bytes_per_sequence", "pa_kv_pool_bytes",
              "gemm_m1_transposed", "transpose_weights"]:
        assert n in names, n


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", pa.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing


def good_dims(**kw):
    d = dict(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
             block_size=16, num_pages=10, max_blocks_per_seq=4,
             kv_dtype=pa.KV_FP16)
    d.update(kw)
    return pa.PaDims(**d)


def attn(d, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, ks=None, vs=None, out=FAKE)
    args.update(kw)
    return pa.load().paged_decode_attn(ctypes.byref(d) if d is not None else None,
                                       args["q"], args["k"], args["v"], args["bt"],
                                       args["lens"], 0.1, args["ks"], args["vs"],
                                       args["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=6, num_kv_heads=4), -2),     # Hq % Hkv != 0
    (dict(head_dim=96), -2),
    (dict(block_size=8), -2),
    (dict(block_size=128), -2),
    (dict(num_kv_heads=0), -2),
    (dict(num_pages=0), -2),
    (dict(max_blocks_per_seq=0), -2),
    (dict(num_seqs=-1), -2),
    (dict(num_q_heads=2 * 129, num_kv_heads=2), -2),  # G > 128
    (dict(kv_dtype=7), -3),
])
def test_bad_dims_rejected(kw, status):
    assert attn(good_dims(**kw)) == status


def test_null_pointers_rejected():
    assert attn(None) == -1
    for key in ["q", "k", "v", "bt", "lens", "out"]:
        assert attn(good_dims(), **{key: None}) == -1, key


def test_decode_step_validation():
    lib = pa.load()
    d = good_dims()
    need = lib.paged_decode_attn_splitk_workspace_size(ctypes.byref(d), 4)

    def step(dims=d, kn=FAKE, vn=FAKE, pos=FAKE, q=FAKE, S=4, ws=FAKE, n=need, out=FAKE):
        return lib.paged_decode_step(ctypes.byref(dims) if dims is not None else None,
                                     q, kn, vn, pos, FAKE, FAKE, FAKE, FAKE, 0.1,
                                     None, None, S, ws, n, out, None)
    assert step(dims=None) == -1
    assert step(kn=None) == -1 and step(vn=None) == -1 and step(pos=None) == -1
    assert step(q=None) == -1 and step(out=None) == -1
    assert step(dims=good_dims(head_dim=96)) == -2
    assert step(S=0) == -4
    assert step(n=need - 1) == -5
    assert step(dims=good_dims(kv_dtype=pa.KV_FP8_E4M3FN)) == -3
    assert step(dims=good_dims(num_seqs=0)) == 0
    # above 1536 (sequence, kv head) pairs the append is launched apart from
    # the attention: every check still comes first, so nothing is launched
    # (a launch on a machine without a GPU would report -6 instead)
    big = good_dims(num_seqs=1000, num_kv_heads=2, num_q_heads=8)
    need_big = lib.paged_decode_attn_splitk_workspace_size(ctypes.byref(big), 4)
    assert step(dims=big, n=need_big - 1) == -5
    assert step(dims=big, S=0) == -4
    assert step(dims=big, out=None) == -1
    assert step(dims=good_dims(num_seqs=1000, kv_dtype=pa.KV_FP8_E4M3FN)) == -3


@pytest.mark.parametrize("kv", [pa.KV_FP8_E4M3FN, pa.KV_INT8])
def test_one_byte_caches_require_scales(kv):
    assert attn(good_dims(kv_dtype=kv)) == -3
    assert attn(good_dims(kv_dtype=kv), ks=FAKE) == -3
    assert attn(good_dims(kv_dtype=kv), vs=FAKE) == -3
    # with both scales the int8 and fp8 kinds pass validation (an empty
    # batch then returns before any launch)
    assert attn(good_dims(kv_dtype=kv, num_seqs=0), ks=FAKE, vs=FAKE) == 0


def test_workspace_counters_sit_at_a_fixed_offset():
    """The merged call's arrival counters are the first 2048 int32 of every
    workspace, whatever the dims and split count: a workspace reused by
    calls of shrinking or growing size never has partials where another
    call keeps its counters. The partials follow them."""
    lib = pa.load()
    sizes = set()
    for B, Hq, Hkv, S in ((2, 8, 2, 4), (7, 32, 8, 16), (1, 96, 1, 64), (300, 64, 8, 2)):
        d = good_dims(num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv)
        n = lib.paged_decode_attn_splitk_workspace_size(ctypes.byref(d), S)
        rows = B * Hq * S
        assert n == 2048 * 4 + rows * 128 * 4 + rows * 4 + B * Hkv * 4
        sizes.add(n)
        import torch
        ws = torch.zeros(n, dtype=torch.uint8)
        o, lse, cnt = pa.split_views(ws, B, Hq, Hkv, S, 128)
        base = ws.data_ptr()
        assert o.data_ptr() - base == 2048 * 4
        assert lse.data_ptr() - base == 2048 * 4 + rows * 128 * 4
        assert cnt.data_ptr() - base == 2048 * 4 + rows * 128 * 4 + rows * 4
        assert pa.sem_view(ws).data_ptr() == base and pa.sem_view(ws).numel() == 2048
    assert len(sizes) == 4


def test_empty_batch_is_a_no_op():
    assert attn(good_dims(num_seqs=0)) == 0


def test_splitk_validation():
    lib = pa.load()
    d = good_dims()
    need = lib.paged_decode_attn_splitk_workspace_size(ctypes.byref(d), 4)
    # arrival counters (fixed 2048 slots), o [B,Hq,S,d], lse [B,Hq,S], count [B,Hkv]
    assert need == 2048 * 4 + 2 * 8 * 4 * 128 * 4 + 2 * 8 * 4 * 4 + 2 * 2 * 4
    assert lib.paged_decode_attn_splitk_workspace_size(ctypes.byref(d), 0) == 0
    call = lambda S, ws, n: lib.paged_decode_attn_splitk(
        ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, None, None, S, ws, n, None)
    assert call(0, FAKE, need) == -4
    assert call(1025, FAKE, 10 ** 9) == -4
    assert call(4, FAKE, need - 1) == -5
    assert call(4, None, need) == -5
    red = lambda S, ws, n, out=FAKE, lens=FAKE: lib.paged_decode_attn_splitk_reduce(
        ctypes.byref(d), lens, S, ws, n, out, None)
    assert red(4, FAKE, need - 4) == -5
    assert red(0, FAKE, need) == -4
    assert red(4, FAKE, need, None) == -1
    assert red(4, FAKE, need, FAKE, None) == -1
    mer = lambda S, ws, n, out=FAKE: lib.paged_decode_attn_splitk_merged(
        ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, None, None, S, ws, n, out, None)
    assert mer(0, FAKE, need) == -4
    assert mer(4, FAKE, need - 1) == -5
    assert mer(4, None, need) == -5
    assert mer(4, FAKE, need, None) == -1


def test_kv_append_validation():
    lib = pa.load()
    d = good_dims()
    call = lambda T, sid=FAKE, **kw: lib.kv_append(
        ctypes.byref(d), T, kw.get("k", FAKE), FAKE, sid, FAKE, FAKE,
        kw.get("ks"), kw.get("vs"), FAKE, FAKE, None)
    assert call(-1) == -2
    assert call(3, sid=None) == -2          # T > B without seq_ids
    assert call(2, k=None) == -1
    assert call(0) == 0                     # nothing to do
    d8 = good_dims(kv_dtype=pa.KV_FP8_E4M3FN)
    assert lib.kv_append(ctypes.byref(d8), 1, FAKE, FAKE, None, FAKE, FAKE, None,
                         None, FAKE, FAKE, None) == -3


def test_static_step_rejects_requests_beyond_its_scratch():
    """paged_decode_step_static checks every argument and the scratch size
    before it touches any device: errors come back on a machine with no GPU."""
    lib = pa.load()

    def call(d, S, out=FAKE, kn=FAKE):
        return lib.paged_decode_step_static(ctypes.byref(d), FAKE, kn, FAKE, FAKE, FAKE,
                                            FAKE, FAKE, FAKE, 0.1, None, None, S, out, None)
    # mixed continuous batch: 256 sequences x 64 q heads x 16 splits of
    # 129 floats = 135 MB of partials > 32 MiB
    big = good_dims(num_seqs=256, num_q_heads=64, num_kv_heads=8)
    assert lib.paged_decode_attn_splitk_workspace_size(ctypes.byref(big), 16) > 32 << 20
    assert call(big, 16) == -7
    assert pa.status_string(-7) != pa.status_string(-99)
    # a request that fits is checked like paged_decode_step
    small = good_dims(num_seqs=32, num_q_heads=32, num_kv_heads=8)
    assert lib.paged_decode_attn_splitk_workspace_size(ctypes.byref(small), 32) <= 32 << 20
    assert call(small, 32, out=None) == -1
    assert call(small, 32, kn=None) == -1
    assert call(small, 0) == -4
    assert call(good_dims(head_dim=96), 4) == -2
    assert call(good_dims(kv_dtype=pa.KV_INT8), 4) == -3
    assert call(good_dims(num_seqs=0), 4) == 0


def test_status_strings_and_version():
    for s in [0, -1, -2, -3, -4, -5, -6, -7, -99]:
        assert isinstance(pa.status_string(s), str) and pa.status_string(s)
    assert pa.version() >= 100


def test_suggest_splits():
    d = pa.PaDims(256, 64, 8, 128, 16, 30000, 2048, pa.KV_FP8_E4M3FN)
    assert pa.suggest_splits(d, 32768) == 17       # 16*2048/2048 + 1
    d1 = pa.PaDims(256, 64, 8, 128, 16, 30000, 2048, pa.KV_FP16)
    assert pa.suggest_splits(d1, 32768) == 9       # 16*1024/2048 + 1
    d2 = pa.PaDims(32, 32, 8, 128, 16, 5000, 256, pa.KV_FP16)
    assert pa.suggest_splits(d2, 4096) == 64       # 16*1024/256 + 1, capped
    d4 = pa.PaDims(4, 32, 8, 128, 64, 9000, 2048, pa.KV_FP16)
    assert pa.suggest_splits(d4, 131072) == 64      # capped
    assert pa.suggest_splits(d4, 1) == 1
    assert pa.suggest_splits(d4, 40) == 3           # two tiles -> at most 3
    d3 = pa.PaDims(64, 96, 1, 128, 32, 20000, 256, pa.KV_FP16)
    assert pa.suggest_splits(d3, 8192) == 64


def test_decode_step_fusion_query():
    """The step appends inside the attention kernel up to 1536 (sequence,
    kv head) pairs and in a launch of its own above."""
    assert pa.step_fuses_append(good_dims()) is True
    assert pa.step_fuses_append(good_dims(num_seqs=768, num_kv_heads=2)) is True
    assert pa.step_fuses_append(good_dims(num_seqs=769, num_kv_heads=2)) is False
    assert pa.step_fuses_append(good_dims(num_seqs=256, num_kv_heads=8,
                                          num_q_heads=64)) is False
    assert pa.load().paged_decode_step_fuses_append(None) == -1
    with pytest.raises(pa.PagedAttnError):
        pa.step_fuses_append(good_dims(head_dim=96))


def test_gemm_validation():
    """The decode projection's argument checks (no device is touched)."""
    lib = pa.load()
    A = ctypes.c_void_p(0x1000)            # 16-byte aligned, never dereferenced

    def call(M=1, N=8, K=64, dt=pa.W_FP16, g=0, x=A, wt=A, sc=None, y=A):
        return lib.gemm_m1_transposed(M, N, K, dt, g, x, wt, sc, y, None)
    assert call(M=0) == -2 and call(M=5) == -2 and call(N=0) == -2
    assert call(K=60) == -2                     # fp16: K % 8
    assert call(dt=pa.W_INT8, K=72, g=8, sc=A) == -2     # group not a multiple of 16
    assert call(dt=pa.W_INT8, K=72, g=16, sc=A) == -2    # K not a multiple of the group
    assert call(dt=pa.W_INT8, K=64, g=16) == -1          # scales missing
    assert call(dt=7) == -3
    assert call(M=4, K=8200) == -2                       # activations exceed 64 KB
    assert call(x=None) == -1 and call(y=None) == -1
    assert call(x=ctypes.c_void_p(0x1008)) == -2         # x not 16-byte aligned
    t = lambda R=4, C=4, e=2, w=A, o=A: lib.transpose_weights(R, C, e, w, o, None)
    assert t(e=3) == -3 and t(R=0) == -2 and t(R=1 << 23) == -2 and t(w=None) == -1
