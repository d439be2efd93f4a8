"""Python binding of libpagedattn, the gfx950 paged MQA/GQA decode library.

Argument marshalling only: shapes and dtypes of torch tensors are checked,
their device pointers and the current HIP stream are handed to the C ABI
declared in include/paged_attn.h, and a negative status becomes an
exception. Every step of the computation runs in the library's kernels.

The library is loaded after torch so that it binds to the HIP runtime torch
already loaded (both carry the soname libamdhip64.so.7). If the library is
not built, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "PaDims", "PagedAttnError", "KV_FP16", "KV_FP8_E4M3FN", "KV_INT8", "library_path",
    "load", "dims", "kv_append", "paged_decode_attn", "paged_decode_attn_splitk",
    "paged_decode_attn_splitk_reduce", "paged_decode_attn_splitk_merged",
    "paged_decode_step", "paged_decode_step_static", "STATIC_SCRATCH_BYTES",
    "paged_decode_advance",
    "splitk_workspace", "splitk_workspace_size",
    "suggest_splits", "step_fuses_append", "status_string", "version",
    "KvPageManager", "kv_bytes_per_sequence", "kv_pool_bytes", "kv_pages_for_budget",
    "W_FP16", "W_INT8", "gemm_m1_transposed", "transpose_weights",
]

KV_FP16 = 0
KV_FP8_E4M3FN = 1
KV_INT8 = 2
W_FP16 = 0          # decode projection weights (include/decode_gemm.h)
W_INT8 = 1
# int32 arrival counters at the start of every split workspace
# (PA_WORKSPACE_SEM_SLOTS in include/paged_attn.h)
WORKSPACE_SEM_SLOTS = 2048
# bytes of the library's own device scratch (PA_STATIC_SCRATCH_BYTES)
STATIC_SCRATCH_BYTES = 32 << 20
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class PagedAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


class PaDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size",
        "num_pages", "max_blocks_per_seq", "kv_dtype")]

    def __repr__(self):
        return "PaDims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


def library_path() -> str:
    return os.path.join(_HERE, "lib", "libpagedattn.so")


def load():
    """Load the shared library (once). Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m paged_mqa_gqa_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, Z, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    D = ctypes.POINTER(PaDims)
    sig = {
        "kv_append": (I, [D, I, P, P, P, P, P, P, P, P, P, P]),
        "paged_decode_attn": (I, [D, P, P, P, P, P, F, P, P, P, P]),
        "paged_decode_attn_splitk_workspace_size": (Z, [D, I]),
        "paged_decode_attn_splitk": (I, [D, P, P, P, P, P, F, P, P, I, P, Z, P]),
        "paged_decode_attn_splitk_reduce": (I, [D, P, I, P, Z, P, P]),
        "paged_decode_attn_splitk_merged": (I, [D, P, P, P, P, P, F, P, P, I, P, Z, P, P]),
        "paged_decode_step": (I, [D, P, P, P, P, P, P, P, P, F, P, P, I, P, Z, P, P]),
        "paged_decode_step_static": (I, [D, P, P, P, P, P, P, P, P, F, P, P, I, P, P]),
        "paged_decode_advance": (I, [D, P, P, P]),
        "paged_decode_attn_suggest_splits": (I, [D, I]),
        "paged_decode_step_fuses_append": (I, [D]),
        "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        # decode projection (include/decode_gemm.h)
        "gemm_m1_transposed": (I, [I, I, I, I, I, P, P, P, P, P]),
        "transpose_weights": (I, [I, I, I, P, P, P]),
        # page manager (include/paged_kv_manager.h)
        "pa_kv_elem_bytes": (I, [I]),
        "pa_kv_bytes_per_sequence": (ctypes.c_int64, [I, I, I, I, I]),
        "pa_kv_pool_bytes": (ctypes.c_int64, [I, I, I, I, I]),
        "pa_kv_pages_for_budget": (ctypes.c_int64, [ctypes.c_int64, I, I, I, I, I]),
        "pa_kvm_create": (P, [I, I, I, I]),
        "pa_kvm_destroy": (None, [P]),
        "pa_kvm_free_pages": (I, [P]),
        "pa_kvm_live_slots": (I, [P]),
        "pa_kvm_length": (I, [P, I]),
        "pa_kvm_pages_held": (I, [P, I]),
        "pa_kvm_admit": (I, [P, I]),
        "pa_kvm_release": (I, [P, I]),
        "pa_kvm_reserve_ahead": (I, [P, I]),
        "pa_kvm_plan_step": (I, [P, P, P, P]),
        "pa_kvm_commit_steps": (I, [P, I]),
        "pa_kvm_block_table": (I, [P, P]),
        "pa_kvm_batch_state": (I, [P, P, P]),
        "pa_version": (I, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load().pa_status_string(int(status)).decode()


def version() -> int:
    return int(load().pa_version())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _kv_dtype(pages: torch.Tensor) -> int:
    """Cache kind from the pool's element type: float16 values, uint8 /
    float8_e4m3fn for fp8 e4m3fn codes, int8 for symmetric int8 codes."""
    if pages.dtype == torch.float16:
        return KV_FP16
    if pages.dtype in (torch.uint8, torch.float8_e4m3fn):
        return KV_FP8_E4M3FN
    if pages.dtype == torch.int8:
        return KV_INT8
    raise TypeError(f"unsupported page dtype {pages.dtype}")


def _need(t, name, dtype=None, ndim=None, shape=None):
    """Check one tensor argument before its pointer crosses the ABI: present,
    contiguous, of the given dtype, rank and exact shape. A mismatch raises
    here, never inside a kernel. (Devices are checked by _on_gpu once every
    shape is known to be right.)"""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, has {t.dim()}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _on_gpu(**tensors):
    """Every given tensor (None entries skipped) on the same GPU."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor, is on {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _scales(d, k_scale, v_scale):
    """Per-kv-head fp32 scales: required for one-byte caches, else ignored."""
    if d.kv_dtype == KV_FP16:
        return None, None
    _need(k_scale, "k_scale", torch.float32, 1, shape=(d.num_kv_heads,))
    _need(v_scale, "v_scale", torch.float32, 1, shape=(d.num_kv_heads,))
    return k_scale, v_scale


def dims(num_seqs, num_q_heads, k_pages: torch.Tensor, block_table: torch.Tensor) -> PaDims:
    """PaDims from a pool allocation [P, Hkv, bs, d] and block table [B, max_blocks].

    The bs * d values of one (page, head) are stored in the library's page
    order (see include/paged_attn.h), not as a [bs, d] matrix."""
    P, Hkv, bs, d = k_pages.shape
    return PaDims(num_seqs, num_q_heads, Hkv, d, bs, P, block_table.shape[1],
                  _kv_dtype(k_pages))


def _check(fn, rc):
    if rc != 0:
        raise PagedAttnError(fn, rc)


def kv_append(k_new, v_new, k_pages, v_pages, block_table, positions,
              seq_ids=None, k_scale=None, v_scale=None, num_seqs=None,
              stream=None):
    """Scatter k_new / v_new [T, Hkv, d] fp16 into the pages (see kv_append in the header)."""
    _need(k_pages, "k_pages", ndim=4)
    _need(v_pages, "v_pages", k_pages.dtype, 4, shape=k_pages.shape)
    _need(block_table, "block_table", torch.int32, 2)
    _need(k_new, "k_new", torch.float16, 3)
    T = k_new.shape[0]
    B = block_table.shape[0] if num_seqs is None else num_seqs
    if B > block_table.shape[0]:
        raise ValueError("num_seqs exceeds the block table's rows")
    d = dims(B, k_pages.shape[1], k_pages, block_table)
    _need(k_new, "k_new", shape=(T, d.num_kv_heads, d.head_dim))
    _need(v_new, "v_new", torch.float16, 3, shape=k_new.shape)
    _need(positions, "positions", torch.int32, 1, shape=(T,))
    if seq_ids is not None:
        _need(seq_ids, "seq_ids", torch.int32, 1, shape=(T,))
    k_scale, v_scale = _scales(d, k_scale, v_scale)
    _on_gpu(k_new=k_new, v_new=v_new, k_pages=k_pages, v_pages=v_pages,
            block_table=block_table, positions=positions, seq_ids=seq_ids,
            k_scale=k_scale, v_scale=v_scale)
    rc = load().kv_append(ctypes.byref(d), T, _ptr(k_new), _ptr(v_new),
                          _ptr(seq_ids), _ptr(positions), _ptr(block_table),
                          _ptr(k_scale), _ptr(v_scale), _ptr(k_pages),
                          _ptr(v_pages), _stream(stream))
    _check("kv_append", rc)


def _attn_checks(q, k_pages, v_pages, block_table, context_lens, k_scale, v_scale):
    """Shapes and dtypes of an attention call's inputs; returns (dims,
    k_scale, v_scale) with the scales None for an fp16 cache."""
    _need(q, "q", torch.float16, 3)
    _need(k_pages, "k_pages", ndim=4)
    _need(v_pages, "v_pages", k_pages.dtype, 4, shape=k_pages.shape)
    B, Hq, dq = q.shape
    _need(block_table, "block_table", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1, shape=(B,))
    d = dims(B, Hq, k_pages, block_table)
    if dq != d.head_dim:
        raise ValueError(f"q has head_dim {dq}, the pages {d.head_dim}")
    if block_table.shape[0] != B:
        raise ValueError(f"block_table has {block_table.shape[0]} rows, q {B} sequences")
    ks, vs = _scales(d, k_scale, v_scale)
    return d, ks, vs


def _out(q, out):
    """The fp16 output [B, Hq, d]: allocated like q, or checked against q."""
    if out is None:
        return torch.empty_like(q)
    _need(out, "out", torch.float16, 3, shape=q.shape)
    return out


def _workspace_bytes(workspace):
    _need(workspace, "workspace")
    return workspace.numel() * workspace.element_size()


def paged_decode_attn(q, k_pages, v_pages, block_table, context_lens, scale,
                      k_scale=None, v_scale=None, out=None, stream=None):
    """Single-pass decode attention; returns out [B, Hq, d] fp16."""
    d, k_scale, v_scale = _attn_checks(q, k_pages, v_pages, block_table, context_lens,
                                       k_scale, v_scale)
    out = _out(q, out)
    _on_gpu(q=q, k_pages=k_pages, v_pages=v_pages, block_table=block_table,
            context_lens=context_lens, k_scale=k_scale, v_scale=v_scale, out=out)
    rc = load().paged_decode_attn(ctypes.byref(d), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                  _ptr(block_table), _ptr(context_lens), float(scale),
                                  _ptr(k_scale), _ptr(v_scale), _ptr(out), _stream(stream))
    _check("paged_decode_attn", rc)
    return out


def splitk_workspace_size(d: PaDims, num_splits: int) -> int:
    return int(load().paged_decode_attn_splitk_workspace_size(ctypes.byref(d), num_splits))


def splitk_workspace(q, k_pages, block_table, num_splits):
    """A zero-filled workspace for the split calls (uint8 device tensor)."""
    d = dims(q.shape[0], q.shape[1], k_pages, block_table)
    return torch.zeros(max(splitk_workspace_size(d, num_splits), 1), dtype=torch.uint8,
                       device=q.device)


def paged_decode_attn_splitk(q, k_pages, v_pages, block_table, context_lens, scale,
                             num_splits, k_scale=None, v_scale=None, workspace=None,
                             stream=None):
    """Split pass; returns the workspace (uint8 tensor; see split_views)."""
    d, k_scale, v_scale = _attn_checks(q, k_pages, v_pages, block_table, context_lens,
                                       k_scale, v_scale)
    if workspace is None:
        workspace = splitk_workspace(q, k_pages, block_table, num_splits)
    nbytes = _workspace_bytes(workspace)
    _on_gpu(q=q, k_pages=k_pages, v_pages=v_pages, block_table=block_table,
            context_lens=context_lens, k_scale=k_scale, v_scale=v_scale,
            workspace=workspace)
    rc = load().paged_decode_attn_splitk(ctypes.byref(d), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                         _ptr(block_table), _ptr(context_lens), float(scale),
                                         _ptr(k_scale), _ptr(v_scale), int(num_splits),
                                         _ptr(workspace), nbytes, _stream(stream))
    _check("paged_decode_attn_splitk", rc)
    return workspace


def paged_decode_attn_splitk_reduce(q_like, k_pages, block_table, context_lens,
                                    num_splits, workspace, out=None, stream=None):
    """Merge pass; q_like gives [B, Hq, d]. Returns out fp16."""
    _need(q_like, "q_like", ndim=3)
    B, Hq, _ = q_like.shape
    _need(k_pages, "k_pages", ndim=4)
    _need(block_table, "block_table", torch.int32, 2)
    d = dims(B, Hq, k_pages, block_table)
    _need(context_lens, "context_lens", torch.int32, 1, shape=(B,))
    if out is None:
        out = torch.empty(q_like.shape, dtype=torch.float16, device=q_like.device)
    _need(out, "out", torch.float16, 3, shape=q_like.shape)
    nbytes = _workspace_bytes(workspace)
    _on_gpu(context_lens=context_lens, workspace=workspace, out=out)
    rc = load().paged_decode_attn_splitk_reduce(ctypes.byref(d), _ptr(context_lens),
                                                int(num_splits), _ptr(workspace), nbytes,
                                                _ptr(out), _stream(stream))
    _check("paged_decode_attn_splitk_reduce", rc)
    return out


def paged_decode_attn_splitk_merged(q, k_pages, v_pages, block_table, context_lens, scale,
                                    num_splits, workspace, k_scale=None, v_scale=None,
                                    out=None, stream=None):
    """Split pass with the merge in the same launch; returns out [B, Hq, d] fp16.

    `workspace` must come from splitk_workspace() (its counters start at zero)
    and must not be shared by two merged calls running at the same time."""
    d, k_scale, v_scale = _attn_checks(q, k_pages, v_pages, block_table, context_lens,
                                       k_scale, v_scale)
    out = _out(q, out)
    nbytes = _workspace_bytes(workspace)
    _on_gpu(q=q, k_pages=k_pages, v_pages=v_pages, block_table=block_table,
            context_lens=context_lens, k_scale=k_scale, v_scale=v_scale,
            workspace=workspace, out=out)
    rc = load().paged_decode_attn_splitk_merged(
        ctypes.byref(d), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
        _ptr(context_lens), float(scale), _ptr(k_scale), _ptr(v_scale), int(num_splits),
        _ptr(workspace), nbytes, _ptr(out), _stream(stream))
    _check("paged_decode_attn_splitk_merged", rc)
    return out


def _step_checks(q, k_new, v_new, positions, k_pages, v_pages, block_table,
                 context_lens, k_scale, v_scale, out):
    d, k_scale, v_scale = _attn_checks(q, k_pages, v_pages, block_table, context_lens,
                                       k_scale, v_scale)
    row = (d.num_seqs, d.num_kv_heads, d.head_dim)
    _need(k_new, "k_new", torch.float16, 3, shape=row)
    _need(v_new, "v_new", torch.float16, 3, shape=row)
    _need(positions, "positions", torch.int32, 1, shape=(d.num_seqs,))
    out = _out(q, out)
    return d, k_scale, v_scale, out


def paged_decode_step(q, k_new, v_new, positions, k_pages, v_pages, block_table,
                      context_lens, scale, num_splits, workspace, k_scale=None,
                      v_scale=None, out=None, stream=None):
    """kv_append of each sequence's new token (k_new/v_new [B, Hkv, d] fp16 at
    positions [B]) and the merged split attention, fused; returns out."""
    d, k_scale, v_scale, out = _step_checks(q, k_new, v_new, positions, k_pages, v_pages,
                                            block_table, context_lens, k_scale, v_scale, out)
    nbytes = _workspace_bytes(workspace)
    _on_gpu(q=q, k_new=k_new, v_new=v_new, positions=positions, k_pages=k_pages,
            v_pages=v_pages, block_table=block_table, context_lens=context_lens,
            k_scale=k_scale, v_scale=v_scale, workspace=workspace, out=out)
    rc = load().paged_decode_step(
        ctypes.byref(d), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(positions),
        _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(context_lens),
        float(scale), _ptr(k_scale), _ptr(v_scale), int(num_splits),
        _ptr(workspace), nbytes, _ptr(out), _stream(stream))
    _check("paged_decode_step", rc)
    return out


def paged_decode_advance(context_lens, positions, k_pages, block_table, stream=None):
    """One decode step on, on the device: for every live slot (position >= 0)
    positions and context_lens grow by one (see paged_decode_advance in the
    header). Capturable after paged_decode_step in one graph."""
    _need(context_lens, "context_lens", torch.int32, 1)
    B = context_lens.shape[0]
    _need(positions, "positions", torch.int32, 1, shape=(B,))
    _need(k_pages, "k_pages", ndim=4)
    _need(block_table, "block_table", torch.int32, 2)
    d = dims(B, k_pages.shape[1], k_pages, block_table)
    _on_gpu(context_lens=context_lens, positions=positions)
    rc = load().paged_decode_advance(ctypes.byref(d), _ptr(context_lens), _ptr(positions),
                                     _stream(stream))
    _check("paged_decode_advance", rc)


def paged_decode_step_static(q, k_new, v_new, positions, k_pages, v_pages, block_table,
                             context_lens, scale, num_splits, k_scale=None, v_scale=None,
                             out=None, stream=None):
    """paged_decode_step without a workspace argument: the library's own
    static device scratch (STATIC_SCRATCH_BYTES per GPU) holds the split
    partials, so the call allocates nothing. Calls on one GPU share that
    scratch and must be ordered on one stream. Returns out."""
    d, k_scale, v_scale, out = _step_checks(q, k_new, v_new, positions, k_pages, v_pages,
                                            block_table, context_lens, k_scale, v_scale, out)
    _on_gpu(q=q, k_new=k_new, v_new=v_new, positions=positions, k_pages=k_pages,
            v_pages=v_pages, block_table=block_table, context_lens=context_lens,
            k_scale=k_scale, v_scale=v_scale, out=out)
    rc = load().paged_decode_step_static(
        ctypes.byref(d), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(positions),
        _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(context_lens),
        float(scale), _ptr(k_scale), _ptr(v_scale), int(num_splits), _ptr(out),
        _stream(stream))
    _check("paged_decode_step_static", rc)
    return out


def gemm_m1_transposed(x, wt, scales_t=None, group_size=128, out=None, stream=None):
    """y [M, N] fp16 = x [M, K] fp16 . W for 1 <= M <= 4, with W given
    transposed as wt [N, K] (fp16, or int8 codes with scales_t [N, K /
    group_size] fp32). See gemm_m1_transposed in include/decode_gemm.h."""
    _need(x, "x", torch.float16, 2)
    M, K = x.shape
    _need(wt, "wt", (torch.float16, torch.int8), 2)
    N = wt.shape[0]
    _need(wt, "wt", shape=(N, K))
    int8 = wt.dtype == torch.int8
    if int8:
        if group_size < 16 or K % group_size:
            raise ValueError(f"group_size {group_size} must be a multiple of 16 dividing K={K}")
        _need(scales_t, "scales_t", torch.float32, 2, shape=(N, K // group_size))
    else:
        scales_t = None
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _need(out, "out", torch.float16, 2, shape=(M, N))
    _on_gpu(x=x, wt=wt, scales_t=scales_t, out=out)
    rc = load().gemm_m1_transposed(M, N, K, W_INT8 if int8 else W_FP16,
                                   group_size if int8 else 0, _ptr(x), _ptr(wt),
                                   _ptr(scales_t), _ptr(out), _stream(stream))
    _check("gemm_m1_transposed", rc)
    return out


def transpose_weights(w, out=None, stream=None):
    """The [cols, rows] copy of a 2-d tensor w [rows, cols] (elements of 1, 2
    or 4 bytes), built on the device: the load-time transposed weight (or
    scales) for gemm_m1_transposed."""
    _need(w, "w", ndim=2)
    R, C = w.shape
    if out is None:
        out = torch.empty((C, R), dtype=w.dtype, device=w.device)
    _need(out, "out", w.dtype, 2, shape=(C, R))
    _on_gpu(w=w, out=out)
    rc = load().transpose_weights(R, C, w.element_size(), _ptr(w), _ptr(out), _stream(stream))
    _check("transpose_weights", rc)
    return out


def split_views(workspace, B, Hq, Hkv, S, D):
    """(o [B,Hq,S,D] f32, lse [B,Hq,S] f32, count [B,Hkv] i32) views of a
    workspace (uint8 tensor), in the header's layout: the arrival counters
    first (sem_view), then o, lse and count."""
    n = B * Hq * S
    base = WORKSPACE_SEM_SLOTS * 4
    f = workspace[base:base + (n * D + n) * 4].view(torch.float32)
    c = workspace[base + (n * D + n) * 4:base + (n * D + n) * 4 + B * Hkv * 4].view(torch.int32)
    return f[:n * D].view(B, Hq, S, D), f[n * D:].view(B, Hq, S), c.view(B, Hkv)


def sem_view(workspace):
    """The merged call's arrival counters (int32 [WORKSPACE_SEM_SLOTS]):
    zero between calls."""
    return workspace[:WORKSPACE_SEM_SLOTS * 4].view(torch.int32)


def suggest_splits(d: PaDims, max_context_len: int) -> int:
    return int(load().paged_decode_attn_suggest_splits(ctypes.byref(d), int(max_context_len)))


def step_fuses_append(d: PaDims) -> bool:
    """Whether paged_decode_step appends inside the attention kernel for d."""
    rc = int(load().paged_decode_step_fuses_append(ctypes.byref(d)))
    _check("paged_decode_step_fuses_append", min(rc, 0))
    return rc == 1


from .kv_manager import (KvPageManager, kv_bytes_per_sequence,  # noqa: E402
                         kv_pages_for_budget, kv_pool_bytes)
