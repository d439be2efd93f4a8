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
    "PaDims", "PagedAttnError", "KV_FP16", "KV_FP8_E4M3FN", "library_path",
    "load", "dims", "kv_append", "paged_decode_attn", "paged_decode_attn_splitk",
    "paged_decode_attn_splitk_reduce", "paged_decode_attn_splitk_merged",
    "paged_decode_step",
    "splitk_workspace", "splitk_workspace_size",
    "suggest_splits", "step_fuses_append", "status_string", "version",
]

KV_FP16 = 0
KV_FP8_E4M3FN = 1
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
        "paged_decode_attn_suggest_splits": (I, [D, I]),
        "paged_decode_step_fuses_append": (I, [D]),
        "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
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
    if pages.dtype == torch.float16:
        return KV_FP16
    if pages.dtype in (torch.uint8, torch.float8_e4m3fn):
        return KV_FP8_E4M3FN
    raise TypeError(f"unsupported page dtype {pages.dtype}")


def _need(t, name, dtype=None, ndim=None, cuda=True):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if cuda and t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, has {t.dim()}")


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
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, torch.float16, 3)
    _need(k_pages, "k_pages", ndim=4); _need(v_pages, "v_pages", ndim=4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(positions, "positions", torch.int32, 1)
    if seq_ids is not None:
        _need(seq_ids, "seq_ids", torch.int32, 1)
    T = k_new.shape[0]
    B = block_table.shape[0] if num_seqs is None else num_seqs
    d = dims(B, k_pages.shape[1], k_pages, block_table)
    if k_new.shape != (T, d.num_kv_heads, d.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [T, Hkv, d]")
    if positions.shape[0] != T or (seq_ids is not None and seq_ids.shape[0] != T):
        raise ValueError("positions/seq_ids must have T entries")
    rc = load().kv_append(ctypes.byref(d), T, _ptr(k_new), _ptr(v_new),
                          _ptr(seq_ids), _ptr(positions), _ptr(block_table),
                          _ptr(k_scale), _ptr(v_scale), _ptr(k_pages),
                          _ptr(v_pages), _stream(stream))
    _check("kv_append", rc)


def _attn_checks(q, k_pages, v_pages, block_table, context_lens, k_scale, v_scale):
    _need(q, "q", torch.float16, 3)
    _need(k_pages, "k_pages", ndim=4); _need(v_pages, "v_pages", ndim=4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    B, Hq, dq = q.shape
    d = dims(B, Hq, k_pages, block_table)
    P, Hkv, bs, hd = k_pages.shape
    if v_pages.shape != k_pages.shape or v_pages.dtype != k_pages.dtype:
        raise ValueError("v_pages must match k_pages' shape [P, Hkv, bs, d] and dtype")
    if dq != hd or block_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("inconsistent q / block_table / context_lens shapes")
    if d.kv_dtype == KV_FP8_E4M3FN:
        _need(k_scale, "k_scale", torch.float32, 1); _need(v_scale, "v_scale", torch.float32, 1)
    return d


def paged_decode_attn(q, k_pages, v_pages, block_table, context_lens, scale,
                      k_scale=None, v_scale=None, out=None, stream=None):
    """Single-pass decode attention; returns out [B, Hq, d] fp16."""
    d = _attn_checks(q, k_pages, v_pages, block_table, context_lens, k_scale, v_scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float16, 3)
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
    """Split pass; returns the workspace (uint8 tensor holding o then lse)."""
    d = _attn_checks(q, k_pages, v_pages, block_table, context_lens, k_scale, v_scale)
    if workspace is None:
        workspace = splitk_workspace(q, k_pages, block_table, num_splits)
    _need(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    rc = load().paged_decode_attn_splitk(ctypes.byref(d), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                         _ptr(block_table), _ptr(context_lens), float(scale),
                                         _ptr(k_scale), _ptr(v_scale), int(num_splits),
                                         _ptr(workspace), nbytes, _stream(stream))
    _check("paged_decode_attn_splitk", rc)
    return workspace


def paged_decode_attn_splitk_reduce(q_like, k_pages, block_table, context_lens,
                                    num_splits, workspace, out=None, stream=None):
    """Merge pass; q_like gives [B, Hq, d]. Returns out fp16."""
    B, Hq, _ = q_like.shape
    d = dims(B, Hq, k_pages, block_table)
    _need(context_lens, "context_lens", torch.int32, 1)
    if out is None:
        out = torch.empty(q_like.shape, dtype=torch.float16, device=q_like.device)
    _need(out, "out", torch.float16, 3)
    nbytes = workspace.numel() * workspace.element_size()
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
    d = _attn_checks(q, k_pages, v_pages, block_table, context_lens, k_scale, v_scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float16, 3)
    _need(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    rc = load().paged_decode_attn_splitk_merged(
        ctypes.byref(d), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
        _ptr(context_lens), float(scale), _ptr(k_scale), _ptr(v_scale), int(num_splits),
        _ptr(workspace), nbytes, _ptr(out), _stream(stream))
    _check("paged_decode_attn_splitk_merged", rc)
    return out


def paged_decode_step(q, k_new, v_new, positions, k_pages, v_pages, block_table,
                      context_lens, scale, num_splits, workspace, k_scale=None,
                      v_scale=None, out=None, stream=None):
    """kv_append of each sequence's new token (k_new/v_new [B, Hkv, d] fp16 at
    positions [B]) and the merged split attention, fused; returns out."""
    d = _attn_checks(q, k_pages, v_pages, block_table, context_lens, k_scale, v_scale)
    _need(k_new, "k_new", torch.float16, 3)
    _need(v_new, "v_new", torch.float16, 3)
    _need(positions, "positions", torch.int32, 1)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float16, 3)
    _need(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    rc = load().paged_decode_step(
        ctypes.byref(d), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(positions),
        _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(context_lens),
        float(scale), _ptr(k_scale), _ptr(v_scale), int(num_splits),
        _ptr(workspace), nbytes, _ptr(out), _stream(stream))
    _check("paged_decode_step", rc)
    return out


def split_views(workspace, B, Hq, Hkv, S, D):
    """(o [B,Hq,S,D] f32, lse [B,Hq,S] f32, count [B,Hkv] i32) views of a workspace."""
    n = B * Hq * S
    f = workspace[:(n * D + n) * 4].view(torch.float32)
    c = workspace[(n * D + n) * 4:(n * D + n) * 4 + B * Hkv * 4].view(torch.int32)
    return f[:n * D].view(B, Hq, S, D), f[n * D:].view(B, Hq, S), c.view(B, Hkv)


def suggest_splits(d: PaDims, max_context_len: int) -> int:
    return int(load().paged_decode_attn_suggest_splits(ctypes.byref(d), int(max_context_len)))


def step_fuses_append(d: PaDims) -> bool:
    """Whether paged_decode_step appends inside the attention kernel for d."""
    rc = int(load().paged_decode_step_fuses_append(ctypes.byref(d)))
    _check("paged_decode_step_fuses_append", min(rc, 0))
    return rc == 1
