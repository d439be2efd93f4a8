"""Paged KV cache: append (scatter) and block-table gather (oracle, tests only).

Source: "优化" on tiny-llm, roadmap table, row 分页 KV — K/V are kept in
fixed-size pages found through a per-sequence block table, written by a
scatter and read by a gather; "TensorRT对Multi-Query Attention的专项优化支持",
KV-cache paragraph — long sequences are cut into fixed-length pages. The
pages give no layout; the library's header fixes it and this file follows it.

Pools are arrays [P, Hkv, bs, d] (the allocation shape); the bs * d
elements of one (page, head) tile are stored in the order below, in units
of 16-token blocks (blk = t // 16, r = t % 16; X = elements per 16 bytes:
8 for fp16, 16 for the one-byte codes; rho(r) = r with its bits 2 and 3 swapped):

  K element (t, i):  ((blk * (d / X) + i // X) * 16 + rho(r)) * X + i % X
  V element (t, i):  (((blk * (d / 16) + i // 16) * 2 + r // 8) * 16 + i % 16) * 8 + r % 8

Token t of sequence b lives in page block_table[b, t // bs], slot t % bs.
Element type is float16, the uint8 code of fp8 e4m3fn, or an int8 code; for
the one-byte types each kv head h has its own float32 scale for K and for V
(value = decode(code) * scale).
"""
from __future__ import annotations

import numpy as np

from . import fp8, int8

KV_DTYPES = ("fp16", "fp8_e4m3fn", "int8")


def chunk_elems(kv_dtype) -> int:
    """Elements per 16-byte chunk: 8 two-byte or 16 one-byte values."""
    return 8 if kv_dtype == "fp16" else 16


def row_order(r):
    """Storage row of slot r (0..15) inside a 16-token K block: the quads
    r = 4..7 and 8..11 trade places (bits 2 and 3 of r swapped)."""
    r = np.asarray(r)
    return (r & 3) | ((r & 4) << 1) | ((r & 8) >> 1)


def k_offset(t, i, d, X):
    """Element offset of K (slot t, dim i) inside a (page, head) tile."""
    t = np.asarray(t); i = np.asarray(i)
    return ((t // 16 * (d // X) + i // X) * 16 + row_order(t % 16)) * X + i % X


def v_offset(t, i, d):
    """Element offset of V (slot t, dim i) inside a (page, head) tile."""
    t = np.asarray(t); i = np.asarray(i)
    r = t % 16
    return (((t // 16 * (d // 16) + i // 16) * 2 + r // 8) * 16 + i % 16) * 8 + r % 8


def empty_pools(num_pages, num_kv_heads, block_size, head_dim, kv_dtype):
    """Pools whose every slot holds the never-written marker: NaN (fp16
    0x7E00, fp8 code 0x7F) or the int8 code -128 that no append produces."""
    shape = (num_pages, num_kv_heads, block_size, head_dim)
    if kv_dtype == "fp16":
        return np.full(shape, np.nan, np.float16), np.full(shape, np.nan, np.float16)
    if kv_dtype == "fp8_e4m3fn":
        return (np.full(shape, fp8.NAN_CODE, np.uint8),
                np.full(shape, fp8.NAN_CODE, np.uint8))
    if kv_dtype == "int8":
        return (np.full(shape, int8.POISON_CODE, np.int8),
                np.full(shape, int8.POISON_CODE, np.int8))
    raise ValueError(kv_dtype)


def _codec(kv_dtype):
    return {"fp8_e4m3fn": fp8, "int8": int8}[kv_dtype]


def kv_append(k_pages, v_pages, block_table, seq_ids, positions, k_new, v_new,
              kv_dtype="fp16", k_scale=None, v_scale=None, inplace=False):
    """Write token i's K/V rows into (block_table[seq_ids[i], pos // bs], pos % bs).

    k_new, v_new: float16 [T, Hkv, d]; seq_ids, positions: int [T].
    fp16 pools receive the bits unchanged; fp8 / int8 pools receive
    quantize(x, scale[h]) of that codec per head. Returns new pools (inputs
    untouched), or with inplace=True writes into the given pools (which must
    be contiguous) and returns them.
    """
    P, H, bs, d = k_pages.shape
    X = chunk_elems(kv_dtype)
    if inplace:
        assert k_pages.flags.c_contiguous and v_pages.flags.c_contiguous
        kf = k_pages.reshape(P, H, bs * d)
        vf = v_pages.reshape(P, H, bs * d)
    else:
        kf = k_pages.copy().reshape(P, H, bs * d)
        vf = v_pages.copy().reshape(P, H, bs * d)
    seq_ids = np.asarray(seq_ids, np.int64)
    positions = np.asarray(positions, np.int64)
    page = np.asarray(block_table, np.int64)[seq_ids, positions // bs]
    slot = positions % bs
    if kv_dtype == "fp16":
        kw = np.asarray(k_new, np.float16)
        vw = np.asarray(v_new, np.float16)
    else:
        ks = np.asarray(k_scale, np.float32)[None, :, None]
        vs = np.asarray(v_scale, np.float32)[None, :, None]
        kw = _codec(kv_dtype).quantize(k_new, ks)
        vw = _codec(kv_dtype).quantize(v_new, vs)
    dims = np.arange(d)
    ko = k_offset(slot[:, None], dims[None, :], d, X)         # [T, d]
    vo = v_offset(slot[:, None], dims[None, :], d)
    # kf[page, :, ko] -> [T, d, Hkv] (advanced indices first), so transpose
    kf[page[:, None], :, ko] = kw.transpose(0, 2, 1)
    vf[page[:, None], :, vo] = vw.transpose(0, 2, 1)
    return kf.reshape(P, H, bs, d), vf.reshape(P, H, bs, d)


def gather(k_pages, v_pages, block_table, b, h, L, kv_dtype="fp16",
           k_scale=None, v_scale=None):
    """Logical K, V of sequence b, kv head h, tokens 0..L-1, as float64 [L, d]."""
    P, H, bs, d = k_pages.shape
    X = chunk_elems(kv_dtype)
    t = np.arange(L)
    page = np.asarray(block_table, np.int64)[b, t // bs]
    slot = t % bs
    dims = np.arange(d)
    kf = k_pages.reshape(P, H, bs * d)
    vf = v_pages.reshape(P, H, bs * d)
    k = kf[page[:, None], h, k_offset(slot[:, None], dims[None, :], d, X)]   # [L, d]
    v = vf[page[:, None], h, v_offset(slot[:, None], dims[None, :], d)]
    if kv_dtype == "fp16":
        return k.astype(np.float64), v.astype(np.float64)
    c = _codec(kv_dtype)
    return (c.decode(k) * np.float64(k_scale[h]),
            c.decode(v) * np.float64(v_scale[h]))
