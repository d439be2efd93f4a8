"""Paged KV cache: append (scatter) and block-table gather (oracle, tests only).

Source: "优化" on tiny-llm, roadmap table, row 分页 KV — K/V are kept in
fixed-size pages found through a per-sequence block table, written by a
scatter and read by a gather; "TensorRT对Multi-Query Attention的专项优化支持",
KV-cache paragraph — long sequences are cut into fixed-length pages. The
pages give no layout; the library's header fixes it and this file follows it:

  k_pages  [P, Hkv, bs, d]   token-major inside a (page, head) tile
  v_pages  [P, Hkv, d, bs]   dimension-major inside a (page, head) tile
  token t of sequence b lives in page block_table[b, t // bs], slot t % bs.

Element type is float16 or the uint8 code of fp8 e4m3fn; for fp8 each kv head
h has its own float32 scale for K and for V (value = decode(code) * scale).
"""
from __future__ import annotations

import numpy as np

from . import fp8


def empty_pools(num_pages, num_kv_heads, block_size, head_dim, kv_dtype):
    """Pools filled with NaN (fp16 0x7E00, fp8 code 0x7F): never-written slots."""
    if kv_dtype == "fp16":
        k = np.full((num_pages, num_kv_heads, block_size, head_dim), np.nan,
                    np.float16)
        v = np.full((num_pages, num_kv_heads, head_dim, block_size), np.nan,
                    np.float16)
    elif kv_dtype == "fp8_e4m3fn":
        k = np.full((num_pages, num_kv_heads, block_size, head_dim),
                    fp8.NAN_CODE, np.uint8)
        v = np.full((num_pages, num_kv_heads, head_dim, block_size),
                    fp8.NAN_CODE, np.uint8)
    else:
        raise ValueError(kv_dtype)
    return k, v


def kv_append(k_pages, v_pages, block_table, seq_ids, positions, k_new, v_new,
              kv_dtype="fp16", k_scale=None, v_scale=None):
    """Write token i's K/V rows into (block_table[seq_ids[i], pos // bs], pos % bs).

    k_new, v_new: float16 [T, Hkv, d]; seq_ids, positions: int [T].
    fp16 pools receive the bits unchanged; fp8 pools receive
    fp8.quantize(x, scale[h]) per head. Returns new pools (inputs untouched).
    """
    k_pages = k_pages.copy()
    v_pages = v_pages.copy()
    bs = k_pages.shape[2]
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
        kw = fp8.quantize(k_new, ks)
        vw = fp8.quantize(v_new, vs)
    # k_pages[page, :, slot, :] has shape [T, Hkv, d]; so does the V view
    # v_pages[page, :, :, slot] ([T, Hkv, d] after advanced indexing).
    k_pages[page, :, slot, :] = kw
    v_pages[page, :, :, slot] = vw
    return k_pages, v_pages


def gather(k_pages, v_pages, block_table, b, h, L, kv_dtype="fp16",
           k_scale=None, v_scale=None):
    """Logical K, V of sequence b, kv head h, tokens 0..L-1, as float64 [L, d]."""
    bs = k_pages.shape[2]
    t = np.arange(L)
    page = np.asarray(block_table, np.int64)[b, t // bs]
    slot = t % bs
    k = k_pages[page, h, slot, :]
    v = v_pages[page, h, :, slot]          # [L, d]
    if kv_dtype == "fp16":
        return k.astype(np.float64), v.astype(np.float64)
    return (fp8.decode(k) * np.float64(k_scale[h]),
            fp8.decode(v) * np.float64(v_scale[h]))
