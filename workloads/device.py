"""Device copies of a seeded workload for the GPU library (tests, benchmark).

The pools start as never-written markers (fp16 NaN 0x7E00, fp8 NaN code 0x7F,
int8 code -128, which no append produces) and are filled by the
library's own kv_append, one call per group of sequences, with the tokens the
generator draws; nothing here computes any part of attention or of the cache
append. Pass `upto_last=True` to leave each sequence's final token out of the
pool, as it stands before a decode step appends it.
"""
from __future__ import annotations

import numpy as np
import torch

from . import Workload


def _nan_pools(w: Workload, device):
    cfg = w.cfg
    shape_k = shape_v = (w.num_pages, cfg.num_kv_heads, cfg.block_size, cfg.head_dim)
    if cfg.kv_dtype == "fp16":
        k = torch.full(shape_k, float("nan"), dtype=torch.float16, device=device)
        v = torch.full(shape_v, float("nan"), dtype=torch.float16, device=device)
    elif cfg.kv_dtype == "int8":
        k = torch.full(shape_k, -128, dtype=torch.int8, device=device)
        v = torch.full(shape_v, -128, dtype=torch.int8, device=device)
    else:
        k = torch.full(shape_k, 0x7F, dtype=torch.uint8, device=device)
        v = torch.full(shape_v, 0x7F, dtype=torch.uint8, device=device)
    return k, v


class DeviceWorkload:
    """Tensors of one workload on the GPU.

    q [B,Hq,d] fp16, k_pages/v_pages, block_table [B,max_blocks] int32,
    context_lens [B] int32, k_scale/v_scale [Hkv] fp32 (None for fp16),
    new_k/new_v [B,Hkv,d] fp16 and positions [B] int32 for one decode-step
    append, scale (float).
    """

    def __init__(self, w: Workload, device="cuda", upto_last=False, seqs=None,
                 tokens_per_call=1 << 18):
        from paged_mqa_gqa_amd import kv_append   # the library under test
        cfg = w.cfg
        self.w = w
        self.cfg = cfg
        self.scale = w.scale
        self.q = torch.from_numpy(w.q).to(device)
        self.block_table = torch.from_numpy(w.block_table).to(device)
        self.context_lens = torch.from_numpy(w.context_lens).to(device)
        ks, vs = w.kv_scales()
        if cfg.kv_dtype == "fp16":
            self.k_scale = self.v_scale = None
        else:
            self.k_scale = torch.from_numpy(ks).to(device)
            self.v_scale = torch.from_numpy(vs).to(device)
        self.k_pages, self.v_pages = _nan_pools(w, device)
        seqs = list(range(cfg.num_seqs)) if seqs is None else list(seqs)
        group, count = [], 0
        for b in seqs + [None]:
            if b is not None:
                n = int(w.context_lens[b]) - (1 if upto_last else 0)
                if n > 0:
                    group.append(b)
                    count += n
            if group and (b is None or count >= tokens_per_call):
                K, V, sid, pos = w.tokens(group, upto_last)
                kv_append(torch.from_numpy(K).to(device), torch.from_numpy(V).to(device),
                          self.k_pages, self.v_pages, self.block_table,
                          torch.from_numpy(pos).to(device),
                          seq_ids=torch.from_numpy(sid).to(device),
                          k_scale=self.k_scale, v_scale=self.v_scale)
                group, count = [], 0
        nk, nv, npos = w.new_tokens()
        self.new_k = torch.from_numpy(nk).to(device)
        self.new_v = torch.from_numpy(nv).to(device)
        self.positions = torch.from_numpy(npos).to(device)

    def kv_bytes(self) -> int:
        return self.w.kv_bytes()


def remap_pages(w: Workload, seqs):
    """A copy of `w` restricted to `seqs`, with their pages renumbered 0..n-1.

    Attention does not depend on physical page ids, so the oracle can check
    sampled sequences of a large workload on a compact pool. The returned
    workload shares the generator streams (same tokens) and keeps the first
    poison page id for unused entries.
    """
    import copy
    sub = copy.copy(w)
    cfg = w.cfg
    bs = cfg.block_size
    seqs = list(seqs)
    nblk = [-(-int(w.context_lens[b]) // bs) for b in seqs]
    n = sum(nblk)
    bt = np.full_like(w.block_table, n)
    off = 0
    for b, k in zip(seqs, nblk):
        bt[b, :k] = np.arange(off, off + k)
        off += k
    sub.block_table = bt
    sub.num_pages = n + 1
    sub.poison_pages = np.array([n])
    return sub
