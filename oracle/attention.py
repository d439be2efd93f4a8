"""Single-token decode attention over a paged KV cache (oracle, tests only).

What is computed, for sequence b and query head j (fp64 throughout):

  G = Hq / Hkv, h = j // G          query heads j = hG..hG+G-1 share kv head h
  L = context_lens[b]               tokens 0..L-1 (the new token included)
  s_t = scale * sum_i q[b, j, i] * K[t, i]
  out[b, j, :] = sum_t exp(s_t - max s) V[t, :] / sum_t exp(s_t - max s)
  L = 0 gives out = 0.

Sources, by page title and section:
  * "TensorRT对Multi-Query Attention的专项优化支持": MHA formula (each head
    owns K_i, V_i) and MQA formula (one shared K, V); decode re-reads all
    cached K/V for every new token.
  * zyxy.net tag page "tensorrt", FMHA abstract: scores, softmax, weighted
    sum of values.
  * "优化" on tiny-llm, section 3: kv heads may be fewer than q heads (GQA).
    Readings taken where the pages are silent: contiguous groups (h = j // G),
    an explicit softmax scale argument, L = 0 returns zeros.

Split-K (the FlashDecoding row of the tiny-llm roadmap names long-context
decode attention without describing it; reading taken): split i of S covers
tokens [i*C, min((i+1)*C, L)) with C = bs * ceil(ceil(L / S) / bs), i.e.
page-aligned equal chunks. Each split yields its own normalised output o_i
and lse_i = m_i + ln(l_i) (natural log); an empty split has o_i = 0 and
lse_i = -inf. The merge is out = sum_i w_i o_i / sum_i w_i with
w_i = exp(lse_i - max_k lse_k), and 0 when every split is empty.
"""
from __future__ import annotations

import math

import numpy as np

from .paged import gather


def _group_scores(qg, k, scale):
    """scale * q . k for the G heads of a group: [G, d] x [L, d] -> [G, L]."""
    return scale * (qg @ k.T)


def decode(q, k_pages, v_pages, block_table, context_lens, scale,
           kv_dtype="fp16", k_scale=None, v_scale=None, seqs=None):
    """Decode attention output, float64 [B, Hq, d] (rows of skipped seqs = 0)."""
    q = np.asarray(q).astype(np.float64)
    B, Hq, d = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    assert G * Hkv == Hq
    out = np.zeros((B, Hq, d), np.float64)
    for b in (range(B) if seqs is None else seqs):
        L = int(context_lens[b])
        if L == 0:
            continue
        for h in range(Hkv):
            k, v = gather(k_pages, v_pages, block_table, b, h, L, kv_dtype,
                          k_scale, v_scale)
            s = _group_scores(q[b, h * G:(h + 1) * G], k, scale)   # [G, L]
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            out[b, h * G:(h + 1) * G] = (p @ v) / p.sum(axis=1, keepdims=True)
    return out


def split_bounds(L, num_splits, block_size):
    """Token ranges [start, end) of the num_splits page-aligned chunks."""
    L = int(L)
    chunk = -(-L // num_splits) if L > 0 else 0
    C = block_size * (-(-chunk // block_size))
    return [(min(i * C, L), min((i + 1) * C, L)) for i in range(num_splits)]


def decode_partials(q, k_pages, v_pages, block_table, context_lens, scale,
                    num_splits, kv_dtype="fp16", k_scale=None, v_scale=None,
                    seqs=None):
    """Per-split normalised outputs o [B, Hq, S, d] and lse [B, Hq, S]."""
    q = np.asarray(q).astype(np.float64)
    B, Hq, d = q.shape
    Hkv = k_pages.shape[1]
    bs = k_pages.shape[2]
    G = Hq // Hkv
    o = np.zeros((B, Hq, num_splits, d), np.float64)
    lse = np.full((B, Hq, num_splits), -np.inf, np.float64)
    for b in (range(B) if seqs is None else seqs):
        L = int(context_lens[b])
        if L == 0:
            continue
        for h in range(Hkv):
            k, v = gather(k_pages, v_pages, block_table, b, h, L, kv_dtype,
                          k_scale, v_scale)
            s = _group_scores(q[b, h * G:(h + 1) * G], k, scale)
            for i, (a, e) in enumerate(split_bounds(L, num_splits, bs)):
                if e <= a:
                    continue
                si = s[:, a:e]
                m = si.max(axis=1, keepdims=True)
                p = np.exp(si - m)
                l = p.sum(axis=1, keepdims=True)
                o[b, h * G:(h + 1) * G, i] = (p @ v[a:e]) / l
                lse[b, h * G:(h + 1) * G, i] = (m + np.log(l))[:, 0]
    return o, lse


def range_partial(q, k_pages, v_pages, block_table, b, h, start, end, scale,
                  kv_dtype="fp16", k_scale=None, v_scale=None):
    """Attention of the G q heads of kv group h of sequence b over the tokens
    [start, end) alone: their normalised output o [G, d] and
    lse [G] = ln sum_{start <= t < end} exp(s_t) (natural log); an empty
    range gives o = 0 and lse = -inf."""
    q = np.asarray(q).astype(np.float64)
    Hq, d = q.shape[1], q.shape[2]
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    if end <= start:
        return np.zeros((G, d)), np.full(G, -math.inf)
    k, v = gather(k_pages, v_pages, block_table, b, h, end, kv_dtype, k_scale, v_scale)
    s = _group_scores(q[b, h * G:(h + 1) * G], k[start:end], scale)       # [G, n]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ v[start:end]) / l, (m + np.log(l))[:, 0]


def merge_partials(o, lse):
    """Log-sum-exp merge of split partials: [..., S, d], [..., S] -> [..., d]."""
    o = np.asarray(o, np.float64)
    lse = np.asarray(lse, np.float64)
    M = lse.max(axis=-1, keepdims=True)
    live = np.isfinite(M)
    Ms = np.where(live, M, 0.0)
    w = np.where(np.isfinite(lse), np.exp(lse - Ms), 0.0)       # [..., S]
    num = (w[..., None] * o).sum(axis=-2)
    den = w.sum(axis=-1, keepdims=True)
    return np.where(live, num / np.where(den > 0, den, 1.0), 0.0)


def lse_of(q, k_pages, v_pages, block_table, context_lens, scale, kv_dtype="fp16",
           k_scale=None, v_scale=None):
    """ln sum_t exp(s_t) over each (b, j)'s whole context; -inf when L = 0."""
    q = np.asarray(q).astype(np.float64)
    B, Hq, d = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    res = np.full((B, Hq), -math.inf)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        for h in range(Hkv):
            k, _ = gather(k_pages, v_pages, block_table, b, h, L, kv_dtype,
                          k_scale, v_scale)
            s = _group_scores(q[b, h * G:(h + 1) * G], k, scale)
            m = s.max(axis=1)
            res[b, h * G:(h + 1) * G] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return res
