"""Oracle-side test helpers: build the oracle's pools from a seeded workload.

Only test code uses this; it calls the generator (workloads) and the oracle.
"""
import numpy as np

import oracle
from workloads import Workload


def oracle_pools(w: Workload, seqs=None, upto_last=False):
    """Pools holding every token of `seqs` (all by default), appended by the oracle.

    Returns (k_pages, v_pages, k_scale, v_scale). Unwritten slots are NaN.
    """
    cfg = w.cfg
    k, v = oracle.empty_pools(w.num_pages, cfg.num_kv_heads, cfg.block_size,
                              cfg.head_dim, cfg.kv_dtype)
    K, V, sid, pos = w.tokens(seqs, upto_last)
    ks, vs = w.kv_scales()
    k, v = oracle.kv_append(k, v, w.block_table, sid, pos, K, V, cfg.kv_dtype,
                            ks, vs)
    return k, v, ks, vs


def oracle_decode(w: Workload, seqs=None):
    k, v, ks, vs = oracle_pools(w, seqs)
    return oracle.decode(w.q, k, v, w.block_table, w.context_lens, w.scale,
                         w.cfg.kv_dtype, ks, vs, seqs=seqs)


def contiguous_reference_sdpa(q, K, V, scale):
    """torch SDPA in float64 on CPU: q [Hq, d], K/V [Hkv, L, d] -> [Hq, d]."""
    import torch
    Hq = q.shape[0]
    Hkv = K.shape[0]
    G = Hq // Hkv
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, :, None, :]
    Kt = torch.from_numpy(np.asarray(K, np.float64)).repeat_interleave(G, 0)[None].contiguous()
    Vt = torch.from_numpy(np.asarray(V, np.float64)).repeat_interleave(G, 0)[None].contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
    return o[0, :, 0, :].numpy()
