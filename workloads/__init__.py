"""Seeded synthetic inputs for paged MQA/GQA decode attention.

This module is the only code that the oracle side and the GPU side of the
tests and of the benchmark share. It draws random numbers, sequence lengths
and the page assignment, and nothing else: it holds no attention arithmetic
and no cache-append arithmetic. The one statistic computed here is the
calibration scale of each kv head of a one-byte cache (its absolute maximum
divided by the largest code: 448 for fp8 e4m3fn, 127 for int8), an input that
both sides receive unchanged.

Shapes follow the workloads of the decode path being modelled:
  * the MHA/MQA definitions on "TensorRT对Multi-Query Attention的专项优化支持"
    (r-odyssey.com, MHA/MQA formula paragraph): q heads share K/V heads;
  * "优化" on tiny-llm (open-infra-ai.github.io, roadmap table, row 分页 KV):
    K/V live in fixed-size pages reached through a per-sequence block table.

Recipe (identical for every configuration):
  * lengths, page permutation and q come from streams keyed by (seed, tag);
  * token t of sequence b has K and V drawn from a stream keyed by
    (seed, 7, b), so any subset of sequences can be regenerated on its own;
  * values are float32 normal draws times `std`, rounded to fp16;
  * the pool holds exactly the pages the sequences need, shuffled without
    replacement, plus poison pages; unused block-table entries point at a
    poison page, so an over-read shows up as NaN rather than as a fault.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

FP8_E4M3FN_MAX = 448.0
INT8_MAX = 127.0
# largest code magnitude of each one-byte cache type (the calibration divisor)
CODE_MAX = {"fp8_e4m3fn": FP8_E4M3FN_MAX, "int8": INT8_MAX}


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str          # "fp16", "fp8_e4m3fn" or "int8"
    std: float             # standard deviation of q, K and V draws
    lens: tuple            # ("fixed", l0, l1, ...), ("uniform", lo, hi),
                           # ("const", L) or ("lognormal", median, sigma, lo, hi)
    max_len: int           # longest length the recipe can produce
    num_splits: int        # split count the benchmark uses (1 = single pass)
    pool_pages: int = 0    # explicit pool size, 0 = sized to the tokens
    seed: int = 0
    scale: float = 0.0     # softmax scale, 0 = 1/sqrt(head_dim)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.head_dim)

    @property
    def max_blocks(self) -> int:
        return -(-self.max_len // self.block_size)

    @property
    def kv_bytes_per_elem(self) -> int:
        return 2 if self.kv_dtype == "fp16" else 1


CONFIGS = {
    # Tiny MQA: 2 sequences (17, 40), 4 q / 1 kv head, d 64, pages of 16,
    # block table a seeded permutation of a 16-page pool, scale 1/8.
    "tiny_mqa": Config("tiny_mqa", 2, 4, 1, 64, 16, "fp16", 1.0,
                       ("fixed", 17, 40), 40, 1, pool_pages=16, seed=1001,
                       scale=0.125),
    # Llama-style GQA layer: batch 32, 32 q / 8 kv heads, d 128, pages of 16,
    # lengths uniform on [512, 4096].
    "gqa_llama": Config("gqa_llama", 32, 32, 8, 128, 16, "fp16", 1.0,
                        ("uniform", 512, 4096), 4096, 32, seed=1002),
    # Wide MQA: batch 64, 96 q / 1 kv head, d 128, pages of 32, 8192 each,
    # values N(0, 0.5) (standard deviation 0.5).
    "wide_mqa": Config("wide_mqa", 64, 96, 1, 128, 32, "fp16", 0.5,
                       ("const", 8192), 8192, 16, seed=1003),
    # Long-context split-K: batch 4, 32 q / 8 kv heads, d 128, pages of 64,
    # 131072 tokens each, 64 splits merged by log-sum-exp.
    "long_splitk": Config("long_splitk", 4, 32, 8, 128, 64, "fp16", 1.0,
                          ("const", 131072), 131072, 64, seed=1004),
    # Mixed continuous batch, fp8 KV: batch 256, 64 q / 8 kv heads, d 128,
    # pages of 16, lengths log-normal (median 1024, sigma 1) clipped to
    # [1, 32768], per-kv-head fp32 scales, one append per sequence.
    "mixed_fp8": Config("mixed_fp8", 256, 64, 8, 128, 16, "fp8_e4m3fn", 1.0,
                        ("lognormal", 1024, 1.0, 1, 32768), 32768, 16,
                        seed=1005),
    # The same mixed batch with an int8 cache (symmetric codes, per-kv-head
    # K and V scales): the cache precision that must not share one scale
    # between K and V.
    "mixed_int8": Config("mixed_int8", 256, 64, 8, 128, 16, "int8", 1.0,
                         ("lognormal", 1024, 1.0, 1, 32768), 32768, 16,
                         seed=1005),
}

CONFIG_ORDER = ["tiny_mqa", "gqa_llama", "wide_mqa", "long_splitk", "mixed_fp8",
                "mixed_int8"]


def _stream(seed: int, tag: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([seed, tag, *extra])


def draw_lengths(cfg: Config) -> np.ndarray:
    kind = cfg.lens[0]
    rng = _stream(cfg.seed, 1)
    if kind == "fixed":
        lens = np.array(cfg.lens[1:], dtype=np.int64)
    elif kind == "uniform":
        lens = rng.integers(cfg.lens[1], cfg.lens[2], size=cfg.num_seqs,
                            endpoint=True)
    elif kind == "const":
        lens = np.full(cfg.num_seqs, cfg.lens[1], dtype=np.int64)
    elif kind == "lognormal":
        _, median, sigma, lo, hi = cfg.lens
        raw = rng.lognormal(mean=math.log(median), sigma=sigma,
                            size=cfg.num_seqs)
        lens = np.clip(np.rint(raw), lo, hi).astype(np.int64)
    else:
        raise ValueError(f"unknown length recipe {cfg.lens!r}")
    assert lens.shape == (cfg.num_seqs,)
    assert lens.max() <= cfg.max_len
    return lens.astype(np.int32)


class Workload:
    """One seeded draw of a configuration.

    Attributes
      context_lens  int32 [B]           tokens to attend over (incl. the new one)
      block_table   int32 [B, max_blocks] page ids; unused entries = poison page
      num_pages     int                 pool size in pages (incl. poison pages)
      poison_pages  int64 [*]           pages that no sequence owns
      q             fp16  [B, Hq, d]
      scale         float               softmax scale
    Token data come from `token_kv(b)`: K and V as fp16 [L_b, Hkv, d] in
    logical (position) order.
    """

    def __init__(self, cfg: Config, seed: int | None = None, cache_tokens: bool = False):
        if seed is not None:
            cfg = dataclasses.replace(cfg, seed=seed)
        self.cfg = cfg
        # keep each sequence's drawn K/V (same values, drawn once) for callers
        # that read them several times over (full-size parity checks)
        self._token_cache = {} if cache_tokens else None
        B, bs = cfg.num_seqs, cfg.block_size
        self.context_lens = draw_lengths(cfg)
        nblk = -(-self.context_lens.astype(np.int64) // bs)
        used = int(nblk.sum())
        rng = _stream(cfg.seed, 2)
        if cfg.pool_pages:
            assert cfg.pool_pages >= used + 1
            perm = rng.permutation(cfg.pool_pages)
            self.num_pages = cfg.pool_pages
            self.poison_pages = np.sort(perm[used:])
        else:
            perm = rng.permutation(used)
            self.num_pages = used + 1
            self.poison_pages = np.array([used], dtype=np.int64)
        poison = int(self.poison_pages[0])
        self.block_table = np.full((B, cfg.max_blocks), poison, dtype=np.int32)
        off = 0
        for b in range(B):
            n = int(nblk[b])
            self.block_table[b, :n] = perm[off:off + n]
            off += n
        qr = _stream(cfg.seed, 3)
        self.q = (qr.standard_normal((B, cfg.num_q_heads, cfg.head_dim),
                                     dtype=np.float32) * cfg.std
                  ).astype(np.float16)
        self.scale = cfg.softmax_scale
        self._scales = None

    # -- token data -------------------------------------------------------
    def token_kv(self, b: int):
        if self._token_cache is not None and b in self._token_cache:
            return self._token_cache[b]
        cfg = self.cfg
        L = int(self.context_lens[b])
        rng = _stream(cfg.seed, 7, b)
        shape = (L, cfg.num_kv_heads, cfg.head_dim)
        k = (rng.standard_normal(shape, dtype=np.float32) * cfg.std
             ).astype(np.float16)
        v = (rng.standard_normal(shape, dtype=np.float32) * cfg.std
             ).astype(np.float16)
        if self._token_cache is not None:
            self._token_cache[b] = (k, v)
        return k, v

    def tokens(self, seqs=None, upto_last: bool = False):
        """K, V fp16 [T, Hkv, d] with seq_ids, positions int32 [T].

        `upto_last` drops each sequence's final token (the one a decode step
        appends), leaving the pool contents that precede that step.
        """
        seqs = range(self.cfg.num_seqs) if seqs is None else seqs
        ks, vs, sid, pos = [], [], [], []
        for b in seqs:
            k, v = self.token_kv(b)
            n = max(0, k.shape[0] - 1) if upto_last else k.shape[0]
            ks.append(k[:n]); vs.append(v[:n])
            sid.append(np.full(n, b, dtype=np.int32))
            pos.append(np.arange(n, dtype=np.int32))
        return (np.concatenate(ks), np.concatenate(vs),
                np.concatenate(sid), np.concatenate(pos))

    def new_tokens(self):
        """The token each sequence appends in a decode step: its last one.

        Returns K, V fp16 [B, Hkv, d] and positions int32 [B] (= L_b - 1;
        a sequence with L_b = 0 gets position -1, which an append skips).
        """
        cfg = self.cfg
        k = np.zeros((cfg.num_seqs, cfg.num_kv_heads, cfg.head_dim), np.float16)
        v = np.zeros_like(k)
        for b in range(cfg.num_seqs):
            kb, vb = self.token_kv(b)
            if kb.shape[0]:
                k[b] = kb[-1]; v[b] = vb[-1]
        return k, v, (self.context_lens - 1).astype(np.int32)

    def step_inputs(self, step: int):
        """q [B, Hq, d] and the new K / V rows [B, Hkv, d] (fp16) of decode
        step `step` >= 1 after the one this draw describes, from streams of
        their own (seed, 8, step): inputs for runs of several decode steps."""
        cfg = self.cfg
        rng = _stream(cfg.seed, 8, step)
        B = cfg.num_seqs
        q = (rng.standard_normal((B, cfg.num_q_heads, cfg.head_dim), dtype=np.float32)
             * cfg.std).astype(np.float16)
        k = (rng.standard_normal((B, cfg.num_kv_heads, cfg.head_dim), dtype=np.float32)
             * cfg.std).astype(np.float16)
        v = (rng.standard_normal((B, cfg.num_kv_heads, cfg.head_dim), dtype=np.float32)
             * cfg.std).astype(np.float16)
        return q, k, v

    # -- one-byte cache calibration ----------------------------------------
    def kv_scales(self):
        """Per-kv-head fp32 scales of a one-byte cache: amax over all of that
        head's K (resp. V) values / the largest code (448 for fp8 e4m3fn,
        127 for int8).

        Returns (k_scale, v_scale), float32 [Hkv]. fp16 workloads get ones.
        """
        cfg = self.cfg
        if self._scales is None:
            H = cfg.num_kv_heads
            ka = np.zeros(H, np.float32); va = np.zeros(H, np.float32)
            if cfg.kv_dtype in CODE_MAX:
                qmax = np.float32(CODE_MAX[cfg.kv_dtype])
                for b in range(cfg.num_seqs):
                    k, v = self.token_kv(b)
                    if k.shape[0] == 0:
                        continue
                    ka = np.maximum(ka, np.abs(k).max(axis=(0, 2)).astype(np.float32))
                    va = np.maximum(va, np.abs(v).max(axis=(0, 2)).astype(np.float32))
                # a head with no data at all keeps scale 1
                ks = np.where(ka > 0, ka / qmax, np.float32(1))
                vs = np.where(va > 0, va / qmax, np.float32(1))
            else:
                ks = np.ones(H, np.float32); vs = np.ones(H, np.float32)
            self._scales = (ks.astype(np.float32), vs.astype(np.float32))
        return self._scales

    # -- accounting -------------------------------------------------------
    def kv_bytes(self) -> int:
        """Bytes of K and V one attention call reads (sum L * Hkv * d * 2 * e)."""
        cfg = self.cfg
        return int(self.context_lens.astype(np.int64).sum()) * \
            cfg.num_kv_heads * cfg.head_dim * 2 * cfg.kv_bytes_per_elem


def arrivals(cfg: Config, count: int, tag: int):
    """Prompts of `count` sequences joining a running batch: lengths from the
    configuration's length recipe and K / V [L, Hkv, d] fp16 per prompt, from
    streams keyed (seed, 10, tag) and (seed, 11, tag, i)."""
    sub = dataclasses.replace(cfg, num_seqs=count, seed=cfg.seed)
    lens = draw_lengths(dataclasses.replace(sub, seed=int(_stream(cfg.seed, 10, tag)
                                                           .integers(2 ** 31))))
    prompts = []
    for i, L in enumerate(lens):
        rng = _stream(cfg.seed, 11, tag, i)
        shape = (int(L), cfg.num_kv_heads, cfg.head_dim)
        k = (rng.standard_normal(shape, dtype=np.float32) * cfg.std).astype(np.float16)
        v = (rng.standard_normal(shape, dtype=np.float32) * cfg.std).astype(np.float16)
        prompts.append((k, v))
    return lens, prompts


@dataclasses.dataclass(frozen=True)
class GemmConfig:
    """A decode projection: M activation rows times a [K, N] weight held
    transposed ([N, K]), fp16 or int8 codes with scales per `group` of k."""
    name: str
    M: int
    K: int
    N: int
    w_dtype: str            # "fp16" or "int8"
    group: int = 128
    seed: int = 0

    @property
    def weight_bytes(self) -> int:
        e = 2 if self.w_dtype == "fp16" else 1
        s = 0 if self.w_dtype == "fp16" else self.N * (self.K // self.group) * 4
        return self.N * self.K * e + s


GEMM_CONFIGS = {
    # The projections around the grouped-query attention layer of the
    # Llama-style workload (32 q / 8 kv heads of 128): QKV (K 4096 -> N
    # (32 + 2 * 8) * 128 = 6144), fp16 and with int8 weights; the output
    # projection (4096 -> 4096); a 32000-row vocabulary head.
    "proj_qkv": GemmConfig("proj_qkv", 1, 4096, 6144, "fp16", seed=2001),
    "proj_qkv_w8a16": GemmConfig("proj_qkv_w8a16", 1, 4096, 6144, "int8", 128, seed=2002),
    "proj_o": GemmConfig("proj_o", 1, 4096, 4096, "fp16", seed=2003),
    "lm_head": GemmConfig("lm_head", 1, 4096, 32000, "fp16", seed=2004),
    # int8 weights with N = 4864, the width the pages time for their W8A16
    # M == 1 path (their K is not given; 896 taken, the model width that
    # goes with a 4864-wide MLP)
    "mlp_w8a16_4864": GemmConfig("mlp_w8a16_4864", 1, 896, 4864, "int8", 128, seed=2005),
}


def make_gemm(cfg: GemmConfig):
    """x [M, K] fp16 ~ N(0, 1); the weight as stored before transposition,
    w [K, N]: fp16 ~ N(0, 1/K) (so y is of order 1), or int8 codes uniform in
    [-127, 127] with scales [K / group, N] uniform in [0.5, 1.5] / (127
    sqrt(K / 3)). Returns (x, w, scales or None)."""
    rng = _stream(cfg.seed, 20)
    x = rng.standard_normal((cfg.M, cfg.K), dtype=np.float32).astype(np.float16)
    if cfg.w_dtype == "fp16":
        w = (rng.standard_normal((cfg.K, cfg.N), dtype=np.float32)
             / np.float32(math.sqrt(cfg.K))).astype(np.float16)
        return x, w, None
    w = rng.integers(-127, 128, (cfg.K, cfg.N), dtype=np.int64).astype(np.int8)
    s = (rng.uniform(0.5, 1.5, (cfg.K // cfg.group, cfg.N))
         / (127.0 * math.sqrt(cfg.K / 3.0))).astype(np.float32)
    return x, w, s


def make(name: str, seed: int | None = None, cache_tokens: bool = False) -> Workload:
    return Workload(CONFIGS[name], seed, cache_tokens)


def make_case(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
              lens, kv_dtype="fp16", std=1.0, seed=0, scale=0.0,
              extra_pages=0, max_len=None) -> Workload:
    """An arbitrary small case with explicit lengths (for parity sweeps)."""
    lens = tuple(int(x) for x in lens)
    max_len = max(max(lens), 1) if max_len is None else max_len
    bs = block_size
    used = sum(-(-l // bs) for l in lens)
    cfg = Config("case", num_seqs, num_q_heads, num_kv_heads, head_dim, bs,
                 kv_dtype, std, ("fixed",) + lens, max_len, 1,
                 pool_pages=used + 1 + extra_pages, seed=seed, scale=scale)
    return Workload(cfg)
