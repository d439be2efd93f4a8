"""The seeded generator produces the shapes and structure of the five workloads."""
import numpy as np
import pytest

from workloads import CONFIG_ORDER, CONFIGS, draw_lengths, make


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_block_table_is_a_partial_permutation(name):
    w = make(name)
    cfg = w.cfg
    nblk = -(-w.context_lens.astype(np.int64) // cfg.block_size)
    used = np.concatenate([w.block_table[b, :nblk[b]] for b in range(cfg.num_seqs)])
    assert len(set(used.tolist())) == len(used)            # no page shared
    assert used.min() >= 0 and used.max() < w.num_pages
    assert not set(used.tolist()) & set(w.poison_pages.tolist())
    for b in range(cfg.num_seqs):                           # unused -> poison
        assert set(w.block_table[b, nblk[b]:].tolist()) <= set(w.poison_pages.tolist())
    assert w.q.shape == (cfg.num_seqs, cfg.num_q_heads, cfg.head_dim)
    assert w.q.dtype == np.float16


def test_length_recipes():
    assert draw_lengths(CONFIGS["tiny_mqa"]).tolist() == [17, 40]
    l2 = draw_lengths(CONFIGS["gqa_llama"])
    assert l2.min() >= 512 and l2.max() <= 4096 and len(l2) == 32
    assert np.all(draw_lengths(CONFIGS["wide_mqa"]) == 8192)
    assert np.all(draw_lengths(CONFIGS["long_splitk"]) == 131072)
    l5 = draw_lengths(CONFIGS["mixed_fp8"])
    assert l5.min() >= 1 and l5.max() <= 32768 and len(l5) == 256
    assert 600 < np.median(l5) < 1700


def test_tiny_pool_is_sixteen_pages_with_eleven_poisoned():
    w = make("tiny_mqa")
    assert w.num_pages == 16 and len(w.poison_pages) == 11
    assert w.block_table.shape == (2, 3)


def test_same_seed_same_data_and_per_sequence_streams():
    a, b = make("gqa_llama"), make("gqa_llama")
    assert np.array_equal(a.block_table, b.block_table)
    ka, va = a.token_kv(5)
    kb, vb = b.token_kv(5)
    assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    assert ka.shape == (a.context_lens[5], 8, 128)
    assert not np.array_equal(a.token_kv(4)[0][:10], ka[:10])


def test_std_applies():
    w = make("wide_mqa")
    k, _ = w.token_kv(0)
    assert 0.45 < float(k[:512].astype(np.float32).std()) < 0.55
