"""The host-side KV page manager (CPU only; the manager never touches a GPU).

Checked against the sizing formula of the pages (2 x layers x kv heads x
head_dim x max_seq_len x element bytes), against invariants (every page is
either free or held by exactly one live slot, rows list a slot's pages in
order and -1 after them, failed calls change nothing) and against a plain
Python model of the same free list driven through a long random sequence of
joins, leaves, decode steps and reservations.
"""
import numpy as np
import pytest

import paged_mqa_gqa_amd as pa
from paged_mqa_gqa_amd.kv_manager import NO_PAGES, NO_SLOT


def test_sizes_follow_the_per_sequence_formula():
    # tiny-llm "优化", section 2: 2 x layers x kv_heads x head_dim x max_seq_len x 2 B
    assert pa.kv_bytes_per_sequence(32, 8, 128, 4096, pa.KV_FP16) == 2 * 32 * 8 * 128 * 4096 * 2
    assert pa.kv_bytes_per_sequence(1, 8, 128, 1000, pa.KV_FP8_E4M3FN) == 2 * 8 * 128 * 1000
    assert pa.kv_bytes_per_sequence(2, 1, 64, 7, pa.KV_INT8) == 2 * 2 * 64 * 7
    # one layer's pools [P, Hkv, bs, d] for K and for V
    assert pa.kv_pool_bytes(100, 8, 128, 16, pa.KV_FP16) == 2 * 100 * 8 * 16 * 128 * 2
    per_page = pa.kv_pool_bytes(1, 8, 128, 16, pa.KV_FP8_E4M3FN)
    assert pa.kv_pages_for_budget(10 * per_page * 3 + 5, 3, 8, 128, 16,
                                  pa.KV_FP8_E4M3FN) == 10
    # a pool of pages for S sequences of L tokens holds exactly their KV
    L, bs = 4096, 16
    assert pa.kv_pool_bytes(32 * L // bs, 8, 128, bs, pa.KV_FP16) == \
        32 * pa.kv_bytes_per_sequence(1, 8, 128, L, pa.KV_FP16)
    with pytest.raises(ValueError):
        pa.kv_bytes_per_sequence(0, 8, 128, 10)
    with pytest.raises(ValueError):
        pa.kv_pool_bytes(10, 8, 128, 16, kv_dtype=9)


def test_invalid_sizes_are_rejected():
    for args in ((0, 16, 4, 8), (10, 8, 4, 8), (10, 16, 0, 8), (10, 16, 4, 0),
                 (10, 48, 4, 8)):
        with pytest.raises(ValueError):
            pa.KvPageManager(*args)


def _check_invariants(m, model=None):
    bt = m.block_table()
    held = []
    for s in range(m.num_slots):
        L = m.length(s)
        row = bt[s]
        if L < 0:
            assert np.all(row == -1)
            assert m.pages_held(s) == -1
            continue
        n = m.pages_held(s)
        assert n >= -(-L // m.block_size)
        assert np.all(row[:n] >= 0) and np.all(row[:n] < m.num_pages)
        assert np.all(row[n:] == -1)
        held.extend(row[:n].tolist())
        if model is not None:
            assert row[:n].tolist() == model["pages"][s]
            assert L == model["len"][s]
    assert len(held) == len(set(held)), "a page is held twice"
    assert len(held) + m.free_pages == m.num_pages
    lens, pos = m.batch_state()
    for s in range(m.num_slots):
        L = m.length(s)
        assert lens[s] == max(L, 0)
        assert pos[s] == (L - 1 if L > 0 else -1)


def test_admit_plan_and_release():
    m = pa.KvPageManager(12, 16, 3, 4)
    assert m.free_pages == 12 and m.live_slots == 0
    a = m.admit(20)                 # 2 pages
    b = m.admit(16)                 # 1 page, exactly full
    c = m.admit(0)                  # no pages yet
    assert (a, b, c) == (0, 1, 2)
    assert m.free_pages == 9
    with pytest.raises(pa.PagedAttnError) as e:
        m.admit(1)
    assert e.value.status == NO_SLOT
    bt, lens, pos = m.plan_step()
    # slot 0: token 20 lands in its second page; slot 1: token 16 needs a
    # new page; slot 2: token 0 needs its first page
    assert lens.tolist() == [21, 17, 1] and pos.tolist() == [20, 16, 0]
    assert [m.pages_held(s) for s in range(3)] == [2, 2, 1]
    assert bt[0, :2].tolist() == [0, 1] and bt[1, :2].tolist() == [2, 3]
    assert bt[2, 0] == 4
    _check_invariants(m)
    m.release(1)
    assert m.free_pages == 12 - 3
    # released pages come back first, last page first
    assert m.admit(32) == 1
    assert m.block_table()[1, :2].tolist() == [2, 3]
    _check_invariants(m)


def test_failed_calls_change_nothing():
    m = pa.KvPageManager(4, 16, 4, 2)
    m.admit(16)
    m.admit(16)
    m.admit(16)
    before = (m.block_table().copy(), m.batch_state(), m.free_pages)
    with pytest.raises(pa.PagedAttnError) as e:
        m.plan_step()                    # 3 slots each need a page, 1 is free
    assert e.value.status == NO_PAGES
    after = (m.block_table(), m.batch_state(), m.free_pages)
    assert np.array_equal(before[0], after[0]) and before[2] == after[2]
    assert all(np.array_equal(x, y) for x, y in zip(before[1], after[1]))
    with pytest.raises(pa.PagedAttnError):
        m.admit(17)                      # two pages, one free
    with pytest.raises(pa.PagedAttnError) as e:
        m.admit(40)                      # more than a row can map
    assert e.value.status == -2
    with pytest.raises(pa.PagedAttnError):
        m.reserve_ahead(17)              # rows of 2 pages hold 32 tokens
    with pytest.raises(pa.PagedAttnError) as e:
        m.commit_steps(1)                # no slot holds room for a 17th token
    assert e.value.status == NO_PAGES
    with pytest.raises(pa.PagedAttnError) as e:
        m.release(3)
    assert e.value.status == NO_SLOT
    assert m.free_pages == 1
    _check_invariants(m)


def test_reserve_ahead_then_commit():
    m = pa.KvPageManager(40, 16, 4, 8)
    for n in (5, 16, 31, 0):
        m.admit(n)
    m.reserve_ahead(10)
    assert [m.pages_held(s) for s in range(4)] == [1, 2, 3, 1]
    m.commit_steps(10)
    assert [m.length(s) for s in range(4)] == [15, 26, 41, 10]
    with pytest.raises(pa.PagedAttnError):
        m.commit_steps(2)                # slot 0 holds room for 16 tokens only
    _check_invariants(m)


def test_random_join_leave_matches_a_python_model():
    """A long random run of joins, leaves, decode steps and reservations:
    after every call the manager's table, lengths and free count equal a
    plain Python model of a LIFO free list."""
    rng = np.random.default_rng(7)
    P, bs, S, MB = 200, 16, 12, 16
    m = pa.KvPageManager(P, bs, S, MB)
    model = {"free": list(range(P - 1, -1, -1)), "pages": [[] for _ in range(S)],
             "len": [-1] * S}

    def need(s, n):
        return -(-n // bs) if n > 0 else 0

    for it in range(3000):
        op = rng.integers(0, 4)
        if op == 0:                                  # join
            n = int(rng.integers(0, 60))
            free_slots = [s for s in range(S) if model["len"][s] < 0]
            k = need(None, n)
            if not free_slots:
                exp = NO_SLOT
            elif k > len(model["free"]):
                exp = NO_PAGES
            else:
                exp = free_slots[0]
            try:
                got = m.admit(n)
            except pa.PagedAttnError as e:
                got = e.status
            assert got == exp, (it, got, exp)
            if exp >= 0:
                model["pages"][exp] = [model["free"].pop() for _ in range(k)]
                model["len"][exp] = n
        elif op == 1:                                # leave
            s = int(rng.integers(0, S))
            try:
                m.release(s)
                got = 0
            except pa.PagedAttnError as e:
                got = e.status
            if model["len"][s] < 0:
                assert got == NO_SLOT
            else:
                assert got == 0
                model["free"].extend(reversed(model["pages"][s]))
                model["pages"][s] = []
                model["len"][s] = -1
        else:                                        # decode step (or reserve)
            steps = 1 if op == 2 else int(rng.integers(0, 4))
            live = [s for s in range(S) if model["len"][s] >= 0]
            extra = [max(0, need(s, model["len"][s] + steps) - len(model["pages"][s]))
                     for s in live]
            too_long = any(need(s, model["len"][s] + steps) > MB for s in live)
            try:
                if op == 2:
                    bt, lens, pos = m.plan_step()
                else:
                    m.reserve_ahead(steps)
                got = 0
            except pa.PagedAttnError as e:
                got = e.status
            if too_long:
                assert got == -2
            elif sum(extra) > len(model["free"]):
                assert got == NO_PAGES
            else:
                assert got == 0
                for s, x in zip(live, extra):
                    model["pages"][s] += [model["free"].pop() for _ in range(x)]
                if op == 2:
                    for s in range(S):
                        if model["len"][s] >= 0:
                            assert lens[s] == model["len"][s] + 1 and pos[s] == model["len"][s]
                            model["len"][s] += 1
                        else:
                            assert lens[s] == 0 and pos[s] == -1
        _check_invariants(m, model)
        # a full row cannot grow: retire the longest sequences now and then
        if it % 50 == 49:
            for s in range(S):
                if model["len"][s] > (MB - 2) * bs:
                    m.release(s)
                    model["free"].extend(reversed(model["pages"][s]))
                    model["pages"][s] = []
                    model["len"][s] = -1
    assert m.live_slots == sum(1 for L in model["len"] if L >= 0)
