"""Python binding of the host-side KV page manager (include/paged_kv_manager.h).

Argument marshalling only: the bookkeeping (free list, each slot's pages and
length, the per-step batch arrays) runs in the library's C++ code; this
module hands it numpy buffers and raises on a negative status.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import KV_FP16, PagedAttnError, load

NO_PAGES = -8
NO_SLOT = -9


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def kv_bytes_per_sequence(num_layers, num_kv_heads, head_dim, max_seq_len, kv_dtype=KV_FP16):
    """2 x layers x kv heads x head_dim x max_seq_len x element bytes."""
    n = int(load().pa_kv_bytes_per_sequence(num_layers, num_kv_heads, head_dim, max_seq_len,
                                             kv_dtype))
    if n < 0:
        raise ValueError("invalid KV cache configuration")
    return n


def kv_pool_bytes(num_pages, num_kv_heads, head_dim, block_size, kv_dtype=KV_FP16):
    """Bytes of one layer's K and V pools of num_pages pages."""
    n = int(load().pa_kv_pool_bytes(num_pages, num_kv_heads, head_dim, block_size, kv_dtype))
    if n < 0:
        raise ValueError("invalid pool configuration")
    return n


def kv_pages_for_budget(budget_bytes, num_layers, num_kv_heads, head_dim, block_size,
                        kv_dtype=KV_FP16):
    """Most pages whose K and V pools over num_layers layers fit the budget."""
    n = int(load().pa_kv_pages_for_budget(int(budget_bytes), num_layers, num_kv_heads,
                                          head_dim, block_size, kv_dtype))
    if n < 0:
        raise ValueError("invalid pool configuration")
    return n


class KvPageManager:
    """Pages of a preallocated pool handed out to a fixed batch of slots.

    `admit(n)` takes a free slot and the pages of its first n tokens,
    `release(slot)` returns them, `plan_step()` gives every live slot the page
    of its next token and returns the step's block table, context lengths and
    append positions (numpy int32) for the decode call; free slots appear as
    length 0 / position -1 sequences, so the batch shape never changes.
    """

    def __init__(self, num_pages, block_size, num_slots, max_blocks_per_seq):
        self._lib = load()
        self._h = self._lib.pa_kvm_create(num_pages, block_size, num_slots,
                                          max_blocks_per_seq)
        if not self._h:
            raise ValueError("invalid page manager sizes")
        self.num_pages, self.block_size = num_pages, block_size
        self.num_slots, self.max_blocks = num_slots, max_blocks_per_seq

    def close(self):
        if self._h:
            self._lib.pa_kvm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, fn, rc):
        if rc < 0:
            raise PagedAttnError(fn, rc)
        return rc

    @property
    def free_pages(self) -> int:
        return int(self._lib.pa_kvm_free_pages(self._h))

    @property
    def live_slots(self) -> int:
        return int(self._lib.pa_kvm_live_slots(self._h))

    def length(self, slot) -> int:
        return int(self._lib.pa_kvm_length(self._h, slot))

    def pages_held(self, slot) -> int:
        return int(self._lib.pa_kvm_pages_held(self._h, slot))

    def admit(self, num_tokens) -> int:
        return self._check("pa_kvm_admit", int(self._lib.pa_kvm_admit(self._h, num_tokens)))

    def release(self, slot):
        self._check("pa_kvm_release", int(self._lib.pa_kvm_release(self._h, slot)))

    def reserve_ahead(self, steps):
        self._check("pa_kvm_reserve_ahead", int(self._lib.pa_kvm_reserve_ahead(self._h, steps)))

    def commit_steps(self, steps):
        self._check("pa_kvm_commit_steps", int(self._lib.pa_kvm_commit_steps(self._h, steps)))

    def block_table(self) -> np.ndarray:
        bt = np.empty((self.num_slots, self.max_blocks), np.int32)
        self._check("pa_kvm_block_table", int(self._lib.pa_kvm_block_table(self._h, _i32p(bt))))
        return bt

    def batch_state(self):
        lens = np.empty(self.num_slots, np.int32)
        pos = np.empty(self.num_slots, np.int32)
        self._check("pa_kvm_batch_state",
                    int(self._lib.pa_kvm_batch_state(self._h, _i32p(lens), _i32p(pos))))
        return lens, pos

    def plan_step(self):
        """(block_table [slots, max_blocks], context_lens [slots], positions [slots])."""
        bt = np.empty((self.num_slots, self.max_blocks), np.int32)
        lens = np.empty(self.num_slots, np.int32)
        pos = np.empty(self.num_slots, np.int32)
        self._check("pa_kvm_plan_step", int(self._lib.pa_kvm_plan_step(
            self._h, _i32p(bt), _i32p(lens), _i32p(pos))))
        return bt, lens, pos
