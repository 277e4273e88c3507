"""A host-side block pool with reference counts, forking and copy-on-write.

This is the bookkeeping side of paged KV memory, used to lay out seeded test and
benchmark batches. It decides *where* tokens live; it computes nothing of the
attention itself.

* The pool hands out fixed-size physical blocks from a global free list and takes
  them back when a sequence ends ("vLLM推理引擎PagedAttention原理与性能优化实战",
  §2.2 and §四; "vLLM 推理优化技术深度调研报告", 维度一.4).
* A new block is taken only when the current one is full ("vLLM 是什么…", §二).
* Sequences that fork share every block; a shared block carries a reference count
  and is read-only. The first write into a shared block takes a fresh block and
  records a (src, dst) copy; the last holder writes in place
  ("vLLM推理引擎PagedAttention原理与性能优化实战", §3.2).

A slot is the flat index block * block_size + offset into the pool.
"""
from __future__ import annotations

from collections import deque


class PoolExhausted(RuntimeError):
    pass


class BlockPool:
    def __init__(self, num_blocks: int, block_size: int = 16, order=None):
        """`order` is the sequence in which free blocks are handed out (a seeded
        permutation scatters logically adjacent blocks across the pool)."""
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = range(self.num_blocks) if order is None else [int(b) for b in order]
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("order must be a permutation of the pool")
        self.free = deque(order)
        self.refcount = [0] * self.num_blocks

    def allocate(self) -> int:
        if not self.free:
            raise PoolExhausted(f"all {self.num_blocks} blocks are in use")
        b = self.free.popleft()
        self.refcount[b] = 1
        return b

    def incref(self, b: int) -> None:
        if self.refcount[b] <= 0:
            raise ValueError(f"block {b} is not allocated")
        self.refcount[b] += 1

    def decref(self, b: int) -> None:
        if self.refcount[b] <= 0:
            raise ValueError(f"block {b} is not allocated")
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free.append(b)

    @property
    def num_free(self) -> int:
        return len(self.free)


class Sequence:
    """One sequence's block list and token count inside a BlockPool."""

    def __init__(self, pool: BlockPool):
        self.pool = pool
        self.blocks: list[int] = []
        self.num_tokens = 0

    def fork(self) -> "Sequence":
        child = Sequence(self.pool)
        for b in self.blocks:
            self.pool.incref(b)
        child.blocks = list(self.blocks)
        child.num_tokens = self.num_tokens
        return child

    def append_slot(self):
        """Make room for one more token. Returns (slot, copy) where copy is a
        (src, dst) block pair when a shared block had to be copied, else None."""
        P = self.pool.block_size
        copy = None
        if self.num_tokens % P == 0:
            self.blocks.append(self.pool.allocate())
        else:
            last = self.blocks[-1]
            if self.pool.refcount[last] > 1:
                fresh = self.pool.allocate()
                self.pool.decref(last)
                self.blocks[-1] = fresh
                copy = (last, fresh)
        slot = self.blocks[-1] * P + self.num_tokens % P
        self.num_tokens += 1
        return slot, copy

    def extend(self, n: int):
        """Append n tokens; returns their slots and any copies made on the way."""
        slots, copies = [], []
        for _ in range(n):
            s, c = self.append_slot()
            slots.append(s)
            if c is not None:
                copies.append(c)
        return slots, copies

    def free(self) -> None:
        for b in self.blocks:
            self.pool.decref(b)
        self.blocks = []
        self.num_tokens = 0
