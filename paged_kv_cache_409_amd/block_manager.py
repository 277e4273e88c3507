"""Python binding of the C++ block manager (include/pkv_block_manager.h): argument marshalling only.

The manager decides where tokens live; its outputs feed the kernels: slots for
reshape_and_cache, copy-on-write pairs for copy_blocks, swap pairs for swap_blocks, and
block-table rows for the attention calls.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib
from .ops import PkvError


def _ptr(a: np.ndarray):
    # the plain address: ctypes.cast would build reference cycles on every call
    return a.ctypes.data if a is not None and a.size else None


class BlockManager:
    def __init__(self, num_gpu_blocks: int, num_host_blocks: int = 0, block_size: int = 16,
                 prefix_caching: bool = False):
        self._lib = _lib.load()
        h = ctypes.c_void_p()
        self._check("pkv_bm_create", self._lib.pkv_bm_create(num_gpu_blocks, num_host_blocks, block_size,
                                                             int(prefix_caching), ctypes.byref(h)))
        self._h = h
        self.block_size = block_size

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @staticmethod
    def _check(fn: str, status: int) -> None:
        if status != 0:
            raise PkvError(fn, status)

    @staticmethod
    def _tokens(tokens, n):
        if tokens is None:
            return None
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        if t.shape != (n,):
            raise ValueError("one token id per token")
        return t

    def add_sequence(self, seq_id: int, num_tokens: int, tokens=None):
        """Returns (slots int64 [num_tokens], cached_tokens)."""
        t = self._tokens(tokens, num_tokens)
        slots = np.empty(num_tokens, dtype=np.int64)
        cached = ctypes.c_int(0)
        self._check("pkv_bm_add_sequence", self._lib.pkv_bm_add_sequence(
            self._h, seq_id, _ptr(t), num_tokens, _ptr(slots), ctypes.byref(cached)))
        return slots, cached.value

    def append(self, seq_id: int, n: int = 1, tokens=None):
        """Returns (slots int64 [n], copy-on-write pairs int64 [k, 2])."""
        t = self._tokens(tokens, n)
        slots = np.empty(n, dtype=np.int64)
        pairs = np.empty((1, 2), dtype=np.int64)
        ncow = ctypes.c_int(0)
        self._check("pkv_bm_append", self._lib.pkv_bm_append(self._h, seq_id, _ptr(t), n, _ptr(slots), _ptr(pairs), 1,
                                                             ctypes.byref(ncow)))
        return slots, pairs[:ncow.value]

    def append_batch(self, seq_ids, tokens=None):
        """One new token for each sequence (a decode step). Returns (slots int64 [n], pairs int64 [k, 2])."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = len(ids)
        t = self._tokens(tokens, n)
        slots = np.empty(n, dtype=np.int64)
        pairs = np.empty((max(n, 1), 2), dtype=np.int64)
        ncow = ctypes.c_int(0)
        self._check("pkv_bm_append_batch", self._lib.pkv_bm_append_batch(
            self._h, _ptr(ids), n, _ptr(t), _ptr(slots), _ptr(pairs), n, ctypes.byref(ncow)))
        return slots, pairs[:ncow.value]

    def append_step(self, seq_ids, tokens=None):
        """append_batch for decode_step's fused copy-on-write. Returns (slots int64 [n],
        cow_src int32 [n]: each sequence's copy-on-write source, -1: none)."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = len(ids)
        t = self._tokens(tokens, n)
        slots = np.empty(n, dtype=np.int64)
        cow_src = np.empty(max(n, 1), dtype=np.int32)
        self._check("pkv_bm_append_step", self._lib.pkv_bm_append_step(
            self._h, _ptr(ids), n, _ptr(t), _ptr(slots), _ptr(cow_src)))
        return slots, cow_src[:n]

    def fork(self, parent_id: int, child_id: int) -> None:
        self._check("pkv_bm_fork", self._lib.pkv_bm_fork(self._h, parent_id, child_id))

    def free(self, seq_id: int) -> None:
        self._check("pkv_bm_free", self._lib.pkv_bm_free(self._h, seq_id))

    def block_tables(self, seq_ids, max_blocks: int, pad_block: int = 0):
        """Returns (tables int32 [n, max_blocks], context_lens int32 [n])."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tables = np.empty((len(ids), max_blocks), dtype=np.int32)
        ctx = np.empty(len(ids), dtype=np.int32)
        self._check("pkv_bm_block_tables", self._lib.pkv_bm_block_tables(
            self._h, _ptr(ids), len(ids), _ptr(tables), max_blocks, pad_block, _ptr(ctx)))
        return tables, ctx

    def _swap(self, fn: str, seq_id: int):
        _, nb, _ = self.sequence_info(seq_id)
        pairs = np.empty((max(nb, 1), 2), dtype=np.int64)
        n = ctypes.c_int(0)
        self._check(fn, getattr(self._lib, fn)(self._h, seq_id, _ptr(pairs), nb, ctypes.byref(n)))
        return pairs[:n.value]

    def swap_out(self, seq_id: int):
        """Returns (GPU block, host block) pairs for swap_blocks."""
        return self._swap("pkv_bm_swap_out", seq_id)

    def swap_in(self, seq_id: int):
        """Returns (host block, GPU block) pairs for swap_blocks."""
        return self._swap("pkv_bm_swap_in", seq_id)

    def num_free(self):
        """(free GPU blocks, known blocks waiting for reuse, free host blocks)."""
        a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        self._check("pkv_bm_num_free", self._lib.pkv_bm_num_free(self._h, ctypes.byref(a), ctypes.byref(b),
                                                                 ctypes.byref(c)))
        return a.value, b.value, c.value

    def refcount(self, block: int) -> int:
        c = ctypes.c_int()
        self._check("pkv_bm_refcount", self._lib.pkv_bm_refcount(self._h, block, ctypes.byref(c)))
        return c.value

    def sequence_info(self, seq_id: int):
        """(tokens, blocks, on_gpu)."""
        a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        self._check("pkv_bm_sequence_info", self._lib.pkv_bm_sequence_info(self._h, seq_id, ctypes.byref(a),
                                                                           ctypes.byref(b), ctypes.byref(c)))
        return a.value, b.value, bool(c.value)
