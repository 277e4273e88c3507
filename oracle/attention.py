"""Paged decode attention as its definition: gather, then textbook softmax attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg use it.

What is computed (the pages' statement of the method):

* The KV cache of a sequence is cut into fixed-size blocks of 16 token slots;
  a per-sequence block table records where each logical block lives in the
  physical pool ("vLLM推理引擎PagedAttention原理与性能优化实战", §2.2;
  "vLLM 是什么…", §二). The logical-to-physical map is an O(1) lookup in the
  block table ("vLLM 推理优化技术深度调研报告", 维度一.3, 公式 3). Its body is
  lost in the text we have; the reading taken here is
  block = BlockTable[s][l // P], offset = l mod P.
* Attention itself is unchanged: Softmax(Q K^T / sqrt(d)) V, with K and V
  gathered from the scattered blocks; the gather is equivalent to ordinary
  attention over the contiguous sequence ("vLLM 推理优化技术深度调研报告",
  维度一.1 误解二, 维度一.3 公式 4, 维度四.5).
* At decode time each sequence contributes one query token per query head.
  Query heads are grouped onto KV heads consecutively: q head h reads KV head
  h // (Hq / Hkv) (the pages never mention grouped heads; this is the plain
  reading). The caller passes `scale` (1/sqrt(d) in every workload here).
* A sequence of context length 0 has no softmax; its output is defined as 0.

Everything is widened to float64 before any arithmetic. Inputs are the raw
storage bits the kernels see, plus their format names (see oracle.formats).
"""
from __future__ import annotations

import numpy as np

from . import formats


def physical_slot(block_table_row, position: int, block_size: int):
    """Logical token position -> (physical block, offset within the block)."""
    return int(block_table_row[position // block_size]), position % block_size


def gather_sequence(cache_bits, block_table_row, context_len: int, kv_head: int):
    """Rows [context_len, D] of one KV head of one sequence, in logical order (raw bits)."""
    block_size = cache_bits.shape[2]
    pos = np.arange(context_len)
    blocks = np.asarray(block_table_row, dtype=np.int64)[pos // block_size]
    return cache_bits[blocks, kv_head, pos % block_size, :]


def decode_kv(bits, kv_format: str, scale: float) -> np.ndarray:
    """Stored KV bits -> float64 values. FP8 values are multiplied by their fp32 scale."""
    vals = formats.to_f64(bits, kv_format)
    if kv_format == formats.FP8_E4M3:
        vals = vals * float(np.float32(scale))
    return vals


def softmax_attention(q, K, V, scale: float) -> np.ndarray:
    """Textbook attention of query rows q [G, D] over keys K [n, D] and values V [n, D]."""
    z = scale * (q @ K.T)                        # [G, n]
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ V                                 # [G, D]


def paged_decode_attention(q_bits, k_cache_bits, v_cache_bits, block_tables, context_lens,
                           scale, q_format: str, kv_format: str,
                           k_scale: float = 1.0, v_scale: float = 1.0, seqs=None) -> np.ndarray:
    """Decode attention for the sequences in `seqs` (default: all).

    q_bits        [S, Hq, D]          raw bits of q (q_format)
    k/v_cache_bits[NB, Hkv, P, D]     raw bits of the pool (kv_format)
    block_tables  [S, max_blocks]     int
    context_lens  [S]                 int, tokens attended (the newest token included)
    Returns float64 [len(seqs), Hq, D].
    """
    q_bits = np.asarray(q_bits)
    S, Hq, D = q_bits.shape
    Hkv = k_cache_bits.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    scale = float(np.float32(scale))
    seqs = range(S) if seqs is None else list(seqs)
    out = np.zeros((len(seqs), Hq, D), dtype=np.float64)
    for i, s in enumerate(seqs):
        ctx = int(context_lens[s])
        if ctx == 0:
            continue
        qs = formats.to_f64(q_bits[s], q_format)                  # [Hq, D]
        for g in range(Hkv):
            K = decode_kv(gather_sequence(k_cache_bits, block_tables[s], ctx, g), kv_format, k_scale)
            V = decode_kv(gather_sequence(v_cache_bits, block_tables[s], ctx, g), kv_format, v_scale)
            out[i, g * G:(g + 1) * G] = softmax_attention(qs[g * G:(g + 1) * G], K, V, scale)
    return out


# --- split over context partitions -------------------------------------------------
# The pages give no split of one sequence's context; the kernels split long
# contexts into partitions and merge them. The merge is an identity of softmax,
# written out here so the tests can pin it against the unsplit definition.

def partition_stats(q, K, V, scale: float):
    """Unnormalised softmax pieces of one context partition: (max m, sum l, weighted sum o)."""
    z = scale * (q @ K.T)
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    return m, e.sum(axis=1), e @ V


def merge_partitions(ms, ls, os_):
    """Combine partition pieces: M = max m_p, out = sum e^(m_p-M) o_p / sum e^(m_p-M) l_p."""
    ms = np.asarray(ms)
    M = ms.max(axis=0)
    w = np.exp(ms - M)
    num = sum(w[p][:, None] * os_[p] for p in range(len(os_)))
    den = (w * np.asarray(ls)).sum(axis=0)
    return num / den[:, None]


# --- prefill chunks ------------------------------------------------------------------
# Long prompts are cut into chunks that are run between decode steps
# ("vLLM推理引擎PagedAttention原理与性能优化实战", §六); the prefill phase is the
# compute-bound part of a request's latency ("vLLM 推理优化技术深度调研报告", 维度一.3
# 公式 5). The pages state no formula for a chunk. The plain reading taken here: a chunk
# of n new tokens is the last n positions of the sequence's context, its K/V are already
# in the cache, and new token i (position ctx - n + i) attends to positions 0 .. ctx - n + i,
# i.e. ordinary causal attention over the whole context so far.

def paged_prefill_attention(q_bits, k_cache_bits, v_cache_bits, block_tables, context_lens,
                            query_start_loc, scale, q_format: str, kv_format: str,
                            k_scale: float = 1.0, v_scale: float = 1.0, seqs=None) -> np.ndarray:
    """Causal attention of each sequence's chunk of new tokens over its paged context.

    q_bits          [T, Hq, D]        raw bits of the new tokens' queries, sequences back to back
    query_start_loc [S + 1]           sequence s owns rows [qsl[s], qsl[s+1]) of q
    context_lens    [S]               int, context length after the chunk (chunk included)
    Returns float64 [T, Hq, D]; rows of sequences outside `seqs` (default: all) stay 0.
    """
    q_bits = np.asarray(q_bits)
    T, Hq, D = q_bits.shape
    Hkv = k_cache_bits.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    S = len(context_lens)
    if len(qsl) != S + 1 or qsl[0] != 0 or qsl[-1] > T or np.any(np.diff(qsl) < 0):
        raise ValueError("query_start_loc must rise from 0 and end within the query rows")
    scale = float(np.float32(scale))
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        ctx, first, n = int(context_lens[s]), int(qsl[s]), int(qsl[s + 1] - qsl[s])
        if n > ctx:
            raise ValueError(f"sequence {s}: chunk of {n} tokens exceeds its context of {ctx}")
        if n == 0:
            continue
        prefix = ctx - n
        qs = formats.to_f64(q_bits[first:first + n], q_format)          # [n, Hq, D]
        for g in range(Hkv):
            K = decode_kv(gather_sequence(k_cache_bits, block_tables[s], ctx, g), kv_format, k_scale)
            V = decode_kv(gather_sequence(v_cache_bits, block_tables[s], ctx, g), kv_format, v_scale)
            for i in range(n):
                seen = prefix + i + 1
                out[first + i, g * G:(g + 1) * G] = softmax_attention(qs[i, g * G:(g + 1) * G],
                                                                       K[:seen], V[:seen], scale)
    return out
