"""Cache writes and copy-on-write block copies, as their definitions.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg use it.

* Writing a new token: each decoded token's K and V rows go into the slot the
  block manager gave it; a new physical block is taken only when the current one
  is full ("vLLM 是什么…", §二). A slot is the flat index block * P + offset of the
  pool; a negative slot means "no write" (a padded batch row). For an FP8 cache
  the row is quantised on the way in: code = encode(fl32(x / scale)).
* Copy-on-write: sequences that share a block point their block tables at the
  same physical block, which is then read-only; the first write to it takes a
  fresh block, copies the old contents there and writes the copy
  ("vLLM推理引擎PagedAttention原理与性能优化实战", §3.2). The copy covers the whole
  block, K and V, for every layer's cache.
* Swapping: under memory pressure whole blocks are moved to CPU memory and back
  ("vLLM 是什么…", §五 误解三; the scheduler reclaims a preempted request's blocks,
  "vLLM推理引擎PagedAttention原理与性能优化实战", §四). A swap copies whole blocks, K and V,
  every layer, from one pool (GPU or host) into another; the block ids on the two sides
  are independent.
"""
from __future__ import annotations

import numpy as np

from . import formats


def quantize_row(bits, in_format: str, kv_format: str, scale: float) -> np.ndarray:
    """One token row as the cache stores it."""
    bits = np.asarray(bits)
    if kv_format == in_format:
        return bits.astype(formats.STORAGE[kv_format])
    if kv_format == formats.FP8_E4M3 and in_format in (formats.F16, formats.BF16):
        x = formats.to_f64(bits, in_format)
        return formats.e4m3_encode(formats.round_to_f32(x / float(np.float32(scale))))
    raise ValueError(f"cannot store {in_format} into a {kv_format} cache")


def reshape_and_cache(k_bits, v_bits, slot_mapping, k_cache_bits, v_cache_bits,
                      in_format: str, kv_format: str, k_scale: float = 1.0, v_scale: float = 1.0):
    """Return (k_cache, v_cache) after writing tokens [T, Hkv, D] into their slots.

    The input caches are not modified; the result is a copy.
    """
    k_out = np.array(k_cache_bits, copy=True)
    v_out = np.array(v_cache_bits, copy=True)
    block_size = k_out.shape[2]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        block, offset = int(slot) // block_size, int(slot) % block_size
        k_out[block, :, offset, :] = quantize_row(k_bits[i], in_format, kv_format, k_scale)
        v_out[block, :, offset, :] = quantize_row(v_bits[i], in_format, kv_format, v_scale)
    return k_out, v_out


def copy_blocks(k_caches, v_caches, src_dst_pairs):
    """Return copies of every layer's (k, v) cache with block dst := block src for each pair."""
    k_out = [np.array(k, copy=True) for k in k_caches]
    v_out = [np.array(v, copy=True) for v in v_caches]
    for src, dst in np.asarray(src_dst_pairs, dtype=np.int64).reshape(-1, 2):
        for layer in range(len(k_out)):
            k_out[layer][dst] = k_caches[layer][src]
            v_out[layer][dst] = v_caches[layer][src]
    return k_out, v_out


def swap_blocks(src_k, src_v, dst_k, dst_v, src_dst_pairs):
    """Return copies of every layer's destination (k, v) pools with dst[layer][d] := src[layer][s]
    for each pair (s, d). Source and destination are different pools (one on the GPU, one
    in host memory); their block counts may differ."""
    k_out = [np.array(k, copy=True) for k in dst_k]
    v_out = [np.array(v, copy=True) for v in dst_v]
    for src, dst in np.asarray(src_dst_pairs, dtype=np.int64).reshape(-1, 2):
        for layer in range(len(k_out)):
            k_out[layer][dst] = src_k[layer][src]
            v_out[layer][dst] = src_v[layer][src]
    return k_out, v_out
