"""Python binding of libpkv.so over torch tensors: argument marshalling only.

Every step of the hot path runs in the HIP kernels behind the C ABI; this module
reads shapes, dtypes and device pointers off torch tensors and raises PkvError on a
non-zero status. torch supplies device memory and the current HIP stream.
"""
from __future__ import annotations

import ctypes
import functools

import torch

from . import _lib
from ._lib import PKV_BF16, PKV_F16, PKV_FP8_E4M3


class PkvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.load().pkv_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


_DT = {torch.float16: PKV_F16, torch.bfloat16: PKV_BF16, torch.uint8: PKV_FP8_E4M3,
       torch.float8_e4m3fn: PKV_FP8_E4M3}


def _dtype(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _dev(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("pkv kernels need device tensors")
        if not t.is_contiguous():
            raise ValueError("pkv kernels need contiguous tensors")


def _workspace(workspace, need: int, device):
    """The decode workspace: the caller's (a contiguous uint8 device tensor of at least
    `need` bytes) or a fresh one; (pointer, bytes), or (None, 0) when none is needed."""
    if workspace is None:
        if not need:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    _dev(workspace)
    if workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor")
    return workspace.data_ptr(), workspace.numel()


# torch.cuda.current_stream() builds a Stream object on every call (about 2.7 µs on the
# MI355X host, a fifth of a small decode step's host time); torch's C accessor returns the
# raw handle of the same stream, where this torch has it.
_current_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> int:
    if stream is None:
        if _current_raw_stream is not None:
            return _current_raw_stream(torch.cuda.current_device())
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PkvError(fn, status)


def partition_tokens(num_seqs: int, num_q_heads: int, num_kv_heads: int, max_context_len: int,
                     partition_size: int = 0) -> int:
    r = _lib.load().pkv_decode_partition_tokens(num_seqs, num_q_heads, num_kv_heads, max_context_len, partition_size)
    if r < 0:
        raise PkvError("pkv_decode_partition_tokens", r)
    return r


@functools.lru_cache(maxsize=256)
def workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int, max_context_len: int,
                   partition_size: int = 0) -> int:
    # (a pure function of its arguments, asked on every decode call: cached)
    return _lib.load().pkv_paged_attention_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                          max_context_len, partition_size)


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                           max_context_len: int, k_scale: float = 1.0, v_scale: float = 1.0,
                           partition_size: int = 0, workspace: torch.Tensor | None = None, stream=None):
    """out[s, h] = softmax(scale * K_s q[s, h]) V_s over the paged cache (see pkv_paged_attention_decode)."""
    _dev(out, q, k_cache, v_cache, block_tables, context_lens)
    S, Hq, D = q.shape
    NB, Hkv, P, D2 = k_cache.shape
    if tuple(out.shape) != (S, Hq, D) or tuple(v_cache.shape) != tuple(k_cache.shape) or D2 != D:
        raise ValueError("shape mismatch")
    if out.dtype != q.dtype or v_cache.dtype != k_cache.dtype:
        raise ValueError("dtype mismatch")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables / context_lens shape mismatch")
    ws_ptr, ws_bytes = _workspace(workspace, workspace_size(S, Hq, Hkv, D, max_context_len, partition_size),
                                  q.device)
    st = _lib.load().pkv_paged_attention_decode(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), S, Hq, Hkv, D, P, NB, block_tables.shape[1], max_context_len,
        _dtype(q), _dtype(k_cache), scale, k_scale, v_scale, 0, partition_size, ws_ptr, ws_bytes,
        _stream(stream))
    _check("pkv_paged_attention_decode", st)
    return out


def gather_probe(k_cache, v_cache, block_tables, context_lens, max_context_len: int, sink: torch.Tensor,
                 stream=None):
    """Measurement aid: read the bytes a decode step over this batch reads, XOR them into
    sink [num_seqs, num_kv_heads] int32 (see pkv_gather_probe)."""
    _dev(k_cache, v_cache, block_tables, context_lens, sink)
    NB, Hkv, P, D = k_cache.shape
    S = context_lens.shape[0]
    if tuple(v_cache.shape) != tuple(k_cache.shape) or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache / v_cache mismatch")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or sink.dtype != torch.int32:
        raise ValueError("block_tables, context_lens and sink must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(sink.shape) != (S, Hkv):
        raise ValueError("block_tables / sink shape mismatch")
    st = _lib.load().pkv_gather_probe(
        k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), S, Hkv, D, P, NB,
        block_tables.shape[1], max_context_len, _dtype(k_cache), sink.data_ptr(), _stream(stream))
    _check("pkv_gather_probe", st)
    return sink


def _step_checks(out, q, k_cache, v_cache, key, value, slot_mapping, block_tables, context_lens):
    _dev(out, q, k_cache, v_cache, key, value, slot_mapping, block_tables, context_lens)
    S, Hq, D = q.shape
    NB, Hkv, P, D2 = k_cache.shape
    if tuple(out.shape) != (S, Hq, D) or tuple(v_cache.shape) != tuple(k_cache.shape) or D2 != D:
        raise ValueError("shape mismatch")
    if tuple(key.shape) != (S, Hkv, D) or tuple(value.shape) != (S, Hkv, D):
        raise ValueError("key/value must be [num_seqs, num_kv_heads, head_dim]")
    if out.dtype != q.dtype or v_cache.dtype != k_cache.dtype or key.dtype != q.dtype or value.dtype != q.dtype:
        raise ValueError("dtype mismatch")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (S,):
        raise ValueError("slot_mapping must be int64 [num_seqs]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables / context_lens shape mismatch")
    return S, Hq, Hkv, D, P, NB


def _cow_ptr(cow_src, S: int):
    """Device address of the per-sequence copy-on-write sources (int32 [num_seqs]), or None."""
    if cow_src is None:
        return None
    _dev(cow_src)
    if cow_src.dtype != torch.int32 or tuple(cow_src.shape) != (S,):
        raise ValueError("cow_src must be int32 [num_seqs]")
    return cow_src.data_ptr()


def decode_step(out, q, k_cache, v_cache, key, value, slot_mapping, block_tables, context_lens, scale: float,
                max_context_len: int, k_scale: float = 1.0, v_scale: float = 1.0, partition_size: int = 0,
                workspace: torch.Tensor | None = None, stream=None, cow_src: torch.Tensor | None = None):
    """Cache write of every sequence's new token, then decode attention, in one launch
    (same results as reshape_and_cache followed by paged_attention_decode). With cow_src
    (int32 [num_seqs], -1: none), the block holding sequence s's last position first becomes
    a copy of block cow_src[s] (same results as copy_blocks of those pairs beforehand)."""
    S, Hq, Hkv, D, P, NB = _step_checks(out, q, k_cache, v_cache, key, value, slot_mapping, block_tables,
                                        context_lens)
    cow = _cow_ptr(cow_src, S)
    ws_ptr, ws_bytes = _workspace(workspace, workspace_size(S, Hq, Hkv, D, max_context_len, partition_size),
                                  q.device)
    st = _lib.load().pkv_decode_step(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), key.data_ptr(), value.data_ptr(),
        slot_mapping.data_ptr(), cow, block_tables.data_ptr(), context_lens.data_ptr(), S, Hq, Hkv, D, P, NB,
        block_tables.shape[1], max_context_len, _dtype(q), _dtype(k_cache), scale, k_scale, v_scale, 0, 0, 0,
        partition_size, ws_ptr, ws_bytes, _stream(stream))
    _check("pkv_decode_step", st)
    return out


def decode_step_no_alloc(out, q, k_cache, v_cache, key, value, slot_mapping, block_tables, context_lens,
                         scale: float, max_context_len: int, k_scale: float = 1.0, v_scale: float = 1.0,
                         partition_size: int = 0, stream=None, cow_src: torch.Tensor | None = None):
    """decode_step without a workspace and without any allocation, by this binding or the
    library: split-context partials go to the library's fixed scratch array of the GPU
    (see pkv_decode_step_no_alloc; calls that overlap in time on one GPU race)."""
    S, Hq, Hkv, D, P, NB = _step_checks(out, q, k_cache, v_cache, key, value, slot_mapping, block_tables,
                                        context_lens)
    cow = _cow_ptr(cow_src, S)
    st = _lib.load().pkv_decode_step_no_alloc(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), key.data_ptr(), value.data_ptr(),
        slot_mapping.data_ptr(), cow, block_tables.data_ptr(), context_lens.data_ptr(), S, Hq, Hkv, D, P, NB,
        block_tables.shape[1], max_context_len, _dtype(q), _dtype(k_cache), scale, k_scale, v_scale, 0, 0, 0,
        partition_size, _stream(stream))
    _check("pkv_decode_step_no_alloc", st)
    return out


def paged_attention_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale: float,
                            max_query_len: int, k_scale: float = 1.0, v_scale: float = 1.0, stream=None):
    """Causal attention of each sequence's chunk of new tokens (rows query_start_loc[s] ..
    query_start_loc[s+1] of q) over its paged context (see pkv_paged_attention_prefill)."""
    _dev(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc)
    T, Hq, D = q.shape
    NB, Hkv, P, D2 = k_cache.shape
    S = context_lens.shape[0]
    if tuple(out.shape) != (T, Hq, D) or tuple(v_cache.shape) != tuple(k_cache.shape) or D2 != D:
        raise ValueError("shape mismatch")
    if out.dtype != q.dtype or v_cache.dtype != k_cache.dtype:
        raise ValueError("dtype mismatch")
    for name, t in (("block_tables", block_tables), ("context_lens", context_lens),
                    ("query_start_loc", query_start_loc)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or query_start_loc.shape != (S + 1,):
        raise ValueError("block_tables / query_start_loc shape mismatch")
    st = _lib.load().pkv_paged_attention_prefill(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), query_start_loc.data_ptr(), S, T, Hq, Hkv, D, P, NB, block_tables.shape[1],
        max_query_len, _dtype(q), _dtype(k_cache), scale, k_scale, v_scale, 0, _stream(stream))
    _check("pkv_paged_attention_prefill", st)
    return out


def reshape_and_cache(key, value, slot_mapping, k_cache, v_cache, k_scale: float = 1.0, v_scale: float = 1.0,
                      stream=None) -> None:
    """Write key/value [T, Hkv, D] rows into their slots of one layer's caches."""
    _dev(key, value, slot_mapping, k_cache, v_cache)
    T, Hkv, D = key.shape
    NB, Hkv2, P, D2 = k_cache.shape
    if tuple(value.shape) != (T, Hkv, D) or Hkv2 != Hkv or D2 != D or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    if value.dtype != key.dtype or v_cache.dtype != k_cache.dtype:
        raise ValueError("dtype mismatch")
    st = _lib.load().pkv_reshape_and_cache(
        key.data_ptr(), value.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        T, Hkv, D, P, NB, _dtype(key), _dtype(k_cache), k_scale, v_scale, 0, 0, _stream(stream))
    _check("pkv_reshape_and_cache", st)


def copy_blocks(k_caches, v_caches, src_dst_pairs, stream=None) -> None:
    """For each (src, dst) pair and layer: cache[dst] = cache[src], K and V."""
    if len(k_caches) != len(v_caches):
        raise ValueError("k_caches and v_caches differ in length")
    _dev(src_dst_pairs, *k_caches, *v_caches)
    if src_dst_pairs.dtype != torch.int64 or src_dst_pairs.dim() != 2 or src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be int64 [num_pairs, 2]")
    ref = k_caches[0]
    for c in (*k_caches, *v_caches):
        if c.shape != ref.shape or c.dtype != ref.dtype:
            raise ValueError("all caches must share shape and dtype")
    n = len(k_caches)
    kp = (ctypes.c_void_p * n)(*[c.data_ptr() for c in k_caches])
    vp = (ctypes.c_void_p * n)(*[c.data_ptr() for c in v_caches])
    block_bytes = ref[0].numel() * ref.element_size()
    st = _lib.load().pkv_copy_blocks(kp, vp, n, src_dst_pairs.data_ptr(), src_dst_pairs.shape[0], block_bytes,
                                     ref.shape[0], _stream(stream))
    _check("pkv_copy_blocks", st)


def swap_blocks(src_k_caches, src_v_caches, dst_k_caches, dst_v_caches, src_dst_pairs, stream=None) -> None:
    """For each (src, dst) pair and layer: dst pool[dst] = src pool[src], K and V. One side is
    the GPU pool, the other a pool in pinned host memory (torch pin_memory=True)."""
    n = len(src_k_caches)
    if not (len(src_v_caches) == len(dst_k_caches) == len(dst_v_caches) == n):
        raise ValueError("the four pool lists differ in length")
    if not src_dst_pairs.is_cuda and not src_dst_pairs.is_pinned():
        raise ValueError("src_dst_pairs must be a device tensor or pinned host memory")
    if src_dst_pairs.dtype != torch.int64 or src_dst_pairs.dim() != 2 or src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be int64 [num_pairs, 2]")
    src, dst = src_k_caches[0], dst_k_caches[0]
    for pools, ref in ((src_k_caches, src), (src_v_caches, src), (dst_k_caches, dst), (dst_v_caches, dst)):
        for c in pools:
            if not (c.is_cuda or c.is_pinned()):
                raise ValueError("pools must be device tensors or pinned host tensors")
            if not c.is_contiguous():
                raise ValueError("pools must be contiguous")
            if c.shape[1:] != ref.shape[1:] or c.dtype != ref.dtype or c.shape[0] != ref.shape[0]:
                raise ValueError("pools on one side must share shape and dtype")
    if src.shape[1:] != dst.shape[1:] or src.dtype != dst.dtype:
        raise ValueError("source and destination blocks differ in shape or dtype")
    ptrs = lambda ts: (ctypes.c_void_p * n)(*[t.data_ptr() for t in ts])
    block_bytes = src[0].numel() * src.element_size()
    st = _lib.load().pkv_swap_blocks(ptrs(src_k_caches), ptrs(src_v_caches), ptrs(dst_k_caches), ptrs(dst_v_caches),
                                     n, src_dst_pairs.data_ptr(), src_dst_pairs.shape[0], block_bytes,
                                     src.shape[0], dst.shape[0], _stream(stream))
    _check("pkv_swap_blocks", st)


CHECKS = {0: "ok", 1: "context_len", 2: "block_id", 3: "slot_range", 4: "slot_duplicate", 5: "slot_not_last",
          6: "slot_shared_block", 7: "pair_range", 8: "pair_duplicate_dst", 9: "pair_dst_is_src",
          10: "cow_range", 11: "cow_no_context", 12: "cow_shared_dst", 13: "cow_dst_is_src", 14: "cow_src_written"}


def validate_inputs(num_blocks: int, block_tables=None, context_lens=None, slot_mapping=None, src_dst_pairs=None,
                    block_size: int = 16, decode_step: bool = False, stream=None,
                    cow_src=None) -> tuple[str, int, int]:
    """Debug check of the values in the index buffers (see include/pkv_validate.h).

    Returns (check, index, value): ("ok", -1, 0), or the name of the first failed check with
    where it failed and the offending value. Tensors on the GPU go through
    pkv_validate_inputs (copied to the host on `stream`), CPU tensors through
    pkv_validate_inputs_host; all given tensors must be on the same side.
    """
    given = [t for t in (block_tables, context_lens, slot_mapping, src_dst_pairs, cow_src) if t is not None]
    on_gpu = {bool(t.is_cuda) for t in given}
    if len(on_gpu) > 1:
        raise ValueError("index tensors must all be on the GPU or all on the CPU")
    for t, dt, name in ((block_tables, torch.int32, "block_tables"), (context_lens, torch.int32, "context_lens"),
                        (slot_mapping, torch.int64, "slot_mapping"), (src_dst_pairs, torch.int64, "src_dst_pairs"),
                        (cow_src, torch.int32, "cow_src")):
        if t is not None and (t.dtype != dt or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous {dt} tensor")
    S = context_lens.shape[0] if context_lens is not None else 0
    if cow_src is not None and tuple(cow_src.shape) != (S,):
        raise ValueError("cow_src must be int32 [num_seqs]")
    maxb = block_tables.shape[1] if block_tables is not None and block_tables.dim() == 2 else 0
    T = slot_mapping.shape[0] if slot_mapping is not None else 0
    n_pairs = src_dst_pairs.shape[0] if src_dst_pairs is not None else 0

    def ptr(t):
        return t.data_ptr() if t is not None else None

    res = _lib.Validation()
    lib = _lib.load()
    common = (ptr(block_tables), ptr(context_lens), S, maxb, block_size, num_blocks, ptr(slot_mapping), T,
              1 if decode_step else 0, ptr(cow_src), ptr(src_dst_pairs), n_pairs)
    if on_gpu == {True}:
        st = lib.pkv_validate_inputs(*common, _stream(stream), ctypes.byref(res))
        _check("pkv_validate_inputs", st)
    else:
        st = lib.pkv_validate_inputs_host(*common, ctypes.byref(res))
        _check("pkv_validate_inputs_host", st)
    return CHECKS.get(res.check, str(res.check)), int(res.index), int(res.value)
