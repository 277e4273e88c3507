"""Paged KV-cache decode attention for AMD Instinct MI355X (gfx950).

Hand-written HIP kernels behind the C ABI of libpkv.so (include/pkv.h); this package
is the thin torch binding over it. No CPU fallback exists.
"""
from .ops import (PkvError, copy_blocks, decode_step, paged_attention_decode, partition_tokens,  # noqa: F401
                  reshape_and_cache, workspace_size)

__all__ = ["PkvError", "paged_attention_decode", "reshape_and_cache", "copy_blocks", "decode_step",
           "workspace_size", "partition_tokens"]
