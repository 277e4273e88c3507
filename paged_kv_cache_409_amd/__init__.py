"""Paged KV-cache attention (decode steps and prefill chunks) for AMD Instinct MI355X (gfx950).

Hand-written HIP kernels behind the C ABI of libpkv.so (include/pkv.h); this package
is the thin torch binding over it. No CPU fallback exists.
"""
from .ops import (PkvError, copy_blocks, decode_step, decode_step_no_alloc, gather_probe,  # noqa: F401
                  paged_attention_decode, paged_attention_prefill, partition_tokens, reshape_and_cache, swap_blocks,
                  validate_inputs, workspace_size)

__all__ = ["PkvError", "paged_attention_decode", "reshape_and_cache", "copy_blocks", "decode_step", "decode_step_no_alloc",
           "paged_attention_prefill", "swap_blocks", "workspace_size", "partition_tokens", "gather_probe",
           "validate_inputs"]
