"""Plain, slow CPU oracle of the paged decode-attention hot path (float64, numpy).

TEST INFRASTRUCTURE ONLY. The oracle exists to check the HIP kernels. Only
`tests/`, the smoke check in `__graft_entry__.py` and the CPU-baseline leg of
`bench.py` may import it. It shares no code with the HIP path and never imports
the product package.

Modules:
  formats    -- exact decoders for f16 / bf16 / OCP E4M3FN, the E4M3FN encoder
  attention  -- block-table gather + textbook softmax attention; split-merge identity
  cache_ops  -- writing new tokens into their slots; copy-on-write block copies

Every function is pinned by tests marked "not gpu" against closed forms,
invariants, library routines and brute force (no function here is unpinned).
"""
from . import attention, cache_ops, formats  # noqa: F401
