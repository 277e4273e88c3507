"""Seeded synthetic decode workloads shared by the tests, the smoke check and the benchmark.

Holds only random draws and block bookkeeping; none of the attention,
quantisation or cache-write arithmetic lives here.
"""
from .configs import ALL_CONFIGS, BLOCK_SIZE_CONFIGS, CONFIGS, PREFILL_CONFIGS, SHARD_CONFIGS, WorkloadConfig  # noqa: F401
from .gen import Batch, Layout, make_batch, make_layout  # noqa: F401
from .swap import SWAP_CONFIGS, SwapConfig, make_swap_pairs, make_swap_pools  # noqa: F401
