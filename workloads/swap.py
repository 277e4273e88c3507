"""Seeded block-swap cases: a preempted request's blocks go to host memory and come back.

When GPU memory runs out, whole blocks are moved to CPU memory and the scheduler reclaims
the blocks of preempted requests ("vLLM 是什么…", §五 误解三; "vLLM推理引擎PagedAttention原理
与性能优化实战", §四). A case holds per-layer K and V pools on both sides and two pair lists:
swap-out (scattered GPU blocks -> host blocks) and swap-in (those host blocks -> other,
freshly free GPU blocks). Values are random and carry no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .gen import ELEM_BYTES, TORCH_DTYPE, _fp8_codes, _normal


@dataclass(frozen=True)
class SwapConfig:
    name: str
    num_layers: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str
    gpu_blocks: int
    host_blocks: int
    swap_blocks: int        # blocks per layer moved each way
    seed: int
    block_size: int = 16
    description: str = ""

    @property
    def block_bytes(self) -> int:
        return self.num_kv_heads * self.block_size * self.head_dim * ELEM_BYTES[self.kv_dtype]

    @property
    def bytes_per_direction(self) -> int:
        return 2 * self.num_layers * self.swap_blocks * self.block_bytes


SWAP_TINY = SwapConfig("swap_tiny", num_layers=3, num_kv_heads=2, head_dim=64, kv_dtype="f16", gpu_blocks=64,
                       host_blocks=40, swap_blocks=20, seed=40908,
                       description="3 layers, 2 kv heads, D 64, fp16: 20 of 64 GPU blocks to a 40-block host pool")
SWAP_70B = SwapConfig("swap_70b", num_layers=8, num_kv_heads=8, head_dim=128, kv_dtype="bf16", gpu_blocks=4096,
                      host_blocks=2048, swap_blocks=1024, seed=40909,
                      description="Llama-2-70B KV shape (8 kv heads, D 128, bf16, 32 KiB blocks), 8 layers: "
                                  "1024 scattered blocks per layer (8 preempted 2048-token requests) out to "
                                  "pinned host memory and back, 512 MiB each way")
SWAP_CONFIGS = {c.name: c for c in (SWAP_TINY, SWAP_70B)}


def make_swap_pairs(cfg: SwapConfig, replica: int = 0):
    """(out_pairs, in_pairs) int64 [n, 2]: GPU -> host, then host -> other free GPU blocks."""
    if 2 * cfg.swap_blocks > cfg.gpu_blocks or cfg.swap_blocks > cfg.host_blocks:
        raise ValueError("pools too small for the swap")
    rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, replica]))
    gpu = rng.permutation(cfg.gpu_blocks)
    host = rng.permutation(cfg.host_blocks)[:cfg.swap_blocks]
    out_pairs = np.stack([gpu[:cfg.swap_blocks], host], axis=1).astype(np.int64)
    in_pairs = np.stack([host, gpu[cfg.swap_blocks:2 * cfg.swap_blocks]], axis=1).astype(np.int64)
    return out_pairs, in_pairs


def make_swap_pools(cfg: SwapConfig, side: str, device="cpu", pin: bool = False, replica: int = 0):
    """Per-layer (k, v) pools [blocks, Hkv, 16, D] of one side ("gpu" or "host"), random values
    (drawn on `device`, then pinned on the host when `pin`)."""
    nb = cfg.gpu_blocks if side == "gpu" else cfg.host_blocks
    shape = (nb, cfg.num_kv_heads, cfg.block_size, cfg.head_dim)
    base = (cfg.seed * 1000 + replica) * 256 + (0 if side == "gpu" else 128)
    pools = []
    for layer in range(cfg.num_layers):
        kv = []
        for t in range(2):
            seed = base + 2 * layer + t
            x = _fp8_codes(shape, device, seed) if cfg.kv_dtype == "fp8_e4m3" else \
                _normal(shape, TORCH_DTYPE[cfg.kv_dtype], device, seed)
            if pin:
                x = x.cpu().pin_memory()
            kv.append(x)
        pools.append(tuple(kv))
    return pools

