"""Test helpers: scatter logical K/V into a block pool; torch tensors -> raw numpy bits."""
from __future__ import annotations

import numpy as np
import torch

NAN16 = np.uint16(0x7E00)


def scatter_to_pool(seqs_bits, num_blocks, block_size, rng, fill=NAN16, perm=None):
    """Place each sequence's rows [ctx, H, D] into random pool blocks.

    Returns (pool [NB, H, P, D], block_tables [S, max_blocks] int32). Unused slots
    and blocks hold `fill`; block-table padding points at a block no sequence owns.
    """
    H, D = seqs_bits[0].shape[1], seqs_bits[0].shape[2]
    dtype = seqs_bits[0].dtype
    nblk = [-(-len(s) // block_size) for s in seqs_bits]
    need = sum(nblk) + 1
    assert need <= num_blocks
    perm = rng.permutation(num_blocks) if perm is None else np.asarray(perm)
    pool = np.full((num_blocks, H, block_size, D), fill, dtype=dtype)
    maxb = max(max(nblk), 1)
    spare = int(perm[need - 1])
    tables = np.full((len(seqs_bits), maxb), spare, dtype=np.int32)
    cursor = 0
    for s, rows in enumerate(seqs_bits):
        for j in range(nblk[s]):
            b = int(perm[cursor])
            cursor += 1
            tables[s, j] = b
            chunk = rows[j * block_size:(j + 1) * block_size]
            pool[b, :, :len(chunk), :] = np.transpose(chunk, (1, 0, 2))
    return pool, tables


def f16_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def torch_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits of a tensor as numpy (uint16 for 16-bit types, uint8 for bytes)."""
    t = t.detach().cpu().contiguous()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.element_size() == 1:
        return t.view(torch.uint8).numpy()
    return t.numpy()
