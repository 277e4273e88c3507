"""Seeded synthetic inputs for the decode workloads.

This module only draws random numbers and lays out blocks; it holds none of the
attention, quantisation or cache-write arithmetic. Both the HIP path and the
oracle consume what it produces.

Recipe (one numpy SeedSequence per workload and replica for the block layout, one
torch generator per tensor for the values):

* context lengths: fixed, or uniform integers in [lo, hi]; the length counts the
  new token of this decode step.
* placement: the pool hands out blocks in a seeded random permutation, so each
  sequence's logical blocks are scattered over the pool. One extra block is
  reserved as a poison block; block-table entries past a sequence's last block
  point at it.
* beam search: per request a 4096-token prompt is forked into `width` parent
  beams (prompt blocks shared), each parent grows a private tail of U[lo, hi]
  tokens, then beam selection picks `width` children by drawing parents with
  replacement; children share their parent's blocks. The decode step's write of
  the new token then copies every still-shared partial last block (copy-on-write).
* values: q, the new token's K/V, and the pool's history slots are N(0, 1) drawn
  in fp32 and rounded to the stored 16-bit type. An fp8 pool is drawn as codes:
  random sign, exponent field 15 - G with G ~ Geometric(1/2) (clamped to [0, 14]),
  uniform 3-bit mantissa, never the NaN code; with the 1/128 scale about half the
  magnitudes fall in [1, 1.875).
* every slot that holds no history before the step (unused pool blocks, tails of
  last blocks, the new token's slot, fresh copy-on-write targets) is filled with
  NaN, as stale reused memory would be.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .blocks import BlockPool, Sequence
from .configs import WorkloadConfig

TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}
BITS_DTYPE = {"f16": torch.int16, "bf16": torch.int16, "fp8_e4m3": torch.uint8}
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0, "fp8_e4m3": 0x7F}
ELEM_BYTES = {"f16": 2, "bf16": 2, "fp8_e4m3": 1}


@dataclass
class Layout:
    """Where every token of a decode batch lives (host numpy arrays)."""
    block_tables: np.ndarray      # int32 [S, max_blocks], padded with poison_block
    context_lens: np.ndarray      # int32 [S], after the step's new tokens
    slot_mapping: np.ndarray      # int64 [T], slot of each of the step's new tokens
    copy_pairs: np.ndarray        # int64 [Pn, 2], copy-on-write (src, dst) of this step
    history_valid: np.ndarray     # bool [NB, P], slots holding KV before the step
    poison_block: int
    query_start_loc: np.ndarray   # int32 [S + 1]: sequence s's new tokens are rows [qsl[s], qsl[s+1])
    cow_src: np.ndarray           # int32 [S]: source of the copy-on-write pair whose destination is
                                  # the block sequence s writes into this step, -1: none


def _seed_streams(cfg: WorkloadConfig, replica: int, n: int):
    ss = np.random.SeedSequence([cfg.seed, replica])
    return [np.random.default_rng(s) for s in ss.spawn(n)]


def _chunk_lens(cfg: WorkloadConfig, ctx, rng) -> np.ndarray:
    """New tokens per sequence this step (1 for a decode step), never more than the context."""
    if not cfg.chunk:
        return np.ones(len(ctx), dtype=np.int64)
    if cfg.chunk[0] == "fixed":
        n = np.full(len(ctx), int(cfg.chunk[1]), dtype=np.int64)
    elif cfg.chunk[0] == "uniform":
        n = rng.integers(cfg.chunk[1], cfg.chunk[2] + 1, size=len(ctx))
    else:
        raise ValueError(f"unknown chunk kind {cfg.chunk[0]!r}")
    return np.minimum(n, np.asarray(ctx, dtype=np.int64))


def make_layout(cfg: WorkloadConfig, replica: int = 0) -> Layout:
    rng_ctx, rng_place, rng_tail, rng_parent, rng_chunk = _seed_streams(cfg, replica, 5)
    P = cfg.block_size
    pool = BlockPool(cfg.num_blocks, P, order=rng_place.permutation(cfg.num_blocks))
    poison = pool.allocate()
    history: list[list[int]] = []
    live: list[Sequence] = []
    kind = cfg.ctx[0]
    if kind in ("fixed", "uniform"):
        if kind == "fixed":
            ctx = np.asarray(cfg.ctx[1], dtype=np.int64)
        else:
            ctx = rng_ctx.integers(cfg.ctx[1], cfg.ctx[2] + 1, size=cfg.num_seqs)
        if len(ctx) != cfg.num_seqs:
            raise ValueError("context list does not match num_seqs")
        new_tokens = _chunk_lens(cfg, ctx, rng_chunk)
        for c, q in zip(ctx, new_tokens):
            seq = Sequence(pool)
            slots, copies = seq.extend(max(int(c) - int(q), 0))   # the history before the step
            assert not copies
            history.append(slots)
            live.append(seq)
    elif kind == "beam":
        if cfg.chunk:
            raise ValueError("beam workloads decode one token per sequence")
        new_tokens = None
        prompt, tail_lo, tail_hi, width = cfg.ctx[1:]
        if cfg.num_seqs % width:
            raise ValueError("num_seqs must be a multiple of the beam width")
        for _ in range(cfg.num_seqs // width):
            root = Sequence(pool)
            prompt_slots, copies = root.extend(prompt)
            assert not copies
            parents = [root.fork() for _ in range(width)]
            root.free()
            parent_slots = []
            for p in parents:
                slots, copies = p.extend(int(rng_tail.integers(tail_lo, tail_hi + 1)))
                if copies:
                    raise ValueError("prompt must end on a block boundary")
                parent_slots.append(prompt_slots + slots)
            picks = rng_parent.integers(0, width, size=width)
            for k in picks:
                live.append(parents[k].fork())
                history.append(parent_slots[k])
            for p in parents:
                p.free()
    else:
        raise ValueError(f"unknown context kind {kind!r}")

    valid = np.zeros(cfg.num_blocks * P, dtype=bool)
    for slots in history:
        valid[np.asarray(slots, dtype=np.int64)] = True

    S = len(live)
    if new_tokens is None:
        new_tokens = np.ones(S, dtype=np.int64)
    query_start_loc = np.zeros(S + 1, dtype=np.int32)
    query_start_loc[1:] = np.cumsum(new_tokens)
    slot_mapping = np.empty(int(query_start_loc[-1]), dtype=np.int64)
    pairs = []
    cow_src = np.full(S, -1, dtype=np.int32)
    for i, seq in enumerate(live):
        for k in range(int(new_tokens[i])):
            slot, copy = seq.append_slot()
            slot_mapping[query_start_loc[i] + k] = slot
            if copy is not None:
                pairs.append(copy)
                cow_src[i] = copy[0]
    block_tables = np.full((S, cfg.max_blocks_per_seq), poison, dtype=np.int32)
    context_lens = np.empty(S, dtype=np.int32)
    for i, seq in enumerate(live):
        if len(seq.blocks) > cfg.max_blocks_per_seq:
            raise ValueError("sequence longer than max_context_len")
        block_tables[i, :len(seq.blocks)] = seq.blocks
        context_lens[i] = seq.num_tokens
    copy_pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    return Layout(block_tables, context_lens, slot_mapping, copy_pairs,
                  valid.reshape(cfg.num_blocks, P), poison, query_start_loc, cow_src)


@dataclass
class Batch:
    """One decode step's inputs, as torch tensors on one device."""
    cfg: WorkloadConfig
    layout: Layout
    q: torch.Tensor              # [T, Hq, D] dtype: the step's new tokens (T = S for a decode step)
    new_k: torch.Tensor          # [T, Hkv, D] dtype
    new_v: torch.Tensor          # [T, Hkv, D] dtype
    k_cache: torch.Tensor        # [NB, Hkv, P, D] kv dtype (uint8 codes for fp8)
    v_cache: torch.Tensor
    block_tables: torch.Tensor   # int32 [S, max_blocks]
    context_lens: torch.Tensor   # int32 [S]
    slot_mapping: torch.Tensor   # int64 [T]
    copy_pairs: torch.Tensor     # int64 [Pn, 2]
    query_start_loc: torch.Tensor  # int32 [S + 1]
    cow_src: torch.Tensor        # int32 [S]

    @property
    def scale(self) -> float:
        return self.cfg.scale

    @property
    def k_scale(self) -> float:
        return self.cfg.kv_scale

    @property
    def v_scale(self) -> float:
        return self.cfg.kv_scale


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, dtype, device, seed):
    x = torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)
    return x.to(dtype)


def _fp8_codes(shape, device, seed):
    g = _gen(device, seed)
    sign = torch.randint(0, 2, shape, generator=g, device=device, dtype=torch.int32)
    geo = torch.empty(shape, device=device, dtype=torch.float32).geometric_(0.5, generator=g)
    # geometric_ can return 0 (its uniform draw may be exactly 1), so clamp both ends:
    # exponent field 14 at most keeps every code finite (0x7F/0xFF are NaN).
    exp_field = (15 - geo.to(torch.int32)).clamp_(min=0, max=14)
    mant = torch.randint(0, 8, shape, generator=g, device=device, dtype=torch.int32)
    return ((sign << 7) | (exp_field << 3) | mant).to(torch.uint8)


def make_pool(cfg: WorkloadConfig, valid: np.ndarray, device, seed: int) -> torch.Tensor:
    shape = (cfg.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim)
    if cfg.kv_dtype == "fp8_e4m3":
        pool = _fp8_codes(shape, device, seed)
    else:
        pool = _normal(shape, TORCH_DTYPE[cfg.kv_dtype], device, seed)
    stale = torch.from_numpy(~valid).to(device)[:, None, :, None].expand(shape)
    pool.view(BITS_DTYPE[cfg.kv_dtype]).masked_fill_(stale, NAN_BITS[cfg.kv_dtype])
    return pool


def make_batch(cfg: WorkloadConfig, device="cpu", replica: int = 0) -> Batch:
    lay = make_layout(cfg, replica)
    S, Hq, Hkv, D = int(lay.query_start_loc[-1]), cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    base = (cfg.seed * 1000 + replica) * 16
    dt = TORCH_DTYPE[cfg.dtype]
    q = _normal((S, Hq, D), dt, device, base + 1)
    new_k = _normal((S, Hkv, D), dt, device, base + 2)
    new_v = _normal((S, Hkv, D), dt, device, base + 3)
    k_cache = make_pool(cfg, lay.history_valid, device, base + 4)
    v_cache = make_pool(cfg, lay.history_valid, device, base + 5)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return Batch(cfg, lay, q, new_k, new_v, k_cache, v_cache, t(lay.block_tables), t(lay.context_lens),
                 t(lay.slot_mapping), t(lay.copy_pairs), t(lay.query_start_loc), t(lay.cow_src))


def kv_bytes_logical(cfg: WorkloadConfig, context_lens) -> int:
    """KV bytes one decode step reads if every sequence's context is read once."""
    return int(np.asarray(context_lens, dtype=np.int64).sum()) * 2 * cfg.num_kv_heads * cfg.head_dim \
        * ELEM_BYTES[cfg.kv_dtype]


def kv_bytes_unique(cfg: WorkloadConfig, layout: Layout) -> int:
    """KV bytes of the distinct physical token slots one decode step reads."""
    P = cfg.block_size
    seen = set()
    for row, ctx in zip(layout.block_tables, layout.context_lens):
        nfull, rem = divmod(int(ctx), P)
        for j in range(nfull):
            seen.add((int(row[j]), P))
        if rem:
            seen.add((int(row[nfull]), rem))
    per_block = {}
    for b, n in seen:
        per_block[b] = max(per_block.get(b, 0), n)
    slots = sum(per_block.values())
    return slots * 2 * cfg.num_kv_heads * cfg.head_dim * ELEM_BYTES[cfg.kv_dtype]
