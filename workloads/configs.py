"""The five seeded synthetic decode workloads, one layer each.

Shapes follow the pages' workloads: a 4-token toy case, a Llama-2-7B-shaped
layer, a Llama-2-70B-shaped grouped-query layer (the 512-token-prompt,
256-token-output workload of "vLLM 推理优化技术深度调研报告", 维度一.5), a long
chain-of-thought decode ("vLLM 是什么…", §三) and beam search sharing a prompt
("vLLM推理引擎PagedAttention原理与性能优化实战", §3.1-§3.2, beam width 4, FP8
cache per §5.2). Block size 16 throughout (§2.2 of the same page).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    seed: int
    dtype: str                     # q / new-token dtype: "f16" | "bf16"
    kv_dtype: str                  # cache dtype: "f16" | "bf16" | "fp8_e4m3"
    ctx: tuple                     # ("fixed", [..]) | ("uniform", lo, hi) | ("beam", prompt, tail_lo, tail_hi, width)
                                   # context length after the step, new tokens included
    max_context_len: int
    block_size: int = 16
    partition_size: int = 0        # 0: the library picks
    kv_scale: float = 1.0          # per-tensor scale of an fp8 cache (both K and V)
    chunk: tuple = ()              # new tokens per sequence this step: () = 1 (a decode step),
                                   # ("fixed", n) or ("uniform", lo, hi) (a prefill chunk, at most the context)
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.max_context_len // self.block_size)

    @property
    def scale(self) -> float:
        return self.head_dim ** -0.5


TINY = WorkloadConfig(
    name="tiny", num_seqs=4, num_q_heads=2, num_kv_heads=2, head_dim=64, num_blocks=64,
    seed=40901, dtype="f16", kv_dtype="f16", ctx=("fixed", [1, 15, 16, 37]), max_context_len=37,
    description="4 seqs, ctx {1,15,16,37}, 2 q = 2 kv heads, D 64, fp16, 64-block pool")

LLAMA2_7B = WorkloadConfig(
    name="llama2_7b", num_seqs=64, num_q_heads=32, num_kv_heads=32, head_dim=128, num_blocks=16384,
    seed=40902, dtype="f16", kv_dtype="f16", ctx=("uniform", 128, 2048), max_context_len=2048,
    description="Llama-2-7B layer: batch 64, 32/32 heads, D 128, fp16, ctx U[128,2048], 16384-block pool")

LLAMA2_70B_GQA = WorkloadConfig(
    name="llama2_70b_gqa", num_seqs=256, num_q_heads=64, num_kv_heads=8, head_dim=128, num_blocks=16384,
    seed=40903, dtype="bf16", kv_dtype="bf16", ctx=("uniform", 512, 768), max_context_len=768,
    description="Llama-2-70B GQA layer: batch 256, 64 q / 8 kv heads, D 128, bf16, ctx U[512,768]")

LONG_COT = WorkloadConfig(
    name="long_cot", num_seqs=8, num_q_heads=32, num_kv_heads=8, head_dim=128, num_blocks=32768,
    seed=40904, dtype="bf16", kv_dtype="bf16", ctx=("fixed", [32768] * 8), max_context_len=32768,
    partition_size=512,
    description="long chain-of-thought: batch 8, 32 q / 8 kv heads, D 128, bf16, ctx 32768, 512-token partitions")

BEAM_COW = WorkloadConfig(
    name="beam_cow", num_seqs=256, num_q_heads=32, num_kv_heads=8, head_dim=128, num_blocks=32768,
    seed=40905, dtype="bf16", kv_dtype="fp8_e4m3", ctx=("beam", 4096, 0, 256, 4), max_context_len=4096 + 256 + 1,
    kv_scale=1.0 / 128.0,
    description="beam search: 64 requests x 4 beams sharing a 4096-token prompt, tails U[0,256], "
                "copy-on-write of shared partial blocks, fp8-e4m3 KV (per-tensor scale 1/128), bf16 q")

CONFIGS = {c.name: c for c in (TINY, LLAMA2_7B, LLAMA2_70B_GQA, LONG_COT, BEAM_COW)}

# Prefill chunks ("vLLM推理引擎PagedAttention原理与性能优化实战", §六): each sequence brings a
# chunk of new tokens that attend causally to its cached context and to each other.
PREFILL_TINY = WorkloadConfig(
    name="prefill_tiny", num_seqs=4, num_q_heads=4, num_kv_heads=2, head_dim=64, num_blocks=64,
    seed=40906, dtype="f16", kv_dtype="f16", ctx=("fixed", [5, 16, 37, 90]), max_context_len=90,
    chunk=("uniform", 1, 40),
    description="4 seqs, ctx {5,16,37,90}, chunks U[1,40], 4 q / 2 kv heads, D 64, fp16, 64-block pool")

PREFILL_70B_GQA = WorkloadConfig(
    name="prefill_70b_gqa", num_seqs=8, num_q_heads=64, num_kv_heads=8, head_dim=128, num_blocks=4096,
    seed=40907, dtype="bf16", kv_dtype="bf16", ctx=("uniform", 512, 4096), max_context_len=4096,
    chunk=("fixed", 512),
    description="Llama-2-70B GQA layer, chunked prefill: 8 seqs, 512-token chunks after cached "
                "prefixes of 0-3584 tokens (ctx U[512,4096]), 64 q / 8 kv heads, D 128, bf16")

# The same batch with an FP8 cache ("vLLM推理引擎PagedAttention原理与性能优化实战", §5.2), served
# by the kernel that widens fp8 tiles on their way into LDS.
PREFILL_70B_GQA_FP8 = replace(PREFILL_70B_GQA, name="prefill_70b_gqa_fp8", kv_dtype="fp8_e4m3", kv_scale=1.0 / 128.0,
                              description="Llama-2-70B GQA layer, chunked prefill as prefill_70b_gqa, with an "
                                          "fp8-e4m3 cache (per-tensor scale 1/128), bf16 q")

PREFILL_CONFIGS = {c.name: c for c in (PREFILL_TINY, PREFILL_70B_GQA, PREFILL_70B_GQA_FP8)}

# The block-size question of "vLLM 推理优化技术深度调研报告", 维度四.5 (bigger pages: fewer
# table entries, more internal fragmentation): the Llama-2-70B GQA decode layer with
# 32- and 64-token blocks, the same seed (the same contexts) and the same pool bytes.
LLAMA2_70B_GQA_P32 = replace(LLAMA2_70B_GQA, name="llama2_70b_gqa_p32", block_size=32, num_blocks=8192,
                             description="Llama-2-70B GQA layer with 32-token blocks (else as llama2_70b_gqa)")
LLAMA2_70B_GQA_P64 = replace(LLAMA2_70B_GQA, name="llama2_70b_gqa_p64", block_size=64, num_blocks=4096,
                             description="Llama-2-70B GQA layer with 64-token blocks (else as llama2_70b_gqa)")
BLOCK_SIZE_CONFIGS = {c.name: c for c in (LLAMA2_70B_GQA_P32, LLAMA2_70B_GQA_P64)}

# One GPU's share of the Llama-2-70B GQA decode layer under 8-way tensor parallelism
# ("vLLM 推理优化技术深度调研报告", 维度一.6): the kv heads split over the GPUs, so each holds
# one kv head (and its 8 query heads) of every block, for the same 256 sequences and contexts.
LLAMA2_70B_GQA_TP8 = replace(LLAMA2_70B_GQA, name="llama2_70b_gqa_tp8", num_q_heads=8, num_kv_heads=1,
                             description="one GPU's share of the Llama-2-70B GQA layer at 8-way tensor parallelism: "
                                         "batch 256, 8 q / 1 kv head, D 128, bf16, ctx U[512,768]")
SHARD_CONFIGS = {c.name: c for c in (LLAMA2_70B_GQA_TP8,)}
ALL_CONFIGS = {**CONFIGS, **PREFILL_CONFIGS, **BLOCK_SIZE_CONFIGS, **SHARD_CONFIGS}
