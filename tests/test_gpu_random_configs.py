"""Seeded sweeps over mixed configurations: head counts, group sizes (powers of two and
others), head dims, q and cache dtypes, block sizes, batch sizes and context lengths.

* Decode: partition sizes (the library's own choice among them) and both context kinds (independent sequences, beams sharing a
  prompt with copy-on-write). Each case runs pkv_decode_step with its copy-on-write
  sources ("vLLM推理引擎PagedAttention原理与性能优化实战", §3.2) and compares both caches
  bit for bit, and the attention within the dtype's tolerance, with the oracle's copies,
  cache write and attention over the same bits ("vLLM 推理优化技术深度调研报告", 维度一.3
  公式3-4).
* Prefill chunks (the first page, §六): chunk lengths up to the whole context. Each case
  writes the chunks' K/V with pkv_reshape_and_cache and runs pkv_paged_attention_prefill,
  against the oracle's cache write and causal attention over the same bits."""
import numpy as np
import pytest

from tests._gpu import (HostBatch, device_batch, gpu_cow_step, gpu_prefill_step, max_err, oracle_caches_after_step,
                        oracle_decode, oracle_prefill, say, tol)
from tests._paged import torch_bits
from workloads import WorkloadConfig

pytestmark = pytest.mark.gpu


def draw_config(case: int) -> tuple[WorkloadConfig, int]:
    rng = np.random.default_rng([4091, case])
    Hkv = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12]))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 16]))
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    kv_dtype = str(rng.choice([dtype, "fp8_e4m3"]))
    P = int(rng.choice([16, 32, 64]))
    partition = int(rng.choice([0, 0, 0, 16, 48, 64, 192, 256]))
    if rng.random() < 0.5:
        width = int(rng.choice([2, 3, 4]))
        S = width * int(rng.integers(1, 13))
        prompt = P * int(rng.integers(0, 400 // P + 1))
        tail = int(rng.integers(1, 80))
        ctx = ("beam", prompt, 0, tail, width)
        max_ctx = prompt + tail + 1
        blocks = (S // width) * (prompt // P + width * (tail // P + 2)) + S * 2 + 8
    else:
        S = int(rng.integers(1, 49))
        hi = int(rng.integers(1, 1500))
        lo = int(rng.integers(1, hi + 1))
        ctx = ("uniform", lo, hi)
        max_ctx = hi
        blocks = S * (hi // P + 2) + 8
    cfg = WorkloadConfig(name=f"sweep{case}_Hkv{Hkv}_G{G}_D{D}_{dtype}_{kv_dtype}_P{P}_{ctx[0]}", num_seqs=S,
                         num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=D, num_blocks=blocks, seed=7000 + case,
                         dtype=dtype, kv_dtype=kv_dtype, ctx=ctx, max_context_len=max_ctx, block_size=P,
                         kv_scale=(1 / 64 if kv_dtype == "fp8_e4m3" else 1.0))
    return cfg, partition


@pytest.mark.parametrize("case", range(128))
def test_random_decode_configuration_matches_oracle(case):
    cfg, partition = draw_config(case)
    b = device_batch(cfg)
    h = HostBatch(b)
    say(cfg.name, "S", cfg.num_seqs, "ctx", cfg.ctx, "partition", partition, "pairs", len(h.copy_pairs))
    out = gpu_cow_step(b, partition)
    kc, vc = oracle_caches_after_step(h)
    np.testing.assert_array_equal(torch_bits(b.k_cache), kc)
    np.testing.assert_array_equal(torch_bits(b.v_cache), vc)
    assert max_err(out, oracle_decode(h, kc, vc)) <= tol(cfg)


def draw_prefill_config(case: int) -> WorkloadConfig:
    rng = np.random.default_rng([4092, case])
    Hkv = int(rng.choice([1, 2, 3, 4, 6, 8]))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16]))
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    kv_dtype = str(rng.choice([dtype, "fp8_e4m3"]))
    P = int(rng.choice([16, 32, 64]))
    S = int(rng.integers(1, 13))
    hi = int(rng.integers(1, 1200))
    lo = int(rng.integers(1, hi + 1))
    chunk = ("uniform", 1, int(rng.integers(1, 400)))
    return WorkloadConfig(name=f"psweep{case}_Hkv{Hkv}_G{G}_D{D}_{dtype}_{kv_dtype}_P{P}", num_seqs=S,
                          num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=D, num_blocks=S * (hi // P + 2) + 8,
                          seed=8000 + case, dtype=dtype, kv_dtype=kv_dtype, ctx=("uniform", lo, hi),
                          max_context_len=hi, block_size=P, chunk=chunk,
                          kv_scale=(1 / 64 if kv_dtype == "fp8_e4m3" else 1.0))


@pytest.mark.parametrize("case", range(64))
def test_random_prefill_configuration_matches_oracle(case):
    cfg = draw_prefill_config(case)
    b = device_batch(cfg)
    h = HostBatch(b)
    say(cfg.name, "S", cfg.num_seqs, "rows", int(h.query_start_loc[-1]), "ctx", cfg.ctx, "chunk", cfg.chunk)
    out = gpu_prefill_step(b)
    kc, vc = oracle_caches_after_step(h)
    np.testing.assert_array_equal(torch_bits(b.k_cache), kc)
    np.testing.assert_array_equal(torch_bits(b.v_cache), vc)
    assert max_err(out, oracle_prefill(h, kc, vc)) <= tol(cfg)
