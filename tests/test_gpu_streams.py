"""Calls on two streams at once. The library keeps no state between calls apart from the
scratch array of the step that allocates nothing, so decode steps and prefill chunks of two
batches, issued alternately on two streams of default priority with their own workspaces,
must give what each gives alone, bit for bit (two model replicas or layers in flight,
"vLLM推理引擎PagedAttention原理与性能优化实战", §四)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_409_amd as pkv
from tests._gpu import clone_batch, device_batch, max_query_len, say
from tests._paged import torch_bits
from workloads import WorkloadConfig

pytestmark = pytest.mark.gpu


def cfg(name, G, seed, kv_dtype="bf16", chunk=None):
    return WorkloadConfig(name=name, num_seqs=24, num_q_heads=2 * G, num_kv_heads=2, head_dim=128,
                          num_blocks=24 * (700 // 16 + 3) + 8, seed=seed, dtype="bf16", kv_dtype=kv_dtype,
                          ctx=("uniform", 1, 700), max_context_len=700, chunk=chunk,
                          kv_scale=(1 / 64 if kv_dtype == "fp8_e4m3" else 1.0))


def step(b, out, ws, partition, stream):
    pkv.decode_step(out, b.q, b.k_cache, b.v_cache, b.new_k, b.new_v, b.slot_mapping, b.block_tables, b.context_lens,
                    b.scale, b.cfg.max_context_len, b.k_scale, b.v_scale, partition, workspace=ws, stream=stream)


def prefill(b, out, stream):
    pkv.reshape_and_cache(b.new_k, b.new_v, b.slot_mapping, b.k_cache, b.v_cache, b.k_scale, b.v_scale, stream=stream)
    pkv.paged_attention_prefill(out, b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.query_start_loc,
                                b.scale, max_query_len(b), b.k_scale, b.v_scale, stream=stream)


def test_decode_steps_on_two_streams_match_each_alone():
    a0, b0 = device_batch(cfg("streams_a", 8, 51)), device_batch(cfg("streams_b", 1, 52, "fp8_e4m3"))
    say("two streams: decode", a0.cfg.name, b0.cfg.name)
    part = 64
    wa = torch.empty(pkv.workspace_size(24, 16, 2, 128, 700, part), dtype=torch.uint8, device="cuda")
    wb = torch.empty(pkv.workspace_size(24, 2, 2, 128, 700, part), dtype=torch.uint8, device="cuda")
    alone = []
    for b0_, ws in ((a0, wa), (b0, wb)):
        b = clone_batch(b0_)
        out = torch.empty_like(b.q)
        step(b, out, ws, part, None)
        torch.cuda.synchronize()
        alone.append((torch_bits(out), torch_bits(b.k_cache), torch_bits(b.v_cache)))
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        a, b = clone_batch(a0), clone_batch(b0)
        oa, ob = torch.empty_like(a.q), torch.empty_like(b.q)
        torch.cuda.synchronize()
        for _ in range(4):      # the same step again on each stream: same caches after the first
            step(a, oa, wa, part, sa)
            step(b, ob, wb, part, sb)
        torch.cuda.synchronize()
        for got, want in zip((oa, a.k_cache, a.v_cache), alone[0]):
            np.testing.assert_array_equal(torch_bits(got), want, err_msg=f"stream a, round {rep}")
        for got, want in zip((ob, b.k_cache, b.v_cache), alone[1]):
            np.testing.assert_array_equal(torch_bits(got), want, err_msg=f"stream b, round {rep}")


def test_prefill_and_decode_on_two_streams_match_each_alone():
    p0 = device_batch(cfg("streams_prefill", 8, 53, chunk=("uniform", 1, 300)))
    d0 = device_batch(cfg("streams_decode", 4, 54))
    say("two streams: prefill beside decode", p0.cfg.name, d0.cfg.name)
    wd = torch.empty(pkv.workspace_size(24, 8, 2, 128, 700, 0), dtype=torch.uint8, device="cuda")
    p, d = clone_batch(p0), clone_batch(d0)
    op, od = torch.empty_like(p.q), torch.empty_like(d.q)
    prefill(p, op, None)
    step(d, od, wd, 0, None)
    torch.cuda.synchronize()
    want = [torch_bits(t) for t in (op, p.k_cache, p.v_cache, od, d.k_cache, d.v_cache)]
    sp, sd = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        p, d = clone_batch(p0), clone_batch(d0)
        op, od = torch.empty_like(p.q), torch.empty_like(d.q)
        torch.cuda.synchronize()
        prefill(p, op, sp)
        step(d, od, wd, 0, sd)
        torch.cuda.synchronize()
        for i, t in enumerate((op, p.k_cache, p.v_cache, od, d.k_cache, d.v_cache)):
            np.testing.assert_array_equal(torch_bits(t), want[i], err_msg=f"tensor {i}, round {rep}")
