"""Hot-path launches captured once in a HIP graph (torch.cuda.graph) and replayed, as a
serving loop replays one captured step per iteration ("vLLM推理引擎PagedAttention原理与性能
优化实战", §四): the fused decode step with copy-on-write, both the form that allocates
nothing and the form with a caller's workspace, and a prefill chunk with its cache write
(the same page, §六). The caches are reset by eager work between replays, and every replay
must give the eager call's output and caches bit for bit. None of these entry points
records a memset, a copy or a synchronisation."""
import numpy as np
import pytest
import torch

import paged_kv_cache_409_amd as pkv
from tests._gpu import device_batch, max_query_len, say
from tests._paged import torch_bits
from workloads import WorkloadConfig

pytestmark = pytest.mark.gpu

REPLAYS = 4


def beam_cfg(kv_dtype, G):
    width, S, prompt, tail = 4, 16, 160, 40
    return WorkloadConfig(name=f"graph_beams_G{G}_{kv_dtype}", num_seqs=S, num_q_heads=2 * G, num_kv_heads=2,
                          head_dim=128, num_blocks=(S // width) * (prompt // 16 + width * (tail // 16 + 2)) + 2 * S + 8,
                          seed=37, dtype="bf16", kv_dtype=kv_dtype, ctx=("beam", prompt, 0, tail, width),
                          max_context_len=prompt + tail + 1, kv_scale=(1 / 64 if kv_dtype == "fp8_e4m3" else 1.0))


def replay_and_compare(run, tensors, reset):
    """Eager run, then capture, then replays with eager resets between them."""
    reset()
    run()
    torch.cuda.synchronize()
    want = [torch_bits(t) for t in tensors]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for r in range(REPLAYS):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, w in zip(tensors, want):
            np.testing.assert_array_equal(torch_bits(t), w, err_msg=f"replay {r}")


@pytest.mark.parametrize("no_alloc", [True, False])
@pytest.mark.parametrize("kv_dtype,G,partition", [("bf16", 4, 0), ("bf16", 8, 64), ("fp8_e4m3", 4, 48),
                                                  ("bf16", 1, 32)])
def test_decode_step_replays_in_a_graph(no_alloc, kv_dtype, G, partition):
    b = device_batch(beam_cfg(kv_dtype, G))
    say(b.cfg.name, "no_alloc", no_alloc, "partition", partition, "copies", int((b.cow_src >= 0).sum()))
    k0, v0 = b.k_cache.clone(), b.v_cache.clone()
    out = torch.empty_like(b.q)
    S, Hq, D = b.q.shape
    ws = None if no_alloc else torch.empty(
        max(pkv.workspace_size(S, Hq, b.k_cache.shape[1], D, b.cfg.max_context_len, partition), 1),
        dtype=torch.uint8, device="cuda")

    def run():
        args = (out, b.q, b.k_cache, b.v_cache, b.new_k, b.new_v, b.slot_mapping, b.block_tables, b.context_lens,
                b.scale, b.cfg.max_context_len, b.k_scale, b.v_scale, partition)
        if no_alloc:
            pkv.decode_step_no_alloc(*args, cow_src=b.cow_src)
        else:
            pkv.decode_step(*args, workspace=ws, cow_src=b.cow_src)

    def reset():
        b.k_cache.copy_(k0)
        b.v_cache.copy_(v0)
        out.fill_(float("nan"))

    replay_and_compare(run, [out, b.k_cache, b.v_cache], reset)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_prefill_chunk_replays_in_a_graph(kv_dtype):
    cfg = WorkloadConfig(name=f"graph_prefill_{kv_dtype}", num_seqs=5, num_q_heads=16, num_kv_heads=2, head_dim=128,
                         num_blocks=5 * (400 // 16 + 3) + 8, seed=41, dtype="bf16", kv_dtype=kv_dtype,
                         ctx=("uniform", 50, 400), max_context_len=400, chunk=("uniform", 1, 200),
                         kv_scale=(1 / 64 if kv_dtype == "fp8_e4m3" else 1.0))
    b = device_batch(cfg)
    say(cfg.name, "rows", int(b.query_start_loc[-1]))
    k0, v0 = b.k_cache.clone(), b.v_cache.clone()
    out = torch.empty_like(b.q)
    max_q = max_query_len(b)

    def run():
        pkv.reshape_and_cache(b.new_k, b.new_v, b.slot_mapping, b.k_cache, b.v_cache, b.k_scale, b.v_scale)
        pkv.paged_attention_prefill(out, b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                                    b.query_start_loc, b.scale, max_q, b.k_scale, b.v_scale)

    def reset():
        b.k_cache.copy_(k0)
        b.v_cache.copy_(v0)
        out.fill_(float("nan"))

    replay_and_compare(run, [out, b.k_cache, b.v_cache], reset)
