"""The fused decode step (cache write + attention in one launch) gives the results of the
two separate calls, bit for bit: the caches after the step and the attention output."""
import numpy as np
import pytest
import torch

from tests._gpu import (HostBatch, clone_batch, device_batch, gpu_fused_step, gpu_step, max_err,
                        oracle_caches_after_step, oracle_decode, say, tol)
from tests._paged import torch_bits
from tests.test_gpu_decode import small_cfg
from workloads import ALL_CONFIGS, WorkloadConfig, make_batch

pytestmark = pytest.mark.gpu


def _compare(b, partition):
    two = clone_batch(b)
    h = HostBatch(b)
    fused_out = gpu_fused_step(b, partition)
    two_out = gpu_step(two, partition)
    torch.cuda.synchronize()
    kc, vc = oracle_caches_after_step(h)
    np.testing.assert_array_equal(torch_bits(b.k_cache), kc)
    np.testing.assert_array_equal(torch_bits(b.v_cache), vc)
    np.testing.assert_array_equal(torch_bits(two.k_cache), kc)       # raw bits: stale slots hold NaN
    np.testing.assert_array_equal(torch_bits(two.v_cache), vc)
    assert torch.equal(fused_out.view(torch.int16), two_out.view(torch.int16))
    return h, kc, vc, fused_out


@pytest.mark.parametrize("partition", [0, 48])
@pytest.mark.parametrize("G,dtype,kv_dtype", [(1, "f16", "f16"), (1, "bf16", "fp8_e4m3"), (4, "bf16", "bf16"),
                                              (8, "bf16", "bf16"), (4, "f16", "fp8_e4m3"), (16, "bf16", "bf16"),
                                              (3, "bf16", "bf16"), (5, "f16", "fp8_e4m3"), (6, "bf16", "bf16"),
                                              (12, "bf16", "bf16")])
def test_fused_step_equals_write_then_decode(G, dtype, kv_dtype, partition):
    cfg = small_cfg(G, 128, dtype, kv_dtype, S=9, ctx=("uniform", 1, 300), max_ctx=300)
    b = device_batch(cfg)
    say(cfg.name, "fused step, partition", partition)
    h, kc, vc, out = _compare(b, partition)
    assert max_err(out, oracle_decode(h, kc, vc)) <= tol(cfg)


@pytest.mark.parametrize("partition", [0, 32])
@pytest.mark.parametrize("G,kv_dtype", [(4, "bf16"), (4, "fp8_e4m3"), (2, "bf16"), (1, "bf16"), (3, "bf16"),
                                        (5, "fp8_e4m3")])
def test_fused_step_with_shared_blocks(G, kv_dtype, partition):
    # Beams: copy-on-write of shared partial blocks, then the fused step (sharing groups
    # for grouped heads).
    cfg = WorkloadConfig(name=f"fused_beam_G{G}_{kv_dtype}", num_seqs=16, num_q_heads=2 * G, num_kv_heads=2,
                         head_dim=128, num_blocks=2048, seed=41 + G, dtype="bf16", kv_dtype=kv_dtype,
                         ctx=("beam", 96, 0, 40, 4), max_context_len=96 + 40 + 1,
                         kv_scale=(1 / 128 if kv_dtype == "fp8_e4m3" else 1.0))
    b = device_batch(cfg)
    assert len(b.copy_pairs) > 0
    say(cfg.name, "fused step, partition", partition)
    h, kc, vc, out = _compare(b, partition)
    assert max_err(out, oracle_decode(h, kc, vc)) <= tol(cfg)


@pytest.mark.parametrize("G", [1, 8])
def test_fused_step_zero_length_rows_and_skipped_slots(G):
    cfg = small_cfg(G, 128, "bf16", "bf16", S=6, ctx=("uniform", 1, 200), max_ctx=200)
    b = device_batch(cfg)
    b.context_lens[2] = 0          # a padded row: no context, but its token is still written
    b.slot_mapping[4] = -1         # a row whose token is not written
    say(cfg.name, "fused step, padded rows")
    h, kc, vc, out = _compare(b, 0)
    assert (out[2] == 0).all()


@pytest.mark.parametrize("name", ["llama2_7b", "llama2_70b_gqa", "long_cot", "beam_cow", "llama2_70b_gqa_tp8"])
def test_full_size_fused_step(name):
    # The launch the benchmark times, on one of its replicas: caches bit for bit and every
    # sequence, head and column of the output against the oracle.
    cfg = ALL_CONFIGS[name]
    say(name, "generate")
    b = make_batch(cfg, "cuda", replica=1)
    say(name, "fused step")
    h, kc, vc, out = _compare(b, None)
    say(name, "oracle over all", cfg.num_seqs, "sequences")
    err = max_err(out, oracle_decode(h, kc, vc))
    say(name, "error beyond rounding", err)
    assert err <= tol(cfg)
