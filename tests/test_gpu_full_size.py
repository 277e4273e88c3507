"""The five workloads at their full sizes, in the launch configuration the benchmark
times: one whole decode step (copy-on-write copies, cache write, attention) on the GPU
against the oracle. Cache contents are compared bit for bit over the whole pool, and
the attention output of every sequence, head and column against the oracle."""
import numpy as np
import pytest
import torch

from tests._gpu import HostBatch, gpu_step, max_err, oracle_caches_after_step, oracle_decode, say, tol
from tests._paged import torch_bits
from workloads import ALL_CONFIGS, make_batch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "llama2_7b", "llama2_70b_gqa", "long_cot", "beam_cow", "llama2_70b_gqa_tp8"])
def test_full_size_step_matches_oracle(name):
    cfg = ALL_CONFIGS[name]
    say(name, "generate")
    b = make_batch(cfg, "cuda", replica=0)
    h = HostBatch(b)
    say(name, "step")
    out = gpu_step(b)
    torch.cuda.synchronize()
    kc, vc = oracle_caches_after_step(h)
    np.testing.assert_array_equal(torch_bits(b.k_cache), kc)
    np.testing.assert_array_equal(torch_bits(b.v_cache), vc)
    say(name, "oracle over all", cfg.num_seqs, "sequences")
    err = max_err(out, oracle_decode(h, kc, vc))
    say(name, "error beyond rounding", err)
    assert err <= tol(cfg)
