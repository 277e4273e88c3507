"""The five workloads at their full sizes, in the launch configuration the benchmark
times: one whole decode step (copy-on-write copies, cache write, attention) on the GPU
against the oracle. Cache contents are compared bit for bit over the whole pool;
attention outputs on a sample of sequences (all heads, all columns)."""
import numpy as np
import pytest
import torch

from tests._gpu import HostBatch, gpu_step, max_err, oracle_caches_after_step, oracle_decode, say, tol
from tests._paged import torch_bits
from workloads import CONFIGS, make_batch

pytestmark = pytest.mark.gpu


def _sample(ctx: np.ndarray, n: int = 12):
    order = np.argsort(ctx, kind="stable")
    pick = set(np.linspace(0, len(ctx) - 1, n).round().astype(int).tolist())
    pick |= {int(order[0]), int(order[-1])}                   # shortest and longest
    return sorted(pick)


@pytest.mark.parametrize("name", ["tiny", "llama2_7b", "llama2_70b_gqa", "long_cot", "beam_cow"])
def test_full_size_step_matches_oracle(name):
    cfg = CONFIGS[name]
    say(name, "generate")
    b = make_batch(cfg, "cuda", replica=0)
    h = HostBatch(b)
    say(name, "step")
    out = gpu_step(b)
    torch.cuda.synchronize()
    kc, vc = oracle_caches_after_step(h)
    np.testing.assert_array_equal(torch_bits(b.k_cache), kc)
    np.testing.assert_array_equal(torch_bits(b.v_cache), vc)
    seqs = _sample(h.context_lens) if cfg.num_seqs > 16 else list(range(cfg.num_seqs))
    ref = oracle_decode(h, kc, vc, seqs=seqs)
    err = max_err(out, ref, seqs)
    say(name, "max abs error", err, "over", len(seqs), "sequences")
    assert err <= tol(cfg)
    g = out.float()
    assert torch.isfinite(g).all()
