"""Zero-size calls of every entry point: a decode batch of no sequences (plain, fused, and
the step that allocates nothing), a cache write of no tokens, copies and swaps of no pairs,
and a prefill of no sequences or of sequences with no new tokens. Each returns success,
launches nothing that writes, and leaves the caches and the output bit for bit as they were
(a server's step may find an empty batch, "vLLM推理引擎PagedAttention原理与性能优化实战", §四)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_409_amd as pkv
from tests._gpu import say
from tests._paged import torch_bits

pytestmark = pytest.mark.gpu

NB, Hkv, P, D, G = 64, 2, 16, 128, 4


def pools(kv_dtype):
    g = torch.Generator(device="cuda").manual_seed(5)
    if kv_dtype == "fp8_e4m3":
        k = torch.randint(0, 127, (NB, Hkv, P, D), dtype=torch.uint8, device="cuda", generator=g)
    else:
        k = torch.randn((NB, Hkv, P, D), device="cuda", generator=g).to(torch.bfloat16)
    return k, k.clone().flip(0).contiguous()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_empty_decode_batches_change_nothing(kv_dtype):
    say("empty decode batches", kv_dtype)
    kc, vc = pools(kv_dtype)
    before = torch_bits(kc), torch_bits(vc)
    q = torch.empty((0, Hkv * G, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    kv = torch.empty((0, Hkv, D), dtype=torch.bfloat16, device="cuda")
    slots = torch.empty(0, dtype=torch.int64, device="cuda")
    bt = torch.empty((0, 4), dtype=torch.int32, device="cuda")
    cl = torch.empty(0, dtype=torch.int32, device="cuda")
    cow = torch.empty(0, dtype=torch.int32, device="cuda")
    pkv.paged_attention_decode(out, q, kc, vc, bt, cl, 0.125, 64, 1.0, 1.0)
    pkv.decode_step(out, q, kc, vc, kv, kv, slots, bt, cl, 0.125, 64, 1.0, 1.0)
    pkv.decode_step(out, q, kc, vc, kv, kv, slots, bt, cl, 0.125, 64, 1.0, 1.0, cow_src=cow)
    pkv.decode_step_no_alloc(out, q, kc, vc, kv, kv, slots, bt, cl, 0.125, 64, 1.0, 1.0)
    pkv.reshape_and_cache(kv, kv, slots, kc, vc, 1.0, 1.0)
    pkv.copy_blocks([kc], [vc], torch.empty((0, 2), dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(torch_bits(kc), before[0])
    np.testing.assert_array_equal(torch_bits(vc), before[1])


def test_empty_prefill_batches_change_nothing():
    say("empty prefill batches")
    kc, vc = pools("bf16")
    before = torch_bits(kc), torch_bits(vc)
    # No sequences at all.
    q = torch.empty((0, Hkv * G, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    pkv.paged_attention_prefill(out, q, kc, vc, torch.empty((0, 4), dtype=torch.int32, device="cuda"),
                                torch.empty(0, dtype=torch.int32, device="cuda"),
                                torch.zeros(1, dtype=torch.int32, device="cuda"), 0.125, 0, 1.0, 1.0)
    # Three sequences with contexts but no new tokens: no rows to write.
    bt = torch.arange(12, dtype=torch.int32, device="cuda").reshape(3, 4)
    pkv.paged_attention_prefill(out, q, kc, vc, bt, torch.tensor([10, 40, 64], dtype=torch.int32, device="cuda"),
                                torch.zeros(4, dtype=torch.int32, device="cuda"), 0.125, 0, 1.0, 1.0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(torch_bits(kc), before[0])
    np.testing.assert_array_equal(torch_bits(vc), before[1])


def test_swaps_of_no_pairs_change_nothing():
    say("empty swaps")
    kc, vc = pools("bf16")
    hk = torch.randn((8, Hkv, P, D)).to(torch.bfloat16).pin_memory()
    hv = torch.randn((8, Hkv, P, D)).to(torch.bfloat16).pin_memory()
    before = torch_bits(kc), torch_bits(vc), torch_bits(hk), torch_bits(hv)
    none = torch.empty((0, 2), dtype=torch.int64, device="cuda")
    pkv.swap_blocks([kc], [vc], [hk], [hv], none)
    pkv.swap_blocks([hk], [hv], [kc], [vc], none)
    torch.cuda.synchronize()
    for got, want in zip((kc, vc, hk, hv), before):
        np.testing.assert_array_equal(torch_bits(got), want)
