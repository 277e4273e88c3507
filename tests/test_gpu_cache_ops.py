"""Bit-exact parity of the cache write and the copy-on-write copies with the oracle."""
import numpy as np
import pytest
import torch

import paged_kv_cache_409_amd as pkv
from oracle import cache_ops, formats
from tests._gpu import HostBatch, device_batch, say
from tests._paged import torch_bits
from workloads import CONFIGS, WorkloadConfig

pytestmark = pytest.mark.gpu


def _cfg(dtype, kv_dtype, D=128, Hkv=4, S=37):
    return WorkloadConfig(name=f"cw_{dtype}_{kv_dtype}_{D}", num_seqs=S, num_q_heads=Hkv, num_kv_heads=Hkv,
                          head_dim=D, num_blocks=S * 8 + 8, seed=21, dtype=dtype, kv_dtype=kv_dtype,
                          ctx=("uniform", 1, 100), max_context_len=100,
                          kv_scale=(0.0134 if kv_dtype == "fp8_e4m3" else 1.0))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype,kv_dtype", [("f16", "f16"), ("bf16", "bf16"), ("bf16", "fp8_e4m3"),
                                            ("f16", "fp8_e4m3")])
def test_reshape_and_cache_bit_exact(dtype, kv_dtype, D):
    cfg = _cfg(dtype, kv_dtype, D)
    b = device_batch(cfg)
    # a padded batch row (negative slot) must be skipped
    b.slot_mapping[5] = -1
    h = HostBatch(b)
    say(cfg.name, "reshape_and_cache")
    pkv.reshape_and_cache(b.new_k, b.new_v, b.slot_mapping, b.k_cache, b.v_cache, b.k_scale, b.v_scale)
    torch.cuda.synchronize()
    ek, ev = cache_ops.reshape_and_cache(h.new_k, h.new_v, h.slot_mapping, h.k_cache, h.v_cache, cfg.dtype,
                                         cfg.kv_dtype, h.k_scale, h.v_scale)
    np.testing.assert_array_equal(torch_bits(b.k_cache), ek)
    np.testing.assert_array_equal(torch_bits(b.v_cache), ev)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fp8_quantisation_of_every_16bit_pattern(dtype):
    # All 65536 input bit patterns (NaN, infinities, subnormals, saturating values) through
    # the cache write at two scales, against the oracle's encoder.
    for scale in (1.0, 0.0134):
        T, Hkv, D = 64, 8, 128                                    # 64 * 8 * 128 = 65536 elements
        pattern = torch.arange(65536, dtype=torch.int32).to(torch.int16)
        key = pattern.view(torch.float16 if dtype == "f16" else torch.bfloat16).reshape(T, Hkv, D).cuda()
        value = key.flip(0).contiguous()
        kc = torch.zeros((T, Hkv, 16, D), dtype=torch.uint8, device="cuda")
        vc = torch.zeros_like(kc)
        slots = (torch.arange(T, dtype=torch.int64) * 16 + 3).cuda()
        say("fp8 encode", dtype, scale)
        pkv.reshape_and_cache(key, value, slots, kc, vc, scale, scale)
        torch.cuda.synchronize()
        x = formats.to_f64(torch_bits(key), dtype)
        with np.errstate(invalid="ignore"):
            want = formats.e4m3_encode(formats.round_to_f32(x / float(np.float32(scale))))
        got = torch_bits(kc)[:, :, 3, :]
        np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("layers", [1, 3, 70])
def test_copy_blocks_bit_exact(layers):
    g = torch.Generator().manual_seed(layers)
    NB, Hkv, D = 64, 2, 64
    ks = [torch.randint(0, 255, (NB, Hkv, 16, D), generator=g, dtype=torch.uint8).cuda() for _ in range(layers)]
    vs = [torch.randint(0, 255, (NB, Hkv, 16, D), generator=g, dtype=torch.uint8).cuda() for _ in range(layers)]
    pairs = np.array([[1, 40], [2, 41], [2, 42], [63, 0], [7, 7]], dtype=np.int64)
    hk = [torch_bits(k) for k in ks]
    hv = [torch_bits(v) for v in vs]
    say("copy_blocks layers", layers)
    pkv.copy_blocks(ks, vs, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    ek, ev = cache_ops.copy_blocks(hk, hv, pairs)
    for layer in range(layers):
        np.testing.assert_array_equal(torch_bits(ks[layer]), ek[layer])
        np.testing.assert_array_equal(torch_bits(vs[layer]), ev[layer])


def test_copy_blocks_empty_list_is_a_no_op():
    k = torch.randint(0, 255, (8, 2, 16, 64), dtype=torch.uint8).cuda()
    v = k.clone()
    before = k.clone()
    pkv.copy_blocks([k], [v], torch.zeros((0, 2), dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(k, before) and torch.equal(v, before)


def test_beam_copy_on_write_pairs_bit_exact():
    cfg = WorkloadConfig(name="beam_small", num_seqs=16, num_q_heads=8, num_kv_heads=2, head_dim=128,
                         num_blocks=1024, seed=12, dtype="bf16", kv_dtype="fp8_e4m3", ctx=("beam", 64, 0, 60, 4),
                         max_context_len=64 + 60 + 1, kv_scale=1 / 128)
    b = device_batch(cfg)
    h = HostBatch(b)
    assert len(h.copy_pairs) > 0
    say(cfg.name, "copy pairs", len(h.copy_pairs))
    pkv.copy_blocks([b.k_cache], [b.v_cache], b.copy_pairs)
    torch.cuda.synchronize()
    (ek,), (ev,) = cache_ops.copy_blocks([h.k_cache], [h.v_cache], h.copy_pairs)
    np.testing.assert_array_equal(torch_bits(b.k_cache), ek)
    np.testing.assert_array_equal(torch_bits(b.v_cache), ev)
