"""Parity of the HIP prefill-chunk path with the oracle (element by element), plus its
invariants on the GPU: chunk composition, placement invariance, determinism, rows
outside the chunks untouched."""
import numpy as np
import pytest
import torch

from tests._gpu import (HostBatch, clone_batch, device_batch, gpu_prefill, gpu_prefill_step, max_err,
                        oracle_caches_after_step, oracle_prefill, say, tol)
from tests._paged import torch_bits
from workloads import PREFILL_CONFIGS, WorkloadConfig, make_batch

pytestmark = pytest.mark.gpu

DTYPES = [("f16", "f16"), ("bf16", "bf16"), ("bf16", "fp8_e4m3"), ("f16", "fp8_e4m3")]


def prefill_cfg(G, D, dtype, kv_dtype, S=6, Hkv=2, ctx=("uniform", 1, 300), chunk=("uniform", 1, 150),
                max_ctx=300, seed=11):
    return WorkloadConfig(
        name=f"prefill_G{G}_D{D}_{dtype}_{kv_dtype}", num_seqs=S, num_q_heads=G * Hkv, num_kv_heads=Hkv,
        head_dim=D, num_blocks=S * (max_ctx // 16 + 3) + 8, seed=seed, dtype=dtype, kv_dtype=kv_dtype,
        ctx=ctx, max_context_len=max_ctx, chunk=chunk, kv_scale=(1 / 128 if kv_dtype == "fp8_e4m3" else 1.0))


def _case(cfg):
    b = device_batch(cfg)
    h = HostBatch(b)
    say(cfg.name, "rows", int(h.query_start_loc[-1]), "ctx", h.context_lens.tolist())
    out = gpu_prefill_step(b)
    torch.cuda.synchronize()
    kc, vc = oracle_caches_after_step(h)
    ref = oracle_prefill(h, kc, vc)
    err = max_err(out, ref)
    assert err <= tol(cfg), f"{cfg.name}: error {err} beyond the output's rounding"
    return b, h, out


@pytest.mark.parametrize("dtype,kv_dtype", DTYPES)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_prefill_matches_oracle(G, D, dtype, kv_dtype):
    _case(prefill_cfg(G, D, dtype, kv_dtype))


@pytest.mark.parametrize("G,dtype,kv_dtype", [(1, "f16", "f16"), (8, "bf16", "bf16"), (4, "bf16", "fp8_e4m3")])
def test_whole_prompts_at_tile_edges(G, dtype, kv_dtype):
    # Prompts prefilled in one chunk, with lengths around the 16-key blocks, the 64-key
    # tiles and the 128-row workgroup tiles.
    lens = [1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 300]
    cfg = prefill_cfg(G, 128, dtype, kv_dtype, S=len(lens), ctx=("fixed", lens), chunk=("fixed", 1000), max_ctx=300)
    b, h, _ = _case(cfg)
    assert (np.diff(h.query_start_loc) == h.context_lens).all()


@pytest.mark.parametrize("S", [7, 256, 257])
@pytest.mark.parametrize("dtype,kv_dtype", [("bf16", "bf16"), ("bf16", "fp8_e4m3")])
def test_many_sequences_in_any_order(S, dtype, kv_dtype):
    # Workgroups visit sequences by decreasing work for up to 256 sequences and in batch
    # order beyond that; equal-work sequences (ties) and empty chunks included.
    rng = np.random.default_rng(S)
    ctx = rng.integers(1, 120, size=S)
    ctx[: S // 3] = 64                                        # ties
    cfg = prefill_cfg(4, 64, dtype, kv_dtype, S=S, Hkv=1, ctx=("fixed", ctx.tolist()), chunk=("uniform", 0, 40),
                      max_ctx=120, seed=S)
    _case(cfg)


@pytest.mark.parametrize("G,dtype,kv_dtype", [(8, "bf16", "bf16"), (2, "f16", "fp8_e4m3")])
def test_one_token_chunks_are_decode_steps(G, dtype, kv_dtype):
    _case(prefill_cfg(G, 128, dtype, kv_dtype, S=12, ctx=("uniform", 1, 700), chunk=("fixed", 1), max_ctx=700))


@pytest.mark.parametrize("G", [1, 8])
def test_chunks_compose_into_one_prefill_bit_for_bit(G):
    # Prefilling prompts in two chunks gives, row for row, the bits of one prefill of
    # the whole prompts: a row's arithmetic depends only on its own keys.
    lens = [70, 200, 129, 33]
    cfg = prefill_cfg(G, 128, "bf16", "bf16", S=4, ctx=("fixed", lens), chunk=("fixed", 1000), max_ctx=200)
    b = device_batch(cfg)
    say(cfg.name, "whole vs two chunks")
    whole = gpu_prefill_step(b)
    cut = torch.tensor([30, 64, 128, 1], dtype=torch.int32, device="cuda")
    qsl = b.query_start_loc.cpu().numpy()
    first_rows = np.concatenate([np.arange(qsl[s], qsl[s] + int(cut[s])) for s in range(4)])
    second_rows = np.concatenate([np.arange(qsl[s] + int(cut[s]), qsl[s + 1]) for s in range(4)])
    # chunk 1: the first cut[s] tokens, context = cut[s]
    qsl1 = torch.zeros(5, dtype=torch.int32, device="cuda")
    qsl1[1:] = torch.cumsum(cut, 0)
    c1 = clone_batch(b)
    c1.q = b.q[torch.from_numpy(first_rows).cuda()].contiguous()
    out1 = gpu_prefill(c1, context_lens=cut, query_start_loc=qsl1, max_q=int(cut.max()))
    # chunk 2: the rest, context = the whole prompt
    rest = b.context_lens - cut
    qsl2 = torch.zeros(5, dtype=torch.int32, device="cuda")
    qsl2[1:] = torch.cumsum(rest, 0)
    c2 = clone_batch(b)
    c2.q = b.q[torch.from_numpy(second_rows).cuda()].contiguous()
    out2 = gpu_prefill(c2, query_start_loc=qsl2, max_q=int(rest.max()))
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), whole[torch.from_numpy(first_rows).cuda()].view(torch.int16))
    assert torch.equal(out2.view(torch.int16), whole[torch.from_numpy(second_rows).cuda()].view(torch.int16))


@pytest.mark.parametrize("G,dtype,kv_dtype", [(8, "bf16", "bf16"), (4, "f16", "fp8_e4m3")])
def test_prefill_is_placement_invariant_and_deterministic(G, dtype, kv_dtype):
    cfg = prefill_cfg(G, 128, dtype, kv_dtype, S=5, ctx=("uniform", 40, 300))
    b = device_batch(cfg)
    say(cfg.name, "placement")
    out = gpu_prefill_step(b)
    again = gpu_prefill(b)
    # move every block of the pool to a new physical place
    perm = torch.randperm(cfg.num_blocks, generator=torch.Generator().manual_seed(3)).cuda()
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(cfg.num_blocks, device="cuda")
    kc = torch.empty_like(b.k_cache)
    vc = torch.empty_like(b.v_cache)
    kc[inv] = b.k_cache
    vc[inv] = b.v_cache
    moved = clone_batch(b)
    moved.block_tables = inv[b.block_tables.long()].int()
    out2 = gpu_prefill(moved, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_rows_outside_the_chunks_are_untouched():
    # Sequences with empty chunks, a chunk cut by max_query_len and a sequence whose
    # offsets leave the query rows: none of them writes where it should not.
    cfg = prefill_cfg(8, 128, "bf16", "bf16", S=5, ctx=("fixed", [50, 80, 90, 60, 40]),
                      chunk=("fixed", 20), max_ctx=90)
    b = device_batch(cfg)
    h = HostBatch(b)
    say(cfg.name, "untouched rows")
    gpu_prefill_step(b)
    kc, vc = oracle_caches_after_step(h)
    sentinel = torch.full_like(b.q, 7.0)
    # sequence 1: empty chunk; sequence 3: offsets past the rows
    qsl = torch.tensor([0, 20, 20, 40, 200, 200], dtype=torch.int32, device="cuda")
    # sequence 0: context shorter than its chunk -> cut to 12 rows
    ctx = b.context_lens.clone()
    ctx[0] = 12
    out = gpu_prefill(b, out=sentinel, context_lens=ctx, query_start_loc=qsl, max_q=20)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    assert (o[12:20] == 7.0).all() and (o[40:] == 7.0).all()
    ref = oracle_prefill(h, kc, vc, seqs=[2], query_start_loc=np.array([0, 20, 20, 40, 100, 100]))
    assert max_err(out[20:40], ref[20:40]) <= tol(cfg)
    assert np.isfinite(o[:12]).all()


@pytest.mark.parametrize("name", ["prefill_70b_gqa", "prefill_70b_gqa_fp8"])
def test_full_size_chunked_prefill_matches_oracle(name):
    # The Llama-2-70B GQA chunked-prefill batch at full size (16-bit and fp8 caches), in the
    # launch the benchmark times: every row of every sequence against the oracle.
    cfg = PREFILL_CONFIGS[name]
    b = make_batch(cfg, "cuda")
    h = HostBatch(b)
    say(cfg.name, "full size")
    out = gpu_prefill_step(b)
    torch.cuda.synchronize()
    kc, vc = oracle_caches_after_step(h)
    np.testing.assert_array_equal(torch_bits(b.k_cache), kc)
    np.testing.assert_array_equal(torch_bits(b.v_cache), vc)
    say(cfg.name, "oracle over all", cfg.num_seqs, "sequences")
    err = max_err(out, oracle_prefill(h, kc, vc))
    say(cfg.name, "error beyond rounding", err)
    assert err <= tol(cfg), f"error {err} beyond the output's rounding"


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_long_contexts_walk_past_the_staged_block_ids(kv_dtype):
    # Contexts of more than 1024 blocks: the workgroup restages its block ids mid-walk.
    cfg = prefill_cfg(8, 128, "bf16", kv_dtype, S=3, Hkv=1, ctx=("fixed", [20000, 16400, 16385]),
                      chunk=("fixed", 40), max_ctx=20000)
    _case(cfg)


@pytest.mark.parametrize("G,dtype,kv_dtype", [(8, "bf16", "bf16"), (4, "f16", "f16"), (8, "bf16", "fp8_e4m3")])
def test_long_prompts_in_one_chunk(G, dtype, kv_dtype):
    # Whole prompts of 4096 and 3500 tokens and 3000-token chunks after prefixes of 1000 and
    # 96 tokens: up to 256 row tiles of one (sequence, kv head), the longest items of any case.
    cfg = prefill_cfg(G, 128, dtype, kv_dtype, S=4, ctx=("fixed", [4096, 3500, 4000, 3096]), chunk=("fixed", 3000),
                      max_ctx=4096, seed=17)
    b, h, _ = _case(cfg)
    n = np.diff(h.query_start_loc)
    assert n.tolist() == [3000, 3000, 3000, 3000] and h.context_lens.tolist() == [4096, 3500, 4000, 3096]
    cfg = prefill_cfg(G, 128, dtype, kv_dtype, S=2, ctx=("fixed", [4096, 3500]), chunk=("fixed", 4096),
                      max_ctx=4096, seed=19)
    b, h, _ = _case(cfg)
    assert np.diff(h.query_start_loc).tolist() == [4096, 3500]
