"""Parity of the HIP decode path with the oracle (element by element), plus the
method's invariants on the GPU: placement invariance, shared = copied blocks,
determinism, split = unsplit, stale slots never read."""
import numpy as np
import pytest
import torch

from tests._gpu import (HostBatch, device_batch, gpu_decode, gpu_step, max_err, oracle_caches_after_step,
                        oracle_decode, say, tol)
from tests._paged import torch_bits
from workloads import WorkloadConfig

pytestmark = pytest.mark.gpu


def small_cfg(G, D, dtype, kv_dtype, S=10, Hkv=2, ctx=("uniform", 1, 600), max_ctx=600, seed=7, nb=None):
    return WorkloadConfig(
        name=f"small_G{G}_D{D}_{dtype}_{kv_dtype}", num_seqs=S, num_q_heads=G * Hkv, num_kv_heads=Hkv,
        head_dim=D, num_blocks=nb or S * (max_ctx // 16 + 3) + 8, seed=seed, dtype=dtype, kv_dtype=kv_dtype,
        ctx=ctx, max_context_len=max_ctx, kv_scale=(1 / 128 if kv_dtype == "fp8_e4m3" else 1.0))


DTYPES = [("f16", "f16"), ("bf16", "bf16"), ("bf16", "fp8_e4m3"), ("f16", "fp8_e4m3")]


def _step_case(cfg, partition_size=0):
    b = device_batch(cfg)
    h = HostBatch(b)
    say(cfg.name, "partition", partition_size)
    out = gpu_step(b, partition_size)
    torch.cuda.synchronize()
    kc, vc = oracle_caches_after_step(h)
    ref = oracle_decode(h, kc, vc)
    err = max_err(out, ref)
    assert err <= tol(cfg), f"{cfg.name}: error {err} beyond the output's rounding"
    return b, out


@pytest.mark.parametrize("dtype,kv_dtype", DTYPES)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_decode_step_matches_oracle(G, D, dtype, kv_dtype):
    _step_case(small_cfg(G, D, dtype, kv_dtype))


@pytest.mark.parametrize("partition", [0, 48])
@pytest.mark.parametrize("dtype,kv_dtype", [("bf16", "bf16"), ("f16", "fp8_e4m3")])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [3, 5, 6, 7, 12])
def test_group_sizes_off_the_powers_of_two_match_oracle(G, D, dtype, kv_dtype, partition):
    # Query-head groups that do not divide 16: workgroups of 4, 3, 2, 2 and 1 sequences
    # whose 16 product columns are filled to 12, 15, 12, 14 and 12, and final merges that
    # split D over 4, 3, 2, 2 and 1 wavefronts.
    _step_case(small_cfg(G, D, dtype, kv_dtype, S=11), partition)


@pytest.mark.parametrize("partition", [16, 48, 256, 512])
@pytest.mark.parametrize("G,dtype,kv_dtype", [(1, "f16", "f16"), (8, "bf16", "bf16"), (4, "bf16", "fp8_e4m3")])
def test_split_context_matches_oracle_and_unsplit(G, dtype, kv_dtype, partition):
    cfg = small_cfg(G, 128, dtype, kv_dtype, S=6, ctx=("uniform", 1, 1100), max_ctx=1100)
    b, split = _step_case(cfg, partition)
    whole = gpu_decode(b, partition_size=0)
    torch.cuda.synchronize()
    diff = (split.float() - whole.float()).abs().max().item()
    assert diff <= 2 * tol(cfg)


@pytest.mark.parametrize("G,dtype,kv_dtype", [(1, "f16", "f16"), (8, "bf16", "bf16"), (4, "bf16", "fp8_e4m3")])
def test_context_lengths_at_block_and_table_edges(G, dtype, kv_dtype):
    # 1, 15, 16, 17, 31, 32, 33 tokens and a completely full block-table row (5 blocks).
    ctx = [1, 15, 16, 17, 31, 32, 33, 80]
    cfg = small_cfg(G, 128, dtype, kv_dtype, S=len(ctx), ctx=("fixed", ctx), max_ctx=80)
    _step_case(cfg)
    _step_case(cfg, partition_size=16)


@pytest.mark.parametrize("G", [1, 8])
def test_zero_length_context_gives_zeros(G):
    cfg = small_cfg(G, 128, "bf16", "bf16", S=6, ctx=("uniform", 1, 200), max_ctx=200)
    b = device_batch(cfg)
    h = HostBatch(b)
    say(cfg.name, "zero-length rows")
    gpu_step(b)
    kc, vc = oracle_caches_after_step(h)
    ctx = b.context_lens.clone()
    ctx[1] = 0
    ctx[4] = 0
    for part in (0, 64):
        out = gpu_decode(b, partition_size=part, context_lens=ctx)
        torch.cuda.synchronize()
        assert (out[1] == 0).all() and (out[4] == 0).all()
        ref = oracle_decode(h, kc, vc, context_lens=ctx.cpu().numpy())
        assert max_err(out, ref) <= tol(cfg)


def _beam_cfg(G, kv_dtype, S=8, prompt=64, tail=40, seed=11):
    return WorkloadConfig(name=f"beam_G{G}_{kv_dtype}", num_seqs=S, num_q_heads=2 * G, num_kv_heads=2, head_dim=128,
                          num_blocks=1024, seed=seed, dtype="bf16", kv_dtype=kv_dtype, ctx=("beam", prompt, 0, tail, 4),
                          max_context_len=prompt + tail + 1, kv_scale=(1 / 128 if kv_dtype == "fp8_e4m3" else 1.0))


@pytest.mark.parametrize("G,dtype,kv_dtype,beams", [(1, "f16", "f16", False), (8, "bf16", "bf16", False),
                                                    (4, "bf16", "fp8_e4m3", False), (4, "bf16", "bf16", True),
                                                    (2, "bf16", "fp8_e4m3", True)])
def test_output_is_bit_identical_under_block_permutation(G, dtype, kv_dtype, beams):
    # Physical placement never changes the result, also where sequences share blocks.
    cfg = (_beam_cfg(G, kv_dtype) if beams else
           small_cfg(G, 128, dtype, kv_dtype, S=8, ctx=("uniform", 1, 400), max_ctx=400))
    b = device_batch(cfg)
    h = HostBatch(b)
    say(cfg.name, "placement")
    a_out = gpu_step(b)
    if beams:
        kc0, vc0 = oracle_caches_after_step(h)
        assert max_err(a_out, oracle_decode(h, kc0, vc0)) <= tol(cfg)
    perm = torch.randperm(cfg.num_blocks, generator=torch.Generator().manual_seed(3)).cuda()
    kc = torch.empty_like(b.k_cache)
    vc = torch.empty_like(b.v_cache)
    kc[perm] = b.k_cache
    vc[perm] = b.v_cache
    b.block_tables = perm.to(torch.int32)[b.block_tables.long()].contiguous()
    b_out = gpu_decode(b, k_cache=kc, v_cache=vc)
    again = gpu_decode(b, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    assert torch.equal(a_out.view(torch.int16), b_out.view(torch.int16))
    assert torch.equal(b_out.view(torch.int16), again.view(torch.int16))   # deterministic


@pytest.mark.parametrize("partition", [0, 64])
@pytest.mark.parametrize("G,kv_dtype", [(4, "bf16"), (4, "fp8_e4m3"), (1, "bf16"), (1, "fp8_e4m3")])
def test_shared_prefix_blocks_equal_private_copies(G, kv_dtype, partition):
    # Beams reading shared prefix blocks give the same outputs as beams reading private
    # copies of every block. With one query head per kv head the kernel reads shared and
    # private blocks with different cache policies and pipelines but the same arithmetic,
    # so the outputs are bit-identical. With grouped heads, a workgroup whose sequences
    # share blocks reads each shared block once for all of them and splits the work over
    # its wavefronts (another summation order), so there the two agree within tolerance.
    cfg = WorkloadConfig(name="beam_small", num_seqs=8, num_q_heads=2 * G, num_kv_heads=2, head_dim=128,
                         num_blocks=1024, seed=11, dtype="bf16", kv_dtype=kv_dtype, ctx=("beam", 64, 0, 40, 4),
                         max_context_len=64 + 40 + 1, kv_scale=(1 / 128 if kv_dtype == "fp8_e4m3" else 1.0))
    b = device_batch(cfg)
    h = HostBatch(b)
    assert len(h.copy_pairs) > 0
    say(cfg.name, G, kv_dtype, "partition", partition, "shared vs private")
    shared = gpu_step(b, partition)
    torch.cuda.synchronize()
    kc, vc = oracle_caches_after_step(h)
    assert max_err(shared, oracle_decode(h, kc, vc)) <= tol(cfg)
    # private copies: give every (sequence, logical block) its own fresh physical block
    bt = b.block_tables.cpu().numpy()
    nb = -(-b.context_lens.cpu().numpy() // 16)
    used = set(int(x) for s in range(cfg.num_seqs) for x in bt[s, :nb[s]])
    used.add(b.layout.poison_block)
    free = [x for x in range(cfg.num_blocks) if x not in used]
    new_bt = bt.copy()
    src, dst = [], []
    for s in range(cfg.num_seqs):
        for j in range(nb[s]):
            f = free.pop()
            src.append(int(bt[s, j]))
            dst.append(f)
            new_bt[s, j] = f
    idx_s = torch.tensor(src, device="cuda")
    idx_d = torch.tensor(dst, device="cuda")
    b.k_cache[idx_d] = b.k_cache[idx_s]
    b.v_cache[idx_d] = b.v_cache[idx_s]
    b.block_tables = torch.from_numpy(new_bt).cuda()
    private = gpu_decode(b, partition_size=partition)
    torch.cuda.synchronize()
    if G == 1:
        assert torch.equal(shared.view(torch.int16), private.view(torch.int16))
    else:
        assert (shared.float() - private.float()).abs().max().item() <= tol(cfg)
    assert max_err(private, oracle_decode(h, kc, vc)) <= tol(cfg)


def test_fp8_cache_over_every_finite_code():
    cfg = small_cfg(4, 128, "bf16", "fp8_e4m3", S=6, ctx=("uniform", 20, 300), max_ctx=300)
    b = device_batch(cfg)
    g = torch.Generator().manual_seed(5)
    valid = torch.from_numpy(b.layout.history_valid)[:, None, :, None].expand(b.k_cache.shape).cuda()
    for cache in (b.k_cache, b.v_cache):
        codes = torch.randint(0, 254, cache.shape, generator=g, dtype=torch.int32)
        codes = torch.where(codes >= 0x7F, codes + 1, codes).to(torch.uint8).cuda()   # skip 0x7F, 0xFF
        cache.copy_(torch.where(valid, codes, cache))
    h = HostBatch(b)
    say(cfg.name, "all fp8 codes")
    out = gpu_step(b)
    torch.cuda.synchronize()
    kc, vc = oracle_caches_after_step(h)
    assert max_err(out, oracle_decode(h, kc, vc)) <= tol(cfg)


@pytest.mark.parametrize("partition", [0, 32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,kv_dtype,tail,width,S", [(2, "bf16", 40, 4, 16), (4, "bf16", 40, 4, 16),
                                                     (4, "fp8_e4m3", 40, 4, 16), (8, "bf16", 40, 4, 16),
                                                     (4, "bf16", 0, 4, 16), (2, "fp8_e4m3", 17, 4, 16),
                                                     (4, "bf16", 30, 2, 10), (16, "bf16", 40, 4, 8),
                                                     (3, "bf16", 40, 4, 16), (5, "bf16", 40, 3, 15),
                                                     (5, "fp8_e4m3", 25, 4, 16), (6, "bf16", 40, 2, 12),
                                                     (7, "bf16", 20, 4, 16), (12, "fp8_e4m3", 40, 4, 8)])
def test_sharing_groups_match_oracle(G, kv_dtype, tail, width, S, D, partition):
    # Workgroups of neighbouring sequences that share blocks read each shared block once
    # for all of them; every sharing pattern the beam generator makes (whole prefixes,
    # tails shared by children of one parent, no private tail at all) against the oracle.
    # Width-2 beams in workgroups of 4 put two requests in one workgroup and leave a
    # partial last workgroup (independent mode); 16 heads per kv head leave one sequence
    # per workgroup (shared blocks then take the cached path). Groups of 3, 5, 6 and 7
    # heads give workgroups of 4, 3, 2 and 2 sequences with partly filled columns; beams
    # of width 3 with 3-sequence workgroups put each request in a workgroup of its own.
    cfg = WorkloadConfig(name=f"groups_G{G}_{kv_dtype}_D{D}_t{tail}_w{width}", num_seqs=S, num_q_heads=2 * G,
                         num_kv_heads=2, head_dim=D, num_blocks=2048, seed=31 + G + tail, dtype="bf16",
                         kv_dtype=kv_dtype, ctx=("beam", 96, 0, tail, width), max_context_len=96 + tail + 1,
                         kv_scale=(1 / 128 if kv_dtype == "fp8_e4m3" else 1.0))
    b = device_batch(cfg)
    h = HostBatch(b)
    say(cfg.name, "partition", partition)
    out = gpu_step(b, partition)
    again = gpu_decode(b, partition_size=partition)
    torch.cuda.synchronize()
    kc, vc = oracle_caches_after_step(h)
    assert max_err(out, oracle_decode(h, kc, vc)) <= tol(cfg)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))   # deterministic


@pytest.mark.parametrize("partition", [0, 1024])
@pytest.mark.parametrize("G,kv_dtype", [(4, "fp8_e4m3"), (2, "bf16")])
def test_long_shared_prefix_groups_match_oracle(G, kv_dtype, partition):
    # A shared prefix of more logical blocks than one pass of a workgroup's wavefronts
    # lists at once (B wavefronts x 64 lanes), with diverged tails: the listing takes
    # several passes per wavefront, in one partition or in several.
    prompt, tail = 4496, 70
    cfg = WorkloadConfig(name=f"long_prefix_G{G}_{kv_dtype}", num_seqs=8, num_q_heads=2 * G, num_kv_heads=2,
                         head_dim=128, num_blocks=4096, seed=57 + G, dtype="bf16", kv_dtype=kv_dtype,
                         ctx=("beam", prompt, 0, tail, 4), max_context_len=prompt + tail + 1,
                         kv_scale=(1 / 128 if kv_dtype == "fp8_e4m3" else 1.0))
    b = device_batch(cfg)
    h = HostBatch(b)
    say(cfg.name, "partition", partition)
    out = gpu_step(b, partition)
    again = gpu_decode(b, partition_size=partition)
    torch.cuda.synchronize()
    kc, vc = oracle_caches_after_step(h)
    assert max_err(out, oracle_decode(h, kc, vc)) <= tol(cfg)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))   # deterministic


@pytest.mark.parametrize("partition", [0, 32768])
def test_very_long_contexts_match_oracle(partition):
    # Contexts of 200000 and 131073 tokens (12500 and 8193 blocks): the library's own
    # split (hundreds of partitions) and the longest partition it accepts.
    ctx = [200000, 131073]
    cfg = small_cfg(4, 128, "bf16", "bf16", S=2, Hkv=1, ctx=("fixed", ctx), max_ctx=200000, seed=13)
    _step_case(cfg, partition)


@pytest.mark.parametrize("G,Hkv", [(1, 40), (2, 24), (8, 12)])
def test_kv_head_counts_off_the_xcd_count_match_oracle(G, Hkv):
    # Work items run in runs of kv heads per XCD; head counts that are not multiples of 8
    # leave padded, partly empty runs at the end of the grid.
    cfg = small_cfg(G, 64, "bf16", "bf16", S=5, Hkv=Hkv, ctx=("uniform", 1, 150), max_ctx=150, seed=21)
    _step_case(cfg)
    _step_case(cfg, partition_size=64)


@pytest.mark.parametrize("G,Hkv,S", [(4, 3, 24), (2, 3, 24), (4, 3, 40), (4, 6, 24), (3, 5, 30)])
def test_every_work_item_of_a_short_xcd_run_is_launched(G, Hkv, S):
    # With 4-sequence workgroups the items run kv head fastest, Hkv per XCD in turn: the grid
    # must cover whole blocks of 8 * Hkv workgroups (3 kv heads, 6 groups and 3 partitions:
    # 54 items, which a grid padded to 64 only partly reached).
    cfg = small_cfg(G, 128, "bf16", "bf16", S=S, Hkv=Hkv, ctx=("uniform", 100, 150), max_ctx=150, seed=23)
    _step_case(cfg, partition_size=64)
    _step_case(cfg, partition_size=48)


@pytest.mark.parametrize("G,dtype,kv_dtype,S,partition", [(1, "f16", "f16", 6000, 0), (8, "bf16", "bf16", 4096, 0),
                                                          (4, "bf16", "fp8_e4m3", 5000, 16),
                                                          (2, "f16", "fp8_e4m3", 3001, 0)])
def test_batches_of_thousands_of_sequences_match_oracle(G, dtype, kv_dtype, S, partition):
    # Grids of thousands of workgroups (and, split into 16-token partitions, tens of
    # thousands of work items plus the reduce); short contexts keep the oracle quick.
    cfg = small_cfg(G, 128, dtype, kv_dtype, S=S, ctx=("uniform", 1, 64), max_ctx=64, seed=29)
    b = device_batch(cfg)
    h = HostBatch(b)
    say(cfg.name, "S", S, "partition", partition)
    out = gpu_step(b, partition)
    torch.cuda.synchronize()
    kc, vc = oracle_caches_after_step(h)
    np.testing.assert_array_equal(torch_bits(b.k_cache), kc)
    np.testing.assert_array_equal(torch_bits(b.v_cache), vc)
    err = max_err(out, oracle_decode(h, kc, vc))
    assert err <= tol(cfg), f"{cfg.name}: error {err} beyond the output's rounding"
