"""Pins of the attention oracle against closed forms, invariants, a library routine and brute force."""
import math

import numpy as np
import pytest
import torch

from oracle import attention, formats
from tests._paged import f16_bits, scatter_to_pool

P = 16


def _oracle_f16(q, ks, vs, scale, num_blocks=64, seed=0, perm=None):
    """q [S,Hq,D] float; ks/vs list of [ctx,Hkv,D] float -> oracle output via a paged pool."""
    rng = np.random.default_rng(seed)
    kb = [f16_bits(k) for k in ks]
    vb = [f16_bits(v) for v in vs]
    kpool, tables = scatter_to_pool(kb, num_blocks, P, rng, perm=perm)
    vpool, tables2 = scatter_to_pool(vb, num_blocks, P, np.random.default_rng(seed), perm=perm)
    assert (tables == tables2).all()
    ctx = np.array([len(k) for k in ks], dtype=np.int32)
    return attention.paged_decode_attention(f16_bits(q), kpool, vpool, tables, ctx, scale, "f16", "f16")


def test_single_token_context_returns_its_value_row():
    # P1: one token -> softmax weight exactly 1 -> output is V[0].
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, 2, 64))
    ks = [rng.standard_normal((1, 2, 64)) for _ in range(3)]
    vs = [rng.standard_normal((1, 2, 64)) for _ in range(3)]
    out = _oracle_f16(q, ks, vs, 0.125)
    for s in range(3):
        np.testing.assert_array_equal(out[s], formats.f16_to_f64(f16_bits(vs[s][0])))


@pytest.mark.parametrize("ctx", [1, 2, 15, 16, 17, 31, 32, 33, 37, 100])
def test_zero_keys_give_the_mean_of_the_values(ctx):
    # P2: K == 0 -> uniform weights; V[t, :] = t -> every output element is (ctx-1)/2.
    Hkv, G, D = 2, 2, 64
    q = np.random.default_rng(ctx).standard_normal((1, Hkv * G, D))
    ks = [np.zeros((ctx, Hkv, D))]
    vs = [np.broadcast_to(np.arange(ctx, dtype=np.float64)[:, None, None], (ctx, Hkv, D)).copy()]
    out = _oracle_f16(q, ks, vs, 1.0)
    np.testing.assert_allclose(out, (ctx - 1) / 2.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("needle", [0, 14, 15, 16, 17, 31, 32, 47])
def test_needle_key_selects_its_value_across_block_boundaries(needle):
    # P3: one key aligned with q and much larger than the rest -> output ~ V[needle].
    rng = np.random.default_rng(needle)
    ctx, D = 48, 64
    q = rng.standard_normal((1, 1, D))
    k = 0.01 * rng.standard_normal((ctx, 1, D))
    k[needle, 0] = 8.0 * q[0, 0] / np.linalg.norm(q[0, 0]) * 8.0
    v = rng.standard_normal((ctx, 1, D))
    out = _oracle_f16(q, [k], [v], 1.0 / 8.0)
    target = formats.f16_to_f64(f16_bits(v[needle, 0]))
    # logit gap >= 64*|q|/8 - small; residual weight e^-gap is far below 1e-6.
    np.testing.assert_allclose(out[0, 0], target, atol=1e-6)
    others = [formats.f16_to_f64(f16_bits(v[t, 0])) for t in range(ctx) if t != needle]
    assert min(np.abs(out[0, 0] - o).max() for o in others) > 1e-3


def test_output_is_invariant_under_physical_placement():
    # P4: the same logical K/V under two placements gives bit-identical outputs.
    rng = np.random.default_rng(7)
    ctxs = [5, 16, 33, 70]
    q = rng.standard_normal((4, 4, 64))
    ks = [rng.standard_normal((c, 2, 64)) for c in ctxs]
    vs = [rng.standard_normal((c, 2, 64)) for c in ctxs]
    a = _oracle_f16(q, ks, vs, 0.125, num_blocks=128, perm=np.random.default_rng(1).permutation(128))
    b = _oracle_f16(q, ks, vs, 0.125, num_blocks=128, perm=np.random.default_rng(2).permutation(128))
    c = _oracle_f16(q, ks, vs, 0.125, num_blocks=128, perm=np.arange(128))
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)


@pytest.mark.parametrize("G", [1, 4, 8])
def test_paged_equals_contiguous_sdpa(G):
    # P5: gather + attention == torch's scaled_dot_product_attention on the contiguous
    # sequence, in float64 on the CPU (grouped heads expanded explicitly).
    rng = np.random.default_rng(G)
    Hkv, D = 2, 64
    ctxs = [1, 15, 16, 37, 129]
    q = rng.standard_normal((len(ctxs), Hkv * G, D))
    ks = [rng.standard_normal((c, Hkv, D)) for c in ctxs]
    vs = [rng.standard_normal((c, Hkv, D)) for c in ctxs]
    scale = 1.0 / math.sqrt(D)
    out = _oracle_f16(q, ks, vs, scale, num_blocks=128)
    for s, c in enumerate(ctxs):
        qq = torch.from_numpy(formats.f16_to_f64(f16_bits(q[s])))[:, None, :]           # [Hq,1,D]
        kk = torch.from_numpy(formats.f16_to_f64(f16_bits(ks[s]))).permute(1, 0, 2)     # [Hkv,c,D]
        vv = torch.from_numpy(formats.f16_to_f64(f16_bits(vs[s]))).permute(1, 0, 2)
        kk = kk.repeat_interleave(G, dim=0)
        vv = vv.repeat_interleave(G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, scale=float(np.float32(scale)))[:, 0, :].numpy()
        np.testing.assert_allclose(out[s], ref, rtol=0, atol=1e-12)


def test_shared_prefix_blocks_equal_private_copies():
    # P6: beams pointing at the same prefix blocks (refcount 4) read exactly what
    # fully private copies of those blocks would give.
    rng = np.random.default_rng(11)
    Hkv, G, D, prefix = 2, 2, 64, 40
    pre_k = f16_bits(rng.standard_normal((prefix, Hkv, D)))
    pre_v = f16_bits(rng.standard_normal((prefix, Hkv, D)))
    tails = [3, 0, 9, 24]
    tk = [f16_bits(rng.standard_normal((t, Hkv, D))) for t in tails]
    tv = [f16_bits(rng.standard_normal((t, Hkv, D))) for t in tails]
    q = f16_bits(rng.standard_normal((4, Hkv * G, D)))
    # private: every beam has its own copy of the prefix
    kb = [np.concatenate([pre_k, t]) for t in tk]
    vb = [np.concatenate([pre_v, t]) for t in tv]
    kp, tab = scatter_to_pool(kb, 64, P, np.random.default_rng(3))
    vp, _ = scatter_to_pool(vb, 64, P, np.random.default_rng(3))
    ctx = np.array([len(x) for x in kb], dtype=np.int32)
    private = attention.paged_decode_attention(q, kp, vp, tab, ctx, 0.125, "f16", "f16")
    # shared: the first 2 full prefix blocks are shared (the partial third one is copied per beam)
    shared_tab = tab.copy()
    shared_tab[:, 0] = tab[0, 0]
    shared_tab[:, 1] = tab[0, 1]
    kp2, vp2 = kp.copy(), vp.copy()
    for s in range(1, 4):  # stale data where the private prefix copies used to be
        for j in range(2):
            kp2[tab[s, j]] = np.uint16(0x7E00)
            vp2[tab[s, j]] = np.uint16(0x7E00)
    shared = attention.paged_decode_attention(q, kp2, vp2, shared_tab, ctx, 0.125, "f16", "f16")
    np.testing.assert_array_equal(private, shared)
    assert np.isfinite(shared).all()


def test_vectorised_oracle_matches_scalar_loops():
    # P7: brute force with math.exp on a tiny batch.
    rng = np.random.default_rng(5)
    Hkv, G, D = 2, 2, 8
    ctxs = [1, 15, 16, 37]
    q = rng.standard_normal((4, Hkv * G, D))
    ks = [rng.standard_normal((c, Hkv, D)) for c in ctxs]
    vs = [rng.standard_normal((c, Hkv, D)) for c in ctxs]
    scale = 0.3
    out = _oracle_f16(q, ks, vs, scale)
    sc = float(np.float32(scale))
    for s, c in enumerate(ctxs):
        qs = formats.f16_to_f64(f16_bits(q[s]))
        K = formats.f16_to_f64(f16_bits(ks[s]))
        V = formats.f16_to_f64(f16_bits(vs[s]))
        for h in range(Hkv * G):
            g = h // G
            z = [sc * sum(qs[h, d] * K[t, g, d] for d in range(D)) for t in range(c)]
            m = max(z)
            e = [math.exp(x - m) for x in z]
            tot = sum(e)
            for d in range(D):
                ref = sum(e[t] * V[t, g, d] for t in range(c)) / tot
                assert abs(out[s, h, d] - ref) <= 1e-12


def test_zero_length_context_outputs_zero():
    q = f16_bits(np.ones((2, 2, 64)))
    pool = np.full((4, 2, P, 64), np.uint16(0x7E00), dtype=np.uint16)
    tables = np.zeros((2, 1), dtype=np.int32)
    out = attention.paged_decode_attention(q, pool, pool, tables, np.array([0, 0]), 0.125, "f16", "f16")
    assert (out == 0).all()


def test_stale_slots_never_reach_the_result():
    # Tail slots of the last block, unused blocks and block-table padding hold NaN.
    rng = np.random.default_rng(9)
    ks = [rng.standard_normal((c, 2, 64)) for c in (1, 15, 17)]
    vs = [rng.standard_normal((c, 2, 64)) for c in (1, 15, 17)]
    out = _oracle_f16(rng.standard_normal((3, 2, 64)), ks, vs, 0.125)
    assert np.isfinite(out).all()


def test_gqa_grouping_is_consecutive():
    # q head h reads kv head h // G: give the two kv heads constant, different values.
    D, G = 64, 4
    q = np.random.default_rng(0).standard_normal((1, 2 * G, D))
    k = np.zeros((20, 2, D))
    v = np.zeros((20, 2, D))
    v[:, 0, :] = 1.0
    v[:, 1, :] = -2.0
    out = _oracle_f16(q, [k], [v], 0.125)
    np.testing.assert_allclose(out[0, :G], 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(out[0, G:], -2.0, rtol=0, atol=1e-14)


def test_fp8_cache_reads_scaled_values():
    # An fp8 pool is read as decode(code) * scale: with every K code 0 and V code
    # 0x38 (= 1.0) the output is exactly v_scale.
    q = f16_bits(np.random.default_rng(0).standard_normal((1, 2, 64)))
    kp = np.zeros((4, 1, P, 64), dtype=np.uint8)
    vp = np.full((4, 1, P, 64), 0x38, dtype=np.uint8)
    out = attention.paged_decode_attention(q, kp, vp, np.array([[2, 1]]), np.array([20]), 0.125,
                                           "f16", "fp8_e4m3", k_scale=3.0, v_scale=0.0078125)
    np.testing.assert_allclose(out, 0.0078125, rtol=1e-14, atol=0)


@pytest.mark.parametrize("bounds", [[0, 512], [0, 100, 512], [0, 1, 2, 300, 511, 512], list(range(0, 513, 64))])
def test_partition_merge_reproduces_unsplit_softmax(bounds):
    # P10: splitting a context into partitions and merging their (m, l, o) pieces is exact.
    rng = np.random.default_rng(len(bounds))
    q = rng.standard_normal((4, 32))
    K = 3.0 * rng.standard_normal((512, 32))
    V = rng.standard_normal((512, 32))
    ref = attention.softmax_attention(q, K, V, 0.2)
    pieces = [attention.partition_stats(q, K[a:b], V[a:b], 0.2) for a, b in zip(bounds[:-1], bounds[1:])]
    merged = attention.merge_partitions([p[0] for p in pieces], [p[1] for p in pieces], [p[2] for p in pieces])
    np.testing.assert_allclose(merged, ref, rtol=0, atol=1e-12)


def test_physical_slot_follows_the_block_table():
    row = [7, 3, 11]
    assert attention.physical_slot(row, 0, 16) == (7, 0)
    assert attention.physical_slot(row, 15, 16) == (7, 15)
    assert attention.physical_slot(row, 16, 16) == (3, 0)
    assert attention.physical_slot(row, 36, 16) == (11, 4)


@pytest.mark.parametrize("block_size", [32, 64])
def test_block_size_changes_only_where_tokens_live(block_size):
    # The same logical K/V in pools of 16-, 32- and 64-token blocks ("vLLM 推理优化技术深度
    # 调研报告", 维度四.5 weighs these sizes) gives the same attention, bit for bit.
    rng = np.random.default_rng(block_size)
    ctxs = [1, 31, 33, 64, 65, 130]
    q = f16_bits(rng.standard_normal((len(ctxs), 4, 32)))
    kb = [f16_bits(rng.standard_normal((c, 2, 32))) for c in ctxs]
    vb = [f16_bits(rng.standard_normal((c, 2, 32))) for c in ctxs]
    outs = []
    for P in (16, block_size):
        kp, tab = scatter_to_pool(kb, 64 * 16 // P + 8, P, np.random.default_rng(1))
        vp, _ = scatter_to_pool(vb, 64 * 16 // P + 8, P, np.random.default_rng(1))
        assert kp.shape[2] == P
        outs.append(attention.paged_decode_attention(q, kp, vp, tab, np.array(ctxs), 0.2, "f16", "f16"))
    np.testing.assert_array_equal(outs[0], outs[1])
