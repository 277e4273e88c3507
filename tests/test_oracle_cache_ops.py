"""Pins of the cache-write and copy-on-write oracles (definition vs element-wise brute force)."""
import numpy as np

from oracle import cache_ops, formats


def _pool(rng, nb=8, h=2, p=16, d=8, dtype=np.uint16):
    return rng.integers(0, 1 << (8 * np.dtype(dtype).itemsize), size=(nb, h, p, d)).astype(dtype)


def test_reshape_and_cache_writes_exactly_the_given_slots():
    rng = np.random.default_rng(0)
    kc, vc = _pool(rng), _pool(rng)
    T, H, D = 5, 2, 8
    k = rng.integers(0, 1 << 15, size=(T, H, D)).astype(np.uint16)
    v = rng.integers(0, 1 << 15, size=(T, H, D)).astype(np.uint16)
    slots = np.array([0, 17, -1, 127, 45])
    ko, vo = cache_ops.reshape_and_cache(k, v, slots, kc, vc, "bf16", "bf16")
    ek, ev = kc.copy(), vc.copy()
    flat_k = ek.transpose(0, 2, 1, 3).reshape(8 * 16, H, D)   # slot-major view, built independently
    flat_v = ev.transpose(0, 2, 1, 3).reshape(8 * 16, H, D)
    for i, s in enumerate(slots):
        if s >= 0:
            flat_k[s] = k[i]
            flat_v[s] = v[i]
    ek = flat_k.reshape(8, 16, H, D).transpose(0, 2, 1, 3)
    ev = flat_v.reshape(8, 16, H, D).transpose(0, 2, 1, 3)
    np.testing.assert_array_equal(ko, ek)
    np.testing.assert_array_equal(vo, ev)
    # inputs untouched
    assert not np.shares_memory(ko, kc)


def test_reshape_and_cache_fp8_quantises_each_element():
    rng = np.random.default_rng(1)
    kc = np.zeros((4, 2, 16, 8), dtype=np.uint8)
    vc = np.zeros((4, 2, 16, 8), dtype=np.uint8)
    x = rng.standard_normal((3, 2, 8)) * 3
    k = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # truncated to bf16 bits
    v = k[::-1].copy()
    ks, vs = 0.0134, 1 / 128
    ko, vo = cache_ops.reshape_and_cache(k, v, [3, 20, 63], kc, vc, "bf16", "fp8_e4m3", ks, vs)
    for i, s in enumerate([3, 20, 63]):
        b, o = divmod(s, 16)
        for h in range(2):
            for d in range(8):
                xk = formats.bf16_to_f64(k[i, h, d])
                want = formats.e4m3_encode(np.float64(np.float32(xk) / np.float32(ks)))
                assert ko[b, h, o, d] == want
                xv = formats.bf16_to_f64(v[i, h, d])
                assert vo[b, h, o, d] == formats.e4m3_encode(np.float64(np.float32(xv) / np.float32(vs)))
    touched = np.zeros((4, 16), bool)
    for s in [3, 20, 63]:
        touched[s // 16, s % 16] = True
    assert (ko.transpose(0, 2, 1, 3)[~touched] == 0).all()


def test_copy_blocks_copies_whole_blocks_for_every_layer():
    rng = np.random.default_rng(2)
    layers = 3
    ks = [_pool(rng, dtype=np.uint8) for _ in range(layers)]
    vs = [_pool(rng, dtype=np.uint8) for _ in range(layers)]
    pairs = np.array([[1, 5], [2, 6], [2, 7]])
    ko, vo = cache_ops.copy_blocks(ks, vs, pairs)
    for layer in range(layers):
        for b in range(8):
            src = {5: 1, 6: 2, 7: 2}.get(b, b)
            np.testing.assert_array_equal(ko[layer][b], ks[layer][src])
            np.testing.assert_array_equal(vo[layer][b], vs[layer][src])


def test_copy_blocks_empty_list_is_a_no_op():
    rng = np.random.default_rng(3)
    k, v = _pool(rng), _pool(rng)
    ko, vo = cache_ops.copy_blocks([k], [v], np.zeros((0, 2), dtype=np.int64))
    np.testing.assert_array_equal(ko[0], k)
    np.testing.assert_array_equal(vo[0], v)


def test_swap_blocks_moves_whole_blocks_between_two_pools():
    # Element-wise brute force over a flat byte view: every byte of a named destination block
    # comes from its source block, every other destination byte is unchanged, the source pool
    # is untouched.
    rng = np.random.default_rng(3)
    L = 3
    gk = [_pool(rng, nb=10) for _ in range(L)]
    gv = [_pool(rng, nb=10) for _ in range(L)]
    hk = [_pool(rng, nb=6) for _ in range(L)]
    hv = [_pool(rng, nb=6) for _ in range(L)]
    pairs = np.array([[9, 0], [2, 5], [4, 3]])
    gk0, hk0 = [g.copy() for g in gk], [h.copy() for h in hk]
    ko, vo = cache_ops.swap_blocks(gk, gv, hk, hv, pairs)
    per_block = 2 * 16 * 8
    for layer in range(L):
        for out, src, dst in ((ko, gk, hk), (vo, gv, hv)):
            o = out[layer].reshape(-1)
            s = src[layer].reshape(-1)
            d = dst[layer].reshape(-1)
            expect = d.copy()
            for a, b in pairs:
                for e in range(per_block):
                    expect[b * per_block + e] = s[a * per_block + e]
            np.testing.assert_array_equal(o, expect)
    assert all((a == b).all() for a, b in zip(gk + hk, gk0 + hk0))   # inputs untouched


def test_swap_out_and_back_in_restores_a_sequences_attention():
    # A preempted sequence's blocks go to host memory and come back into other GPU blocks;
    # with its block table pointed at the new blocks its attention output is unchanged,
    # bit for bit ("vLLM 是什么…", §五: swapping moves blocks, not values).
    from oracle import attention
    rng = np.random.default_rng(4)
    nb, H, D, ctx = 12, 2, 16, 37
    kc = (rng.standard_normal((nb, H, 16, D))).astype(np.float16).view(np.uint16)
    vc = (rng.standard_normal((nb, H, 16, D))).astype(np.float16).view(np.uint16)
    q = (rng.standard_normal((1, 2 * H, D))).astype(np.float16).view(np.uint16)
    table = np.array([[7, 2, 10]])
    before = attention.paged_decode_attention(q, kc, vc, table, [ctx], 0.25, "f16", "f16")
    host_k = np.zeros((4, H, 16, D), np.uint16)
    host_v = np.zeros((4, H, 16, D), np.uint16)
    out_pairs = np.array([[7, 3], [2, 0], [10, 1]])
    (hk,), (hv,) = cache_ops.swap_blocks([kc], [vc], [host_k], [host_v], out_pairs)
    wiped_k = np.full_like(kc, 0x7E00)          # the GPU blocks were reused meanwhile
    wiped_v = np.full_like(vc, 0x7E00)
    in_pairs = np.array([[3, 0], [0, 5], [1, 11]])
    (gk,), (gv,) = cache_ops.swap_blocks([hk], [hv], [wiped_k], [wiped_v], in_pairs)
    after = attention.paged_decode_attention(q, gk, gv, np.array([[0, 5, 11]]), [ctx], 0.25, "f16", "f16")
    np.testing.assert_array_equal(before, after)


def test_swap_within_one_pool_is_copy_on_write():
    rng = np.random.default_rng(5)
    k, v = [_pool(rng)], [_pool(rng)]
    pairs = np.array([[1, 6], [3, 0]])
    sk, sv = cache_ops.swap_blocks(k, v, k, v, pairs)
    ck, cv = cache_ops.copy_blocks(k, v, pairs)
    np.testing.assert_array_equal(sk[0], ck[0])
    np.testing.assert_array_equal(sv[0], cv[0])
