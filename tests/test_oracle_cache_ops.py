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
