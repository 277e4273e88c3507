"""Pins of the prefill-chunk oracle: causal SDPA, decode steps, chunk composition, brute force."""
import math

import numpy as np
import pytest
import torch

from oracle import attention, formats
from tests._paged import NAN16, f16_bits, scatter_to_pool

P = 16


def _pool(ks, vs, num_blocks=128, seed=0, perm=None):
    """Logical K/V rows per sequence ([ctx, Hkv, D] float) -> (k pool, v pool, tables, ctx)."""
    kb = [f16_bits(k) for k in ks]
    vb = [f16_bits(v) for v in vs]
    kp, tab = scatter_to_pool(kb, num_blocks, P, np.random.default_rng(seed), perm=perm)
    vp, tab2 = scatter_to_pool(vb, num_blocks, P, np.random.default_rng(seed), perm=perm)
    assert (tab == tab2).all()
    return kp, vp, tab, np.array([len(k) for k in ks], dtype=np.int32)


def _qsl(chunks):
    return np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)


def _case(seed, ctxs, chunks, Hkv=2, G=2, D=32):
    rng = np.random.default_rng(seed)
    ks = [rng.standard_normal((c, Hkv, D)) for c in ctxs]
    vs = [rng.standard_normal((c, Hkv, D)) for c in ctxs]
    q = f16_bits(rng.standard_normal((sum(chunks), Hkv * G, D)))
    return q, ks, vs


@pytest.mark.parametrize("G", [1, 4])
def test_whole_prompt_equals_causal_sdpa(G):
    # A chunk that is the whole prompt is ordinary causal self-attention: torch's
    # scaled_dot_product_attention(is_causal=True) in float64 on the contiguous sequence.
    Hkv, D = 2, 32
    ctxs = [1, 16, 37, 70]
    q, ks, vs = _case(G, ctxs, ctxs, Hkv, G, D)
    kp, vp, tab, ctx = _pool(ks, vs)
    qsl = _qsl(ctxs)
    out = attention.paged_prefill_attention(q, kp, vp, tab, ctx, qsl, 0.2, "f16", "f16")
    for s, c in enumerate(ctxs):
        qq = torch.from_numpy(formats.f16_to_f64(q[qsl[s]:qsl[s + 1]])).permute(1, 0, 2)      # [Hq,c,D]
        kk = torch.from_numpy(formats.f16_to_f64(f16_bits(ks[s]))).permute(1, 0, 2).repeat_interleave(G, 0)
        vv = torch.from_numpy(formats.f16_to_f64(f16_bits(vs[s]))).permute(1, 0, 2).repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True,
                                                               scale=float(np.float32(0.2)))
        np.testing.assert_allclose(out[qsl[s]:qsl[s + 1]], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_chunk_after_cached_prefix_equals_sdpa_with_shifted_mask():
    # A chunk of n tokens after `prefix` cached ones: row i sees keys 0 .. prefix + i, which
    # is the lower triangle of the [n, ctx] score matrix shifted right by `prefix` (torch.tril).
    Hkv, G, D = 2, 4, 32
    ctxs, chunks = [40, 33, 90], [7, 33, 16]
    q, ks, vs = _case(3, ctxs, chunks, Hkv, G, D)
    kp, vp, tab, ctx = _pool(ks, vs)
    qsl = _qsl(chunks)
    out = attention.paged_prefill_attention(q, kp, vp, tab, ctx, qsl, 0.25, "f16", "f16")
    for s, (c, n) in enumerate(zip(ctxs, chunks)):
        mask = torch.ones(n, c, dtype=torch.bool).tril(diagonal=c - n)
        qq = torch.from_numpy(formats.f16_to_f64(q[qsl[s]:qsl[s + 1]])).permute(1, 0, 2)
        kk = torch.from_numpy(formats.f16_to_f64(f16_bits(ks[s]))).permute(1, 0, 2).repeat_interleave(G, 0)
        vv = torch.from_numpy(formats.f16_to_f64(f16_bits(vs[s]))).permute(1, 0, 2).repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=0.25)
        np.testing.assert_allclose(out[qsl[s]:qsl[s + 1]], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_chunk_rows_equal_one_decode_step_each():
    # New token i of a chunk is what a decode step at context prefix + i + 1 would compute.
    ctxs, chunks = [17, 50, 64], [17, 9, 1]
    q, ks, vs = _case(4, ctxs, chunks)
    kp, vp, tab, ctx = _pool(ks, vs)
    qsl = _qsl(chunks)
    out = attention.paged_prefill_attention(q, kp, vp, tab, ctx, qsl, 0.3, "f16", "f16")
    for s, (c, n) in enumerate(zip(ctxs, chunks)):
        for i in range(n):
            row = qsl[s] + i
            step = attention.paged_decode_attention(q[row:row + 1], kp, vp, tab[s:s + 1],
                                                    np.array([c - n + i + 1]), 0.3, "f16", "f16")
            np.testing.assert_array_equal(out[row], step[0])


def test_chunks_compose_into_one_prefill():
    # Prefilling a 53-token prompt in chunks of 20 and 33 gives the rows of one 53-token
    # prefill; while the first chunk runs, the slots of the later tokens still hold NaN.
    Hkv, G, D = 2, 2, 32
    rng = np.random.default_rng(6)
    k = rng.standard_normal((53, Hkv, D))
    v = rng.standard_normal((53, Hkv, D))
    q = f16_bits(rng.standard_normal((53, Hkv * G, D)))
    kp, vp, tab, _ = _pool([k], [v])
    whole = attention.paged_prefill_attention(q, kp, vp, tab, [53], [0, 53], 0.2, "f16", "f16")
    kp1, vp1 = kp.copy(), vp.copy()
    for t in range(20, 53):
        kp1[tab[0, t // P], :, t % P] = NAN16
        vp1[tab[0, t // P], :, t % P] = NAN16
    first = attention.paged_prefill_attention(q[:20], kp1, vp1, tab, [20], [0, 20], 0.2, "f16", "f16")
    second = attention.paged_prefill_attention(q[20:], kp, vp, tab, [53], [0, 33], 0.2, "f16", "f16")
    np.testing.assert_array_equal(np.concatenate([first, second]), whole)


def test_rows_ignore_tokens_after_their_position():
    # Changing the K/V of position p changes exactly the rows at positions >= p.
    ctxs, chunks = [45], [30]
    q, ks, vs = _case(8, ctxs, chunks)
    kp, vp, tab, ctx = _pool(ks, vs)
    base = attention.paged_prefill_attention(q, kp, vp, tab, ctx, [0, 30], 0.3, "f16", "f16")
    p = 31                                  # chunk row 16
    ks[0][p] += 1.0
    vs[0][p] -= 2.0
    kp2, vp2, _, _ = _pool(ks, vs)
    moved = attention.paged_prefill_attention(q, kp2, vp2, tab, ctx, [0, 30], 0.3, "f16", "f16")
    row = p - (45 - 30)
    np.testing.assert_array_equal(moved[:row], base[:row])
    assert (np.abs(moved[row:] - base[row:]).max(axis=(1, 2)) > 1e-6).all()


def test_prefill_matches_scalar_loops():
    # Brute force with math.exp on a tiny batch with cached prefixes.
    Hkv, G, D = 2, 2, 8
    ctxs, chunks = [5, 19, 33], [5, 3, 17]
    q, ks, vs = _case(9, ctxs, chunks, Hkv, G, D)
    kp, vp, tab, ctx = _pool(ks, vs)
    qsl = _qsl(chunks)
    sc = float(np.float32(0.7))
    out = attention.paged_prefill_attention(q, kp, vp, tab, ctx, qsl, 0.7, "f16", "f16")
    for s, (c, n) in enumerate(zip(ctxs, chunks)):
        K = formats.f16_to_f64(f16_bits(ks[s]))
        V = formats.f16_to_f64(f16_bits(vs[s]))
        for i in range(n):
            qs = formats.f16_to_f64(q[qsl[s] + i])
            seen = c - n + i + 1
            for h in range(Hkv * G):
                g = h // G
                z = [sc * sum(qs[h, d] * K[t, g, d] for d in range(D)) for t in range(seen)]
                m = max(z)
                e = [math.exp(x - m) for x in z]
                tot = sum(e)
                for d in range(D):
                    ref = sum(e[t] * V[t, g, d] for t in range(seen)) / tot
                    assert abs(out[qsl[s] + i, h, d] - ref) <= 1e-12


def test_prefill_is_invariant_under_physical_placement():
    ctxs, chunks = [33, 70], [20, 64]
    q, ks, vs = _case(10, ctxs, chunks)
    qsl = _qsl(chunks)
    res = []
    for seed in (1, 2):
        kp, vp, tab, ctx = _pool(ks, vs, perm=np.random.default_rng(seed).permutation(128))
        res.append(attention.paged_prefill_attention(q, kp, vp, tab, ctx, qsl, 0.2, "f16", "f16"))
    np.testing.assert_array_equal(res[0], res[1])
    assert np.isfinite(res[0]).all()


def test_empty_chunks_and_bad_offsets():
    ctxs, chunks = [10, 20, 30], [0, 4, 0]
    q, ks, vs = _case(11, ctxs, chunks)
    kp, vp, tab, ctx = _pool(ks, vs)
    out = attention.paged_prefill_attention(q, kp, vp, tab, ctx, _qsl(chunks), 0.2, "f16", "f16")
    assert out.shape == (4, 4, 32) and np.isfinite(out).all()
    with pytest.raises(ValueError):                      # a chunk longer than its context
        attention.paged_prefill_attention(q, kp, vp, tab, [10, 3, 30], _qsl(chunks), 0.2, "f16", "f16")
    with pytest.raises(ValueError):                      # offsets that fall
        attention.paged_prefill_attention(q, kp, vp, tab, ctx, [0, 4, 2, 4], 0.2, "f16", "f16")


def test_fp8_prefill_reads_scaled_values():
    # With every V code 0x38 (1.0) the output is v_scale, whatever the keys.
    q = f16_bits(np.random.default_rng(0).standard_normal((5, 2, 64)))
    kp = np.random.default_rng(1).integers(0, 0x70, size=(4, 1, P, 64)).astype(np.uint8)
    vp = np.full((4, 1, P, 64), 0x38, dtype=np.uint8)
    out = attention.paged_prefill_attention(q, kp, vp, np.array([[2, 1]]), [20], [0, 5], 0.125,
                                            "f16", "fp8_e4m3", k_scale=0.5, v_scale=0.0078125)
    np.testing.assert_allclose(out, 0.0078125, rtol=1e-14, atol=0)
