"""Pins of oracle.attention: library routine, brute force, closed forms, invariants."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import cache
from oracle.block_manager import BlockManagerModel


def rand(rng, *shape):
    return rng.standard_normal(shape)


def sdpa_decode(q, K, V, scale):
    """torch fp64 scaled_dot_product_attention on contiguous K/V (GQA expanded)."""
    Hq, Hkv = q.shape[0], K.shape[1]
    g = Hq // Hkv
    qt = torch.from_numpy(q)[:, None, :]                                  # [Hq, 1, D]
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, 0)    # [Hq, n, D]
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, 0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
    return o[:, 0, :].numpy()


@pytest.mark.parametrize("Hq,Hkv,D,n", [(4, 4, 8, 1), (4, 4, 64, 47), (8, 2, 16, 300),
                                         (16, 2, 32, 129), (6, 3, 5, 17)])
def test_decode_matches_torch_sdpa_fp64(Hq, Hkv, D, n):
    rng = np.random.default_rng(Hq * 1000 + n)
    q, K, V = rand(rng, Hq, D), rand(rng, n, Hkv, D), rand(rng, n, Hkv, D)
    scale = 1 / math.sqrt(D)
    got = att.dense_decode(q, K, V, scale)
    want = sdpa_decode(q, K, V, scale)
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def brute_force_decode(q, K, V, scale):
    """Scalar loops with math.exp / math.fsum: an independent restatement."""
    Hq, D = q.shape
    n, Hkv, _ = K.shape
    g = Hq // Hkv
    out = np.zeros((Hq, D))
    for h in range(Hq):
        kv = h // g
        scores = [scale * math.fsum(q[h, d] * K[j, kv, d] for d in range(D)) for j in range(n)]
        top = max(scores)
        e = [math.exp(x - top) for x in scores]
        z = math.fsum(e)
        for d in range(D):
            out[h, d] = math.fsum(e[j] * V[j, kv, d] for j in range(n)) / z
    return out


@pytest.mark.parametrize("seed", range(6))
def test_decode_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.integers(1, 3))
    D = int(rng.integers(1, 9))
    n = int(rng.integers(1, 41))
    q, K, V = rand(rng, Hq, D), rand(rng, n, Hkv, D), rand(rng, n, Hkv, D)
    scale = float(rng.uniform(0.1, 2.0))
    got = att.dense_decode(q, K, V, scale)
    want = brute_force_decode(q, K, V, scale)
    assert np.max(np.abs(got - want)) <= 1e-13 * max(1.0, np.max(np.abs(want)))


def test_closed_forms():
    rng = np.random.default_rng(5)
    D = 7
    # one token: the output is that token's value
    q, K, V = rand(rng, 3, D), rand(rng, 1, 3, D), rand(rng, 1, 3, D)
    assert np.array_equal(att.dense_decode(q, K, V, 0.3), V[0])
    # zero query (all scores equal): the mean of V
    n = 11
    K, V = rand(rng, n, 1, D), rand(rng, n, 1, D)
    got = att.dense_decode(np.zeros((2, D)), K, V, 0.5)
    assert np.allclose(got, V[:, 0, :].mean(0)[None, :], rtol=0, atol=1e-14)
    # identical keys: also the mean of V
    K = np.repeat(rand(rng, 1, 1, D), n, axis=0)
    got = att.dense_decode(rand(rng, 1, D), K, V, 0.5)
    assert np.allclose(got[0], V[:, 0, :].mean(0), rtol=0, atol=1e-14)
    # two tokens: weights are the logistic function of the score difference
    q, K, V = rand(rng, 1, D), rand(rng, 2, 1, D), rand(rng, 2, 1, D)
    s = 0.7
    x0, x1 = s * q[0] @ K[0, 0], s * q[0] @ K[1, 0]
    w0 = 1 / (1 + math.exp(-(x0 - x1)))
    assert np.allclose(att.dense_decode(q, K, V, s)[0], w0 * V[0, 0] + (1 - w0) * V[1, 0],
                       rtol=0, atol=1e-14)
    # constant values: the output is that constant
    V = np.full((n, 1, D), 2.5)
    assert np.allclose(att.dense_decode(rand(rng, 1, D), rand(rng, n, 1, D), V, 1.0), 2.5,
                       rtol=0, atol=1e-14)


def test_softmax_weights_sum_to_one():
    rng = np.random.default_rng(9)
    for n in (1, 2, 50, 3000):
        w, l = att.softmax_weights(rand(rng, 16), rand(rng, n, 16), 0.25)
        assert abs(w.sum() / l - 1) < 1e-12
        assert w.max() == 1.0 and (w > 0).all()


def _paged_setup(rng, S, Hq, Hkv, D, B, NB, lens):
    bm = BlockManagerModel(NB, B, free_order=rng.permutation(NB))
    k = np.full((NB, Hkv, B, D), np.nan)
    v = np.full((NB, Hkv, D, B), np.nan)
    logical = []
    for s, n in enumerate(lens):
        slots = bm.add_seq(s, n)
        K, V = rand(rng, n, Hkv, D), rand(rng, n, Hkv, D)
        cache.write_kv(k, v, K, V, slots, B)
        logical.append((K, V))
    maxb = max((n + B - 1) // B for n in lens)
    tables, ctx = bm.block_tables(range(S), maxb)
    return k, v, np.array(tables), np.array(ctx), logical


def test_paged_equals_dense_and_ignores_poison():
    rng = np.random.default_rng(11)
    S, Hq, Hkv, D, B = 4, 8, 2, 16, 16
    lens = [47, 612, 130, 1900]
    k, v, tables, ctx, logical = _paged_setup(rng, S, Hq, Hkv, D, B, 256, lens)
    q = rand(rng, S, Hq, D)
    got = att.paged_decode(q, k, v, tables, ctx, B, 0.25)
    assert np.isfinite(got).all()
    for s in range(S):
        assert np.array_equal(got[s], att.dense_decode(q[s], *logical[s], 0.25))


def test_layout_permutation_invariance_bitwise():
    # Paging leaves the attention result unchanged (tinycto FAQ): relabelling
    # the physical blocks changes nothing, bit for bit.
    rng = np.random.default_rng(12)
    S, Hq, Hkv, D, B, NB = 3, 4, 2, 8, 4, 80
    k, v, tables, ctx, _ = _paged_setup(rng, S, Hq, Hkv, D, B, NB, [5, 37, 64])
    q = rand(rng, S, Hq, D)
    base = att.paged_decode(q, k, v, tables, ctx, B, 0.5)
    pi = rng.permutation(NB)
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[pi] = k
    v2[pi] = v
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1)
    assert np.array_equal(att.paged_decode(q, k2, v2, t2, ctx, B, 0.5), base)


def test_merge_of_any_split_equals_unsplit():
    rng = np.random.default_rng(13)
    for n in (1, 2, 17, 500):
        q, K, V = rand(rng, 32), rand(rng, n, 32), rand(rng, n, 32)
        whole = att.dense_decode(q[None], K[:, None], V[:, None], 0.2)[0]
        for _ in range(5):
            cuts = sorted(set(rng.integers(1, n, size=min(n - 1, 4)).tolist())) if n > 1 else []
            bounds = [0] + cuts + [n]
            st = [att.partition_state(q, K[a:b], V[a:b], 0.2) for a, b in zip(bounds, bounds[1:])]
            ms, ls, os_ = zip(*st)
            got = att.merge_partitions(ms, ls, np.stack(os_))
            assert np.max(np.abs(got - whole)) <= 1e-13 * max(1, np.max(np.abs(whole)))


def test_chunk_of_one_is_decode():
    rng = np.random.default_rng(14)
    n, Hq, Hkv, D = 40, 4, 2, 8
    q, K, V = rand(rng, 1, Hq, D), rand(rng, n, Hkv, D), rand(rng, n, Hkv, D)
    assert np.array_equal(att.chunk_attend(q, K, V, 0.3)[0], att.dense_decode(q[0], K, V, 0.3))


def test_chunk_without_prefix_is_causal_sdpa():
    rng = np.random.default_rng(15)
    C, Hq, Hkv, D = 33, 4, 2, 16
    q, K, V = rand(rng, C, Hq, D), rand(rng, C, Hkv, D), rand(rng, C, Hkv, D)
    got = att.chunk_attend(q, K, V, 0.25)
    g = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, 0)
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, 0)
    want = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, is_causal=True,
                                                            scale=0.25).permute(1, 0, 2).numpy()
    assert np.max(np.abs(got - want)) <= 1e-12


def test_chunk_with_prefix_matches_masked_sdpa():
    rng = np.random.default_rng(16)
    C, P, Hq, Hkv, D = 20, 45, 8, 2, 16
    n = P + C
    q, K, V = rand(rng, C, Hq, D), rand(rng, n, Hkv, D), rand(rng, n, Hkv, D)
    got = att.chunk_attend(q, K, V, 0.25)
    g = Hq // Hkv
    mask = torch.arange(n)[None, :] <= (P + torch.arange(C))[:, None]       # [C, n]
    qt = torch.from_numpy(q).permute(1, 0, 2)
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, 0)
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, 0)
    want = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask,
                                                            scale=0.25).permute(1, 0, 2).numpy()
    assert np.max(np.abs(got - want)) <= 1e-12


def test_bf16_bits_exact():
    vals = np.array([0.0, 1.0, -2.5, 3.140625, 65280.0, -1e-3], dtype=np.float32)
    t = torch.from_numpy(vals).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(att.bf16_bits_to_f64(bits), t.to(torch.float64).numpy())


# -- paged_chunk_attend: the chunk of new tokens read through block tables ---------------
#
# Pins that do not go through chunk_attend's own arithmetic: a hand-computed case on a
# scattered pool, masked torch SDPA on the logical K/V, and bitwise invariance to relabelling
# the physical blocks.  The chunk is appended with the block manager model after a prefill
# that ends mid-block, so the chunk starts inside a shared-with-prefix block.

def _paged_chunk_setup(rng, S, Hkv, D, B, NB, cached, C):
    bm = BlockManagerModel(NB, B, free_order=rng.permutation(NB))
    k = np.full((NB, Hkv, B, D), np.nan)
    v = np.full((NB, Hkv, D, B), np.nan)
    logical = []
    for s in range(S):
        K, V = rand(rng, cached[s] + C, Hkv, D), rand(rng, cached[s] + C, Hkv, D)
        cache.write_kv(k, v, K[:cached[s]], V[:cached[s]], bm.add_seq(s, cached[s]), B)
        logical.append((K, V))
    slots, pairs = bm.append_slots(list(range(S)), C)
    assert not pairs
    for s in range(S):
        K, V = logical[s]
        cache.write_kv(k, v, K[cached[s]:], V[cached[s]:], slots[s * C:(s + 1) * C], B)
    maxb = max((n + C + B - 1) // B for n in cached)
    tables, ctx = bm.block_tables(range(S), maxb)
    return k, v, np.array(tables), np.array(ctx), logical


def test_paged_chunk_hand_case():
    # One head, D = 1, scale 1, B = 2; the sequence's three tokens live in physical blocks 5
    # and 2 of a NaN-filled pool.  Keys 0, ln 3, 0 and values 1, 2, 6: chunk row 0 (position
    # 1) weighs keys 0..1 as 1 : 3, row 1 (position 2) weighs keys 0..2 as 1 : 3 : 1.
    B, NB = 2, 8
    k = np.full((NB, 1, B, 1), np.nan)
    v = np.full((NB, 1, 1, B), np.nan)
    keys, vals = [0.0, math.log(3.0), 0.0], [1.0, 2.0, 6.0]
    for j, blk in enumerate([5, 5, 2]):
        k[blk, 0, j % B, 0] = keys[j]
        v[blk, 0, 0, j % B] = vals[j]
    tables = np.array([[5, 2, -1]])
    q = np.ones((1, 2, 1, 1))
    got = att.paged_chunk_attend(q, k, v, tables, np.array([3]), B, 1.0)
    assert np.allclose(got[0, :, 0, 0], [(1 + 3 * 2) / 4, (1 + 3 * 2 + 6) / 5], rtol=0, atol=1e-15)


def test_paged_chunk_matches_masked_sdpa_on_logical_kv():
    rng = np.random.default_rng(17)
    S, Hq, Hkv, D, B, C = 3, 8, 2, 16, 16, 21
    cached = [0, 37, 100]
    k, v, tables, ctx, logical = _paged_chunk_setup(rng, S, Hkv, D, B, 64, cached, C)
    assert list(ctx) == [n + C for n in cached]
    q = rand(rng, S, C, Hq, D)
    got = att.paged_chunk_attend(q, k, v, tables, ctx, B, 0.25)
    assert np.isfinite(got).all()
    g = Hq // Hkv
    for s in range(S):
        K, V = logical[s]
        n = K.shape[0]
        mask = torch.arange(n)[None, :] <= (cached[s] + torch.arange(C))[:, None]
        qt = torch.from_numpy(q[s]).permute(1, 0, 2)
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, 0)
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, 0)
        want = torch.nn.functional.scaled_dot_product_attention(
            qt, Kt, Vt, attn_mask=mask, scale=0.25).permute(1, 0, 2).numpy()
        assert np.max(np.abs(got[s] - want)) <= 1e-12
        assert np.array_equal(got[s], att.chunk_attend(q[s], K, V, 0.25))


def test_paged_chunk_layout_permutation_invariance_bitwise():
    rng = np.random.default_rng(18)
    S, Hq, Hkv, D, B, C, NB = 2, 4, 2, 8, 4, 9, 60
    k, v, tables, ctx, _ = _paged_chunk_setup(rng, S, Hkv, D, B, NB, [13, 30], C)
    q = rand(rng, S, C, Hq, D)
    base = att.paged_chunk_attend(q, k, v, tables, ctx, B, 0.5)
    pi = rng.permutation(NB)
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[pi] = k
    v2[pi] = v
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1)
    assert np.array_equal(att.paged_chunk_attend(q, k2, v2, t2, ctx, B, 0.5), base)
