"""Pins of oracle.cache: the pool layout, the slot scatter and the table gather."""

import json
import os

import numpy as np

from oracle import cache
from oracle.block_manager import BlockManagerModel

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cache_layout_tiny.json")))


def test_layout_fixture():
    g = GOLD
    NB, H, B, D = g["num_blocks"], g["hkv"], g["block_size"], g["head_dim"]
    T = len(g["slots"])
    t, h, d = np.meshgrid(np.arange(T), np.arange(H), np.arange(D), indexing="ij")
    key = (100 * t + 10 * h + d + 1).astype(np.int32)
    k = np.zeros((NB, H, B, D), np.int32)
    v = np.zeros((NB, H, D, B), np.int32)
    cache.write_kv(k, v, key, -key, g["slots"], B)
    want_k = np.zeros(k.size, np.int32)
    for off, val in g["k_flat_nonzero"].items():
        want_k[int(off)] = val
    want_v = np.zeros(v.size, np.int32)
    for off, val in g["v_flat_nonzero"].items():
        want_v[int(off)] = val
    assert np.array_equal(k.reshape(-1), want_k)
    assert np.array_equal(v.reshape(-1), want_v)


def test_negative_slot_writes_nothing():
    k = np.full((2, 1, 4, 2), 7, np.int16)
    v = np.full((2, 1, 2, 4), 7, np.int16)
    cache.write_kv(k, v, np.ones((2, 1, 2), np.int16), np.ones((2, 1, 2), np.int16), [-1, -5], 4)
    assert (k == 7).all() and (v == 7).all()


def test_copy_blocks_whole_block():
    rng = np.random.default_rng(0)
    k = rng.integers(0, 1000, (5, 2, 4, 3))
    v = rng.integers(0, 1000, (5, 2, 3, 4))
    k0, v0 = k.copy(), v.copy()
    cache.copy_blocks(k, v, [(1, 3), (4, 0)])
    assert np.array_equal(k[3], k0[1]) and np.array_equal(v[3], v0[1])
    assert np.array_equal(k[0], k0[4]) and np.array_equal(v[0], v0[4])
    for b in (1, 2, 4):
        assert np.array_equal(k[b], k0[b]) and np.array_equal(v[b], v0[b])


def test_write_then_gather_round_trip_through_block_manager():
    # Writing each token at the slot the block manager gives it and reading it
    # back through the table returns the logical sequence, for any free order,
    # with copy-on-write in between; unused slots are never read (NaN poison).
    rng = np.random.default_rng(3)
    B, H, D, NB = 4, 2, 3, 64
    bm = BlockManagerModel(NB, B, free_order=rng.permutation(NB))
    k = np.full((NB, H, B, D), np.nan)
    v = np.full((NB, H, D, B), np.nan)
    logical = {}

    def put(sid, slots):
        rows = rng.standard_normal((len(slots), H, D))
        cache.write_kv(k, v, rows, -rows, slots, B)
        logical.setdefault(sid, []).extend(rows)

    put(0, bm.add_seq(0, 9))
    bm.fork(0, 1)
    logical[1] = list(logical[0])
    for step in range(12):
        ids = [0, 1] if step % 3 else [1, 0]
        slots, pairs = bm.append_slots(ids, 1)
        if step == 0:
            assert len(pairs) == 1          # the shared, partly filled last block
        cache.copy_blocks(k, v, pairs)
        rows = rng.standard_normal((2, H, D))
        cache.write_kv(k, v, rows, -rows, slots, B)
        for sid, row in zip(ids, rows):
            logical[sid].append(row)
    rows_t, lens = bm.block_tables([0, 1], 16)
    for sid in (0, 1):
        K, V = cache.gather_sequence(k, v, rows_t[sid], lens[sid], B)
        want = np.stack(logical[sid])
        assert K.shape == want.shape
        assert np.array_equal(K, want) and np.array_equal(V, -want)


def test_swap_layout_and_round_trip():
    # Hand-checked layout: pool of 3 blocks, Hkv = 1, B = 2, D = 2; K block p holds
    # 10p + (0, 1, 2, 3) row-major, V block p holds 100 + 10p + (0, 1, 2, 3).
    k = (10 * np.arange(3)[:, None] + np.arange(4)).reshape(3, 1, 2, 2)
    v = (100 + 10 * np.arange(3)[:, None] + np.arange(4)).reshape(3, 1, 2, 2)
    host = cache.swap_out(k, v, [2, 0])
    assert host.tolist() == [[[20, 21, 22, 23], [120, 121, 122, 123]],
                             [[0, 1, 2, 3], [100, 101, 102, 103]]]
    # back into other blocks: block 1 receives old block 2, block 2 receives old block 0
    k2, v2 = k.copy(), v.copy()
    cache.swap_in(k2, v2, host, [1, 2])
    assert np.array_equal(k2[1], k[2]) and np.array_equal(v2[1], v[2])
    assert np.array_equal(k2[2], k[0]) and np.array_equal(v2[2], v[0])
    assert np.array_equal(k2[0], k[0]) and np.array_equal(v2[0], v[0])


def test_swap_preserves_what_the_table_reads():
    # a sequence swapped out and back in onto different blocks reads the same K/V
    rng = np.random.default_rng(5)
    NB, H, B, D = 12, 2, 4, 3
    k = rng.integers(0, 1 << 15, (NB, H, B, D)).astype(np.int16)
    v = rng.integers(0, 1 << 15, (NB, H, D, B)).astype(np.int16)
    model = BlockManagerModel(NB, B)
    model.add_seq(7, 10)                      # blocks 0, 1, 2
    rows, _ = model.block_tables([7], 3)
    K0, V0 = cache.gather_sequence(k, v, rows[0], 10, B)
    host = cache.swap_out(k, v, model.swap_out(7))
    model.add_seq(8, 12)                      # takes blocks 3, 4, 5 (front of the pool)
    k[[3, 4, 5]] = 0
    v[[3, 4, 5]] = 0
    model.free_seq(8)
    new = model.swap_in(7)                    # blocks 6, 7, 8
    assert new == [6, 7, 8]
    cache.swap_in(k, v, host, new)
    rows, _ = model.block_tables([7], 3)
    K1, V1 = cache.gather_sequence(k, v, rows[0], 10, B)
    assert np.array_equal(K0, K1) and np.array_equal(V0, V1)
