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
