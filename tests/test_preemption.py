"""Preemption by swapping and truncation in the host block manager: libpa against the oracle's
integer model (bit-exact) and against hand-derived pins of the fixed policy.

"Taming the Tail", "Infrastructure Scale": when the pool runs out of physical blocks, a request
can be paused and its KV-cache moved to CPU RAM.  The policy details (which blocks, in which
order) are this library's fixed reading, stated in oracle/block_manager.py and include/pa.h."""

import random

import numpy as np
import pytest

from oracle.block_manager import BlockManagerModel
from oracle.block_manager import InvalidArg as ModelInvalid
from oracle.block_manager import OutOfBlocks as ModelOOB
from oracle.block_manager import Swapped as ModelSwapped

from test_block_manager import same_state


def same_swap_state(lib_bm, model):
    st, ms = lib_bm.stats(), model.stats()
    for k in ("swapped_seqs", "swapped_tokens", "swap_outs", "swap_ins"):
        assert st[k] == ms[k], k
    for s, n in model.swapped.items():
        assert lib_bm.seq_len(s) == n


def test_swap_and_truncate_pins(libpa):
    """A hand-traced script (pool of 8 blocks, B = 4, free order 0..7)."""
    bm = libpa.BlockManager(8, 4)
    model = BlockManagerModel(8, 4)
    for m in (bm, model):
        m.add_seq(1, 6)          # blocks [0, 1]
        m.fork(1, 2)             # counts 2, 2
        m.add_seq(3, 4)          # block [2]
    # swapping out a sequence that shares: its blocks come back in logical order, the shared
    # ones stay live (count 1), nothing joins the pool
    assert list(bm.swap_out(1)) == [0, 1] == model.swap_out(1)
    assert [bm.refcount(b) for b in (0, 1, 2)] == [1, 1, 1]
    assert list(bm.free_list()) == [3, 4, 5, 6, 7]
    # a private block joins the back of the pool
    assert list(bm.swap_out(3)) == [2] == model.swap_out(3)
    assert list(bm.free_list()) == [3, 4, 5, 6, 7, 2]
    # a swapped sequence keeps its length; everything else refuses it
    assert bm.seq_len(1) == 6 and list(bm.seq_lens([1, 2])) == [6, 6]
    with pytest.raises(libpa.Swapped):
        bm.block_tables([1], 4)
    with pytest.raises(libpa.Swapped):
        bm.append_slots([2, 1], 1)
    with pytest.raises(libpa.Swapped):
        bm.fork(1, 9)
    with pytest.raises(libpa.Swapped):
        bm.swap_out(1)
    with pytest.raises(libpa.SeqExists):
        bm.add_seq(1, 3)
    # swapping in takes ceil(6 / 4) = 2 fresh private blocks from the front
    assert list(bm.swap_in(1)) == [3, 4] == model.swap_in(1)
    t, l = bm.block_tables([1, 2], 2)
    assert t.tolist() == [[3, 4], [0, 1]] and list(l) == [6, 6]
    # truncating to 3 tokens keeps ceil(3 / 4) = 1 block; block 1 reaches count 0
    bm.truncate(2, 3)
    model.truncate(2, 3)
    assert list(bm.free_list()) == [5, 6, 7, 2, 1]
    # the kept block is private: the next token goes in place, position 3 of block 0
    slots, pairs = bm.append_slots([2], 1)
    assert list(slots) == [3] and len(pairs) == 0
    assert model.append_slots([2], 1) == ([3], [])
    # a truncated sequence that shares its kept partial block copies it on the next append
    for m in (bm, model):
        m.fork(2, 4)
        m.truncate(4, 2)
    slots, pairs = bm.append_slots([4], 1)
    assert list(slots) == [5 * 4 + 2] and [tuple(p) for p in pairs] == [(0, 5)]
    assert model.append_slots([4], 1) == ([22], [(0, 5)])
    assert list(bm.swap_in(3)) == [6] == model.swap_in(3)
    st = bm.stats()
    assert (st["swap_outs"], st["swap_ins"], st["swapped_seqs"]) == (2, 2, 0)
    same_state(bm, model, sorted(model.seqs))


def test_swap_errors_change_nothing(libpa):
    bm = libpa.BlockManager(6, 4)
    model = BlockManagerModel(6, 4)
    for m in (bm, model):
        m.add_seq(1, 9)   # 3 blocks
        m.add_seq(2, 8)   # 2 blocks
        m.swap_out(1)     # 3 blocks back to the pool
        m.add_seq(3, 12)  # takes them: the pool is empty
    before = (list(bm.free_list()), bm.stats())
    with pytest.raises(libpa.OutOfBlocks):
        bm.swap_in(1)
    with pytest.raises(ModelOOB):
        model.swap_in(1)
    with pytest.raises(libpa.PaError):
        bm.swap_in(2)                 # live, not swapped
    with pytest.raises(ModelInvalid):
        model.swap_in(2)
    with pytest.raises(libpa.UnknownSeq):
        bm.swap_out(77)
    with pytest.raises(libpa.PaError):
        bm.truncate(2, 9)             # longer than the sequence
    with pytest.raises(libpa.Swapped):
        bm.truncate(1, 2)
    with pytest.raises(ModelSwapped):
        model.truncate(1, 2)
    assert (list(bm.free_list()), bm.stats()) == before
    # freeing a swapped sequence just forgets it
    bm.free_seq(1)
    model.free_seq(1)
    same_state(bm, model, sorted(model.seqs))
    same_swap_state(bm, model)
    with pytest.raises(libpa.UnknownSeq):
        bm.seq_len(1)


def test_pool_exhaustion_forces_a_swap(libpa):
    """Decoding until the pool is full, the scheduler's choice ([TT] "Infrastructure Scale"):
    swap the longest sequence out, go on with the others, swap it back in once blocks are free."""
    B, NB = 16, 40
    bm = libpa.BlockManager(NB, B)
    lens = [100, 150, 180, 130]            # 7 + 10 + 12 + 9 = 38 blocks
    for i, n in enumerate(lens):
        bm.add_seq(i, n)
    live = [0, 1, 2, 3]
    steps = 0
    while True:
        try:
            bm.append_slots(live, 1)
            steps += 1
        except libpa.OutOfBlocks:
            break
    assert bm.stats()["free_blocks"] < len(live)
    victim = max(live, key=bm.seq_len)
    saved = bm.swap_out(victim)
    assert len(saved) == -(-bm.seq_len(victim) // B)
    live.remove(victim)
    bm.append_slots(live, 1)            # room again
    bm.free_seq(live.pop(0))            # a request finishes
    back = bm.swap_in(victim)
    assert len(back) == len(saved)
    assert bm.stats()["used_blocks"] + bm.stats()["free_blocks"] == NB


def test_random_ops_with_swap_and_truncate_bit_exact(libpa):
    rng = random.Random(4321)
    for B in (1, 4, 16):
        NB = 90
        order = rng.sample(range(NB), NB)
        bm = libpa.BlockManager(NB, B, order)
        model = BlockManagerModel(NB, B, order)
        next_id = 0
        for step in range(900):
            live = sorted(model.seqs)
            swapped = sorted(model.swapped)
            op = rng.random()
            if op < 0.15 or not live:
                n = rng.randrange(0, 3 * B + 3)
                try:
                    want = model.add_seq(next_id, n)
                except ModelOOB:
                    with pytest.raises(libpa.OutOfBlocks):
                        bm.add_seq(next_id, n)
                else:
                    assert list(bm.add_seq(next_id, n)) == want
                next_id += 1
            elif op < 0.25:
                p = rng.choice(live)
                model.fork(p, next_id)
                bm.fork(p, next_id)
                next_id += 1
            elif op < 0.55:
                ids = rng.sample(live, rng.randint(1, len(live)))
                k = rng.randint(0, 2 * B + 1)
                try:
                    want_slots, want_pairs = model.append_slots(ids, k)
                except ModelOOB:
                    with pytest.raises(libpa.OutOfBlocks):
                        bm.append_slots(ids, k)
                else:
                    slots, pairs = bm.append_slots(ids, k)
                    assert list(slots) == want_slots
                    assert [tuple(p) for p in pairs] == want_pairs
            elif op < 0.65:
                s = rng.choice(live)
                assert list(bm.swap_out(s)) == model.swap_out(s)
            elif op < 0.75 and swapped:
                s = rng.choice(swapped)
                try:
                    want = model.swap_in(s)
                except ModelOOB:
                    with pytest.raises(libpa.OutOfBlocks):
                        bm.swap_in(s)
                else:
                    assert list(bm.swap_in(s)) == want
            elif op < 0.87:
                s = rng.choice(live)
                keep = rng.randint(0, model.seqs[s].n)
                model.truncate(s, keep)
                bm.truncate(s, keep)
            else:
                s = rng.choice(live + swapped)
                model.free_seq(s)
                bm.free_seq(s)
            if step % 50 == 0:
                same_state(bm, model, sorted(model.seqs))
                same_swap_state(bm, model)
        same_state(bm, model, sorted(model.seqs))
        same_swap_state(bm, model)
