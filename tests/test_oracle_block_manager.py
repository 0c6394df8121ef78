"""Pins of the block-manager model (oracle.block_manager)."""

import random

import pytest

from oracle.block_manager import (BlockManagerModel, InvalidArg, OutOfBlocks, SeqExists,
                                  UnknownSeq)


def check_invariants(bm: BlockManagerModel):
    # every block is either free (count 0) or referenced by exactly `count` table entries
    counts = [0] * bm.num_blocks
    for seq in bm.seqs.values():
        assert len(seq.blocks) == (seq.n + bm.block_size - 1) // bm.block_size
        for b in seq.blocks:
            counts[b] += 1
    assert counts == bm.ref
    assert sorted(bm.free) == [b for b in range(bm.num_blocks) if bm.ref[b] == 0]
    assert len(set(bm.free)) == len(bm.free)


def test_token_17_allocates_one_block():
    # tinycto "1. Underlying Mechanism": with B=16, token 17 takes a new block.
    bm = BlockManagerModel(8, 16)
    bm.add_seq(1, 1)
    assert len(bm.free) == 7
    for _ in range(15):                       # tokens 2..16: no allocation
        bm.append_slots([1], 1)
        assert len(bm.free) == 7
    bm.append_slots([1], 1)                   # token 17
    assert len(bm.free) == 6
    assert len(bm.seqs[1].blocks) == 2


def test_worked_example_1_block_counts():
    # KV-cache chapter, Worked Example 1: ceil(n/16) = 3/39/9/119 blocks, 170 total.
    bm = BlockManagerModel(256, 16)
    for i, n in enumerate([47, 612, 130, 1900]):
        bm.add_seq(i, n - 1)
        bm.append_slots([i], 1)
    rows, lens = bm.block_tables([0, 1, 2, 3], 128)
    assert [sum(1 for b in r if b >= 0) for r in rows] == [3, 39, 9, 119]
    assert 256 - len(bm.free) == 170
    assert lens == [47, 612, 130, 1900]
    assert bm.stats()["tail_waste_slots"] == 31
    check_invariants(bm)


def test_answer_a6_refcount_teardown():
    # KV-cache chapter, answer A6: A and B share P0 (count 2); tearing A down
    # leaves count 1 and the block live; it is freed only after B goes too.
    bm = BlockManagerModel(4, 16)
    bm.add_seq("A", 10)
    p0 = bm.seqs["A"].blocks[0]
    bm.fork("A", "B")
    assert bm.refcount(p0) == 2
    free_before = len(bm.free)
    bm.free_seq("A")
    assert bm.refcount(p0) == 1
    assert len(bm.free) == free_before and p0 not in bm.free
    bm.free_seq("B")
    assert bm.refcount(p0) == 0 and p0 in bm.free


def test_hand_trace_fifo_fork_cow():
    # Hand-worked trace of the fixed policy: FIFO pool, batch-order CoW.
    bm = BlockManagerModel(5, 2, free_order=[2, 0, 3, 1, 4])
    assert bm.add_seq(10, 3) == [4, 5, 0]          # blocks [2, 0]
    assert bm.add_seq(11, 1) == [6]                # block 3
    bm.fork(10, 12)                                # 12 shares [2, 0]
    assert bm.refcount(2) == 2 and bm.refcount(0) == 2
    slots, pairs = bm.append_slots([10, 12], 1)
    # seq 10 writes position 3 into shared block 0 -> copy to block 1;
    # seq 12 then finds block 0 private (count 1) and writes in place.
    assert pairs == [(0, 1)]
    assert slots == [1 * 2 + 1, 0 * 2 + 1]
    assert bm.seqs[10].blocks == [2, 1] and bm.seqs[12].blocks == [2, 0]
    assert bm.refcount(0) == 1 and bm.refcount(1) == 1 and bm.refcount(2) == 2
    bm.free_seq(10)                                # 2: 2->1, 1: 1->0 (freed)
    assert list(bm.free) == [4, 1]
    slots, pairs = bm.append_slots([12, 11], 1)    # 12: pos 4 -> new block 4; 11: pos 1 in place
    assert slots == [4 * 2 + 0, 3 * 2 + 1] and pairs == []
    assert list(bm.free) == [1]
    check_invariants(bm)


def test_cow_families_copy_k_minus_1():
    # four sharers of a partial last block writing in one step: 3 copies.
    bm = BlockManagerModel(64, 16)
    bm.add_seq(0, 20)
    for c in (1, 2, 3):
        bm.fork(0, c)
    last = bm.seqs[0].blocks[-1]
    assert bm.refcount(last) == 4
    slots, pairs = bm.append_slots([0, 1, 2, 3], 1)
    assert len(pairs) == 3 and all(src == last for src, _ in pairs)
    assert bm.seqs[3].blocks[-1] == last and bm.refcount(last) == 1
    assert len(set(slots)) == 4
    check_invariants(bm)


def test_full_last_block_needs_no_copy():
    bm = BlockManagerModel(64, 16)
    bm.add_seq(0, 32)
    bm.fork(0, 1)
    _, pairs = bm.append_slots([0, 1], 1)
    assert pairs == []
    assert bm.seqs[0].blocks[:2] == bm.seqs[1].blocks[:2]
    assert bm.seqs[0].blocks[2] != bm.seqs[1].blocks[2]
    check_invariants(bm)


def test_shared_prompt_live_allocator_pins():
    # Derived pins of this policy for Worked Example 2's workload (380-token
    # prompt, 500 requests x 90 tokens, B=16): with copy-on-write the block
    # straddling the prompt's end is private per request (answer A3).
    for keep_template, expect in ((True, 24 + 7 * 500), (False, 23 + 7 * 500)):
        bm = BlockManagerModel(4096, 16)
        bm.add_seq("T", 380)
        for r in range(500):
            bm.fork("T", r)
        if not keep_template:
            bm.free_seq("T")
        for r in range(500):
            bm.append_slots([r], 90)
        assert 4096 - len(bm.free) == expect
        check_invariants(bm)


def test_errors_leave_state_unchanged():
    bm = BlockManagerModel(4, 16)
    bm.add_seq(0, 40)                               # 3 blocks
    snap = (list(bm.free), list(bm.ref), {k: (list(v.blocks), v.n) for k, v in bm.seqs.items()})

    def same():
        return snap == (list(bm.free), list(bm.ref),
                        {k: (list(v.blocks), v.n) for k, v in bm.seqs.items()})

    with pytest.raises(OutOfBlocks):
        bm.add_seq(1, 17)                           # needs 2, 1 free
    assert same()
    with pytest.raises(OutOfBlocks):
        bm.append_slots([0], 40)                    # needs 3 more
    assert same()
    with pytest.raises(UnknownSeq):
        bm.append_slots([0, 9], 1)
    assert same()
    with pytest.raises(InvalidArg):
        bm.append_slots([0, 0], 1)
    assert same()
    with pytest.raises(SeqExists):
        bm.add_seq(0, 1)
    with pytest.raises(SeqExists):
        bm.fork(0, 0)
    with pytest.raises(UnknownSeq):
        bm.free_seq(5)
    with pytest.raises(InvalidArg):
        bm.block_tables([0], 2)
    assert same()


def test_random_ops_keep_invariants():
    rng = random.Random(7)
    for B in (1, 4, 16):
        bm = BlockManagerModel(96, B, free_order=rng.sample(range(96), 96))
        next_id = 0
        for _ in range(600):
            live = sorted(bm.seqs)
            op = rng.random()
            try:
                if op < 0.25 or not live:
                    bm.add_seq(next_id, rng.randrange(0, 3 * B + 2))
                    next_id += 1
                elif op < 0.45:
                    bm.fork(rng.choice(live), next_id)
                    next_id += 1
                elif op < 0.85:
                    ids = rng.sample(live, rng.randint(1, len(live)))
                    before = {s: list(bm.seqs[s].blocks) for s in ids}
                    slots, pairs = bm.append_slots(ids, rng.randint(0, 2 * B))
                    assert len(slots) == len(set(slots))
                    # every block written this step is private afterwards
                    for slot in slots:
                        assert bm.ref[slot // B] == 1
                    for src, dst in pairs:
                        assert bm.ref[dst] == 1 and bm.ref[src] >= 1
                    assert len(pairs) <= len(ids)
                    del before
                else:
                    bm.free_seq(rng.choice(live))
            except OutOfBlocks:
                pass
            check_invariants(bm)
