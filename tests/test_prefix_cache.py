"""The automatic prefix cache of the host block manager: libpa against the oracle's integer
model (bit-exact) and against the chapter's printed numbers.

KV-cache chapter, "RadixAttention": cached token sequences form a radix tree; a request reuses
the blocks of its longest cached prefix and prefills only the rest; least recently used leaves
are evicted when memory runs low, reference counting protecting what running requests use.
Answer A3: only whole blocks that are entirely prefix can be shared."""

import json
import os
import random

import pytest

from oracle.block_manager import BlockManagerModel
from oracle.block_manager import OutOfBlocks as ModelOOB

from test_block_manager import same_state

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "accounting_pins.json")))


def same_cache_state(bm, model):
    st, ms = bm.stats(), model.stats()
    for k in ("cached_blocks", "cache_hit_blocks", "cache_evictions", "used_blocks",
              "free_blocks"):
        assert st[k] == ms[k], k


def serve(m, n_req, prompt, suffix, B):
    """Each request: a cached add of prompt + its own suffix, then its blocks go in the cache
    (its K/V are written by then); returns the cached-token count of every request."""
    hits = []
    for r in range(n_req):
        toks = prompt + [10 ** 6 + 1000 * r + i for i in range(suffix)]
        _, n_cached = m.add_seq_cached(r, toks)
        m.cache_insert(r, toks)
        hits.append(n_cached)
    return hits


@pytest.mark.parametrize("lib", [True, False])
def test_worked_example_2_and_answer_a3(libpa, lib):
    """A 380-token prompt and 90-token questions, B = 16: answer A3's 23 shareable blocks (368
    tokens) are reused by every request after the first; 30 blocks for the first request and
    ceil((470 - 368) / 16) = 7 for each other one: 30 + 499 * 7 = 3,523 blocks.  (Worked
    Example 2 prints 3,024 under its claim that the prompt ends on a block boundary, which 380
    does not.)"""
    g, a3 = GOLD["worked_example_2"], GOLD["answer_a3"]
    B, n = g["block_size"], g["n_requests"]
    m = libpa.BlockManager(4000, B) if lib else BlockManagerModel(4000, B)
    prompt = list(range(100, 100 + g["prompt_tokens"]))
    hits = serve(m, n, prompt, g["suffix_tokens"], B)
    assert hits[0] == 0 and set(hits[1:]) == {a3["shareable_b16"]["tokens"]}
    assert m.stats()["used_blocks"] == 30 + (n - 1) * 7 == 3523


@pytest.mark.parametrize("lib", [True, False])
def test_answer_a3_block_size_64(libpa, lib):
    a3 = GOLD["answer_a3"]
    m = libpa.BlockManager(64, 64) if lib else BlockManagerModel(64, 64)
    hits = serve(m, 3, list(range(a3["shared_prompt_tokens"])), 90, 64)
    assert hits == [0, a3["shareable_b64"]["tokens"], a3["shareable_b64"]["tokens"]]


@pytest.mark.parametrize("lib", [True, False])
def test_answer_a5(libpa, lib):
    """A block-aligned 512-token prompt, 60-token suffixes, 1,000 requests: 4,032 blocks."""
    g = GOLD["answer_a5"]
    m = libpa.BlockManager(5000, g["block_size"]) if lib else BlockManagerModel(5000, g["block_size"])
    hits = serve(m, g["n_requests"], list(range(g["prompt_tokens"])), g["suffix_tokens"],
                 g["block_size"])
    assert set(hits[1:]) == {g["prompt_tokens"]}
    assert m.stats()["used_blocks"] == g["shared_blocks"]


def test_lru_eviction_and_protection(libpa):
    """A hand-traced script: pool of 6 blocks, B = 2, free order 0..5."""
    bm = libpa.BlockManager(6, 2)
    model = BlockManagerModel(6, 2)
    for m in (bm, model):
        m.add_seq(1, 4)                    # blocks 0, 1
        m.cache_insert(1, [7, 7, 8, 8])    # nodes (7,7)->0 and (8,8)->1; tick 0
        m.add_seq(2, 4)                    # blocks 2, 3
        m.cache_insert(2, [5, 5, 6, 6])    # nodes (5,5)->2 and (6,6)->3; tick 1
        m.free_seq(1)                      # blocks 0, 1 live only in the cache
        m.free_seq(2)                      # blocks 2, 3 too
    assert bm.stats()["free_blocks"] == 2 and bm.stats()["cached_blocks"] == 4
    # a cached add reuses (7,7) (block 0, now also held by sequence 3; use refreshed to tick 2)
    # and takes block 4 for its third token
    slots, n_cached = bm.add_seq_cached(3, [7, 7, 9])
    assert list(slots) == [0, 1, 8] and n_cached == 2
    assert model.add_seq_cached(3, [7, 7, 9]) == ([0, 1, 8], 2)
    # 3 blocks with only block 5 free: the shortfall of 2 is evicted first, each time the
    # oldest leaf only the tree holds: (8,8) of tick 0, then (6,6) of tick 1.  (7,7) is held
    # by sequence 3; (5,5) is no leaf while (6,6) is there.  Freed blocks join the back.
    for m in (bm, model):
        m.add_seq(4, 6)
    assert bm.stats()["cache_evictions"] == 2
    assert list(bm.free_list()) == list(model.free)
    t, _ = bm.block_tables([4], 3)
    assert t.tolist() == [[5, 1, 3]]
    # what is left to evict: (5,5), a leaf only the tree holds; (7,7) stays protected
    with pytest.raises(libpa.OutOfBlocks):
        bm.add_seq(5, 4)                   # needs 2, can free 1: nothing changes
    with pytest.raises(ModelOOB):
        model.add_seq(5, 4)
    assert bm.stats()["cached_blocks"] == 2 and bm.stats()["cache_evictions"] == 2
    assert bm.cache_evict(10) == 1 == model.cache_evict(10)
    same_state(bm, model, sorted(model.seqs))
    same_cache_state(bm, model)


def test_swap_in_evicts_cached_leaves(libpa):
    """Swap-in allocates like an add: a short pool is first topped up from the cache's least
    recently used leaves.  Hand-traced: pool of 6 blocks, B = 2, free order 0..5."""
    bm = libpa.BlockManager(6, 2)
    model = BlockManagerModel(6, 2)
    for m in (bm, model):
        m.add_seq(1, 4)                    # blocks 0, 1
        m.cache_insert(1, [7, 7, 8, 8])    # nodes (7,7)->0 and (8,8)->1
        m.free_seq(1)                      # free: 2 3 4 5
        m.add_seq(2, 6)                    # blocks 2, 3, 4; free: 5
    assert list(bm.swap_out(2)) == [2, 3, 4] == model.swap_out(2)   # free: 5 2 3 4
    for m in (bm, model):
        m.add_seq(3, 6)                    # blocks 5, 2, 3; free: 4
    with pytest.raises(libpa.OutOfBlocks):
        bm.add_seq(4, 8)                   # needs 4, can reach 3: nothing changes
    with pytest.raises(ModelOOB):
        model.add_seq(4, 8)
    assert bm.stats()["cached_blocks"] == 2
    # 3 blocks, 1 free: (8,8) goes first (a leaf), then (7,7), a leaf once (8,8) is gone
    assert list(bm.swap_in(2)) == [4, 1, 0] == model.swap_in(2)
    assert bm.stats()["cache_evictions"] == 2 and bm.stats()["cached_blocks"] == 0
    same_state(bm, model, sorted(model.seqs))
    same_cache_state(bm, model)


def test_random_ops_with_prefix_cache_bit_exact(libpa):
    rng = random.Random(777)
    for B in (2, 4, 16):
        NB = 70
        order = rng.sample(range(NB), NB)
        bm = libpa.BlockManager(NB, B, order)
        model = BlockManagerModel(NB, B, order)
        prompts = [[rng.randrange(50) for _ in range(rng.randint(0, 5 * B))] for _ in range(4)]
        tokens = {}
        next_id = 0
        for step in range(700):
            live = sorted(model.seqs)
            op = rng.random()
            if op < 0.3 or not live:
                toks = rng.choice(prompts) + [rng.randrange(50) for _ in range(rng.randint(0, 3 * B))]
                try:
                    want = model.add_seq_cached(next_id, toks)
                except ModelOOB:
                    with pytest.raises(libpa.OutOfBlocks):
                        bm.add_seq_cached(next_id, toks)
                else:
                    slots, nc = bm.add_seq_cached(next_id, toks)
                    assert (list(slots), nc) == want
                    tokens[next_id] = toks
                next_id += 1
            elif op < 0.5:
                s = rng.choice(live)
                if s in tokens:
                    k = rng.randint(0, min(len(tokens[s]), model.seqs[s].n))
                    assert bm.cache_insert(s, tokens[s][:k]) == model.cache_insert(s, tokens[s][:k])
            elif op < 0.7:
                ids = rng.sample(live, rng.randint(1, len(live)))
                k = rng.randint(1, B + 1)
                try:
                    want_slots, want_pairs = model.append_slots(ids, k)
                except ModelOOB:
                    with pytest.raises(libpa.OutOfBlocks):
                        bm.append_slots(ids, k)
                else:
                    slots, pairs = bm.append_slots(ids, k)
                    assert list(slots) == want_slots
                    assert [tuple(p) for p in pairs] == want_pairs
                    for s in ids:
                        tokens.pop(s, None)   # its new tokens are unknown to the cache
            elif op < 0.78:
                p = rng.choice(live)
                model.fork(p, next_id)
                bm.fork(p, next_id)
                next_id += 1
            elif op < 0.84:
                s = rng.choice(live)
                keep = rng.randint(0, model.seqs[s].n)
                model.truncate(s, keep)
                bm.truncate(s, keep)
                if s in tokens:
                    tokens[s] = tokens[s][:keep]
            elif op < 0.88:
                n = rng.randint(0, 4)
                assert bm.cache_evict(n) == model.cache_evict(n)
            elif op < 0.91:
                s = rng.choice(live)
                assert list(bm.swap_out(s)) == model.swap_out(s)
            elif op < 0.94 and model.swapped:
                s = rng.choice(sorted(model.swapped))
                try:
                    want = model.swap_in(s)
                except ModelOOB:
                    with pytest.raises(libpa.OutOfBlocks):
                        bm.swap_in(s)
                else:
                    assert list(bm.swap_in(s)) == want   # private copies: may evict cached leaves
            else:
                s = rng.choice(live + sorted(model.swapped))
                model.free_seq(s)
                bm.free_seq(s)
                tokens.pop(s, None)
            if step % 50 == 0:
                same_state(bm, model, sorted(model.seqs))
                same_cache_state(bm, model)
        same_state(bm, model, sorted(model.seqs))
        same_cache_state(bm, model)
