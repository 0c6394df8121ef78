"""Pins of oracle.accounting against the numbers the KV-cache chapter prints."""

import json
import os

import pytest

from oracle import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "accounting_pins.json")))


def test_worked_example_1_printed_dict():
    g = GOLD["worked_example_1"]
    got = acc.rounded(acc.paged_vs_naive(g["seq_lengths"], g["block_size"], g["max_seq_len"]))
    assert got == g["printed"]


def test_worked_example_1_hand_trace():
    g = GOLD["worked_example_1"]
    B = g["block_size"]
    blocks = [acc.blocks_for(n, B) for n in g["seq_lengths"]]
    assert blocks == g["blocks_per_request"]
    assert sum(blocks) == g["total_blocks"]
    r = acc.paged_vs_naive(g["seq_lengths"], B, g["max_seq_len"])
    assert r["paged_slots"] - r["total_actual_tokens"] == g["paged_waste_slots"]
    assert r["naive_slots"] - r["total_actual_tokens"] == g["naive_waste_slots"]


@pytest.mark.parametrize("key", ["answer_a2", "answer_a3"])
def test_answers_a2_a3(key):
    g = GOLD[key]
    B = g["block_size"]
    blocks = [acc.blocks_for(n, B) for n in g["seq_lengths"]]
    assert blocks == g["blocks_per_request"]
    assert [b * B - n for b, n in zip(blocks, g["seq_lengths"])] == g["waste_per_request"]
    r = acc.paged_vs_naive(g["seq_lengths"], B, g["max_seq_len"])
    assert r["paged_slots"] == g["paged_slots"]
    assert r["paged_slots"] - r["total_actual_tokens"] == g["paged_waste_slots"]
    assert round(r["paged_fragmentation_pct"], 2) == g["paged_fragmentation_pct"]
    if "naive_slots" in g:
        assert r["naive_slots"] == g["naive_slots"]
        assert round(r["naive_fragmentation_pct"], 2) == g["naive_fragmentation_pct"]
        assert round(r["memory_reduction_factor"], 2) == g["memory_reduction_factor"]


def test_answer_a3_table_entries_and_shareable_prefix():
    g = GOLD["answer_a3"]
    lens = g["seq_lengths"]
    assert sum(acc.blocks_for(n, 16) for n in lens) == g["table_entries_b16"]
    assert sum(acc.blocks_for(n, 64) for n in lens) == g["table_entries_b64"]
    for B, key in ((16, "shareable_b16"), (64, "shareable_b64")):
        s = acc.shareable_prefix(g["shared_prompt_tokens"], B)
        assert s["blocks"] == g[key]["blocks"]
        assert s["tokens"] == g[key]["tokens"]
        assert round(100 * s["fraction"], 1) == g[key]["pct"]


@pytest.mark.parametrize("key", ["answer_a5", "worked_example_2"])
def test_prefix_sharing(key):
    g = GOLD[key]
    r = acc.prefix_sharing_blocks(g["prompt_tokens"], g["suffix_tokens"], g["n_requests"],
                                  g["block_size"])
    assert r["prompt_blocks"] == g["prompt_blocks"]
    assert r["suffix_blocks"] == g["suffix_blocks"]
    assert r["unshared_blocks"] == g["unshared_blocks"]
    assert r["shared_blocks"] == g["shared_blocks"]
    assert round(r["reduction_factor"], 2) == g["reduction_factor"]


def test_tail_waste_is_below_one_block():
    # Taming the Tail, "Why This Crushes Tail Latency": the only waste is in the
    # last block of a sequence, fewer than B slots.
    for B in (1, 16, 32, 64):
        for n in range(1, 300):
            w = acc.blocks_for(n, B) * B - n
            assert 0 <= w <= B - 1


def test_blocks_for_brute_force():
    # ceil by counting: the smallest k with k*B >= n
    for B in (1, 2, 3, 16, 32):
        for n in range(0, 200):
            k = 0
            while k * B < n:
                k += 1
            assert acc.blocks_for(n, B) == k
