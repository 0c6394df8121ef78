"""Slot accounting: paged allocation versus a contiguous max-length reservation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Written from the KV-cache chapter (aicomputerinstitute.com, grade 12):

* "Worked Example 1: how much memory fragmentation actually costs" -- a request
  of n tokens holds ceil(n / B) blocks under paging and a full max_seq_len
  buffer under contiguous reservation; fragmentation is the unused share of
  the slots each scheme holds, in percent; the reduction factor is the ratio
  of the two slot counts.  The chapter rounds the three ratios to two decimals
  for printing; the functions here return raw floats and ``rounded`` applies
  the chapter's two-decimal rounding.
* "Worked Example 2: what a shared system prompt is actually worth" and answer
  A5 -- without sharing every request holds its own copy of the prompt blocks;
  with sharing the prompt blocks are held once.
* Answer A3 -- only blocks that are entirely prompt can be shared; the block
  that straddles the end of the prompt is private to each request.
"""

from __future__ import annotations


def blocks_for(tokens: int, block_size: int) -> int:
    """Number of fixed-size blocks that hold ``tokens`` tokens (rounded up)."""
    if tokens < 0 or block_size <= 0:
        raise ValueError("tokens must be >= 0 and block_size > 0")
    return (tokens + block_size - 1) // block_size


def paged_vs_naive(seq_lengths, block_size: int, max_seq_len: int) -> dict:
    """Accounting of Worked Example 1 (raw, unrounded ratios).

    Keys follow the names the chapter prints so that its output can be
    compared entry by entry.
    """
    lengths = [int(n) for n in seq_lengths]
    if not lengths:
        raise ValueError("need at least one request")
    tokens_used = sum(lengths)
    paged = block_size * sum(blocks_for(n, block_size) for n in lengths)
    naive = max_seq_len * len(lengths)
    return {
        "total_actual_tokens": tokens_used,
        "paged_slots": paged,
        "naive_slots": naive,
        "paged_fragmentation_pct": 100.0 * (paged - tokens_used) / paged,
        "naive_fragmentation_pct": 100.0 * (naive - tokens_used) / naive,
        "memory_reduction_factor": naive / paged,
    }


def rounded(result: dict) -> dict:
    """The chapter's presentation: the three ratios rounded to 2 decimals."""
    out = dict(result)
    for key in ("paged_fragmentation_pct", "naive_fragmentation_pct",
                "memory_reduction_factor"):
        out[key] = round(out[key], 2)
    return out


def prefix_sharing_blocks(prompt_tokens: int, suffix_tokens: int,
                          n_requests: int, block_size: int) -> dict:
    """Blocks held by ``n_requests`` requests that share one prompt.

    Worked Example 2 / answer A5: the prompt occupies ceil(P/B) blocks and each
    request's own part ceil(U/B) blocks; unshared, every request holds both;
    shared, the prompt blocks are held once.
    """
    p = blocks_for(prompt_tokens, block_size)
    u = blocks_for(suffix_tokens, block_size)
    unshared = (p + u) * n_requests
    shared = p + u * n_requests
    return {"prompt_blocks": p, "suffix_blocks": u, "unshared_blocks": unshared,
            "shared_blocks": shared, "reduction_factor": unshared / shared}


def shareable_prefix(prompt_tokens: int, block_size: int) -> dict:
    """Answer A3: whole blocks that lie entirely inside the shared prompt."""
    full = prompt_tokens // block_size
    tokens = full * block_size
    return {"blocks": full, "tokens": tokens,
            "fraction": tokens / prompt_tokens if prompt_tokens else 0.0}
