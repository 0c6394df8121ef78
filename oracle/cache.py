"""Paged KV cache: slot scatter, copy-on-write block copy, table reconstruction.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Layout of the physical pool (a choice of this library's interface; the pages
fix only that a token's address is its physical block times the block size
plus its offset, Taming the Tail, "The Kernel Engineering" snippet):

* K pool ``k_cache[num_blocks, Hkv, B, D]``: in block p, kv-head h, the key of
  the token at offset o is the row ``k_cache[p, h, o, :]``;
* V pool ``v_cache[num_blocks, Hkv, D, B]``: the value of that token is the
  column ``v_cache[p, h, :, o]`` (values are stored transposed inside a block).

A slot is ``p * B + o``.  Negative slots mark tokens that are not written.

The functions work on arrays of any dtype and copy bits only (no arithmetic),
so bf16 pools can be handled as uint16 arrays.
"""

from __future__ import annotations

import numpy as np


def write_kv(k_cache: np.ndarray, v_cache: np.ndarray, key: np.ndarray,
             value: np.ndarray, slots, block_size: int) -> None:
    """Store token t's key/value (``key[t]``, ``value[t]`` of shape [Hkv, D]) at slots[t].

    Writes only what the slot names; every other byte of the pools is left
    unchanged.  Taming the Tail, "The Hidden Tax": each step stores only the
    new token's K/V; tinycto "1. Underlying Mechanism": a step writes the new
    token's entries and nothing else.
    """
    B = block_size
    for t, slot in enumerate(slots):
        slot = int(slot)
        if slot < 0:
            continue
        p, o = divmod(slot, B)
        k_cache[p, :, o, :] = key[t]
        v_cache[p, :, :, o] = value[t]


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs) -> None:
    """Copy-on-write: physical block ``dst`` becomes a copy of block ``src``.

    KV-cache chapter, "PagedAttention: borrowing virtual memory": the writer
    gets a private copy of the shared block before it writes.  The whole block
    (every kv-head, every slot) is copied, in K and V.
    """
    for src, dst in pairs:
        k_cache[int(dst)] = k_cache[int(src)]
        v_cache[int(dst)] = v_cache[int(src)]


def gather_sequence(k_cache: np.ndarray, v_cache: np.ndarray, table_row,
                    n_tokens: int, block_size: int):
    """Contiguous K and V ([n, Hkv, D] each) of one sequence, via its block table.

    Token j lives in logical block j // B at offset j % B; the table maps the
    logical block to the physical one (Taming the Tail, "How the Architecture
    Works" and the kernel snippet).  Only positions j < n are read: table
    entries past the last used block and the unused tail of the last block are
    never touched ("The Kernel Engineering", item 3: the unaligned last block).
    """
    B = block_size
    j = np.arange(n_tokens)
    row = np.asarray(table_row)
    phys = row[j // B]
    if n_tokens and (phys.min() < 0 or phys.max() >= k_cache.shape[0]):
        raise ValueError("block table names a block outside the pool")
    off = j % B
    K = k_cache[phys, :, off, :]           # [n, Hkv, D]
    V = v_cache[phys, :, :, off]           # [n, Hkv, D]
    return K, V


def swap_out(k_cache: np.ndarray, v_cache: np.ndarray, blocks) -> np.ndarray:
    """Contents of whole physical blocks, as moved to host memory when a request is paused.

    Taming the Tail, "Infrastructure Scale": when the pool runs out of blocks a
    request can be paused and its KV-cache moved to CPU RAM.  The host buffer
    layout is this library's interface: for block i of ``blocks``, its K part
    ``k_cache[blocks[i]]`` ([Hkv, B, D]) flattened, then its V part
    ``v_cache[blocks[i]]`` ([Hkv, D, B]) flattened.  Returns [n, 2, Hkv*B*D].
    """
    blocks = [int(b) for b in blocks]
    out = np.empty((len(blocks), 2, k_cache[0].size), dtype=k_cache.dtype)
    for i, b in enumerate(blocks):
        out[i, 0] = k_cache[b].reshape(-1)
        out[i, 1] = v_cache[b].reshape(-1)
    return out


def swap_in(k_cache: np.ndarray, v_cache: np.ndarray, host: np.ndarray, blocks) -> None:
    """Put saved block contents (the layout ``swap_out`` returns) into physical blocks."""
    for i, b in enumerate(int(x) for x in blocks):
        k_cache[b] = host[i, 0].reshape(k_cache.shape[1:])
        v_cache[b] = host[i, 1].reshape(v_cache.shape[1:])
