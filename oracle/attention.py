"""Paged attention as its plain definition: dense softmax attention in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages state that paging changes where K and V live, not what attention
computes: the result equals standard multi-head attention exactly (vLLM
PagedAttention (tinycto), FAQ and "Common Misconceptions"), with the same
scores, softmax and floating-point operation count as contiguous attention
(KV-cache chapter, "Common misconception").  The oracle is therefore: rebuild each sequence's contiguous
K/V from its block table (``cache.gather_sequence``), then run textbook
attention on it.

Readings where the pages are silent (each also listed in the design notes):

* a decode query attends to every cached position of its sequence including
  the token written in the same step (the context length counts it);
* grouped-query attention maps query head h to kv-head h // (Hq / Hkv);
* scores are ``scale * q.k`` with a caller-given scale (1/sqrt(D) in every
  workload); softmax uses the natural exponential;
* a chunk of C new queries of a sequence with n tokens in total: query i sits
  at position n - C + i and sees positions 0 .. n - C + i (causal inside the
  chunk, every earlier token visible).

All arithmetic is float64; inputs are upcast exactly (bf16 and fp32 values are
representable in float64).
"""

from __future__ import annotations

import numpy as np

from .cache import gather_sequence


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 numbers given as their uint16 bit patterns."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def softmax_weights(q_row, K_head, scale: float):
    """Unnormalised weights w_j = exp(x_j - max x) and their sum, x_j = scale q.k_j."""
    x = scale * (_f64(K_head) @ _f64(q_row))
    w = np.exp(x - x.max())
    return w, w.sum()


def dense_decode(q, K, V, scale: float) -> np.ndarray:
    """One query token per head over contiguous K/V.

    q: [Hq, D]; K, V: [n, Hkv, D] (n >= 1).  Returns out [Hq, D] in float64.
    """
    q, K, V = _f64(q), _f64(K), _f64(V)
    Hq = q.shape[0]
    Hkv = K.shape[1]
    if K.shape[0] < 1:
        raise ValueError("attention over an empty context is undefined")
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    g = Hq // Hkv
    out = np.empty_like(q)
    for h in range(Hq):
        kv = h // g
        w, l = softmax_weights(q[h], K[:, kv, :], scale)
        out[h] = (w @ V[:, kv, :]) / l
    return out


def paged_decode(q, k_cache, v_cache, block_tables, ctx_lens, block_size: int,
                 scale: float) -> np.ndarray:
    """Decode attention for a batch through block tables.

    q: [S, Hq, D]; pools as in ``cache``; block_tables: [S, max_blocks];
    ctx_lens: [S] (including the token written this step).  Returns [S, Hq, D].
    """
    q = _f64(q)
    out = np.empty_like(q)
    for s in range(q.shape[0]):
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], int(ctx_lens[s]),
                               block_size)
        out[s] = dense_decode(q[s], K, V, scale)
    return out


def chunk_attend(q, K, V, scale: float) -> np.ndarray:
    """Chunked query over contiguous K/V of one sequence.

    q: [C, Hq, D] are the queries of the last C positions of a sequence whose
    K/V ([n, Hkv, D]) already include the chunk.  Row i sees K/V[0 .. n-C+i].
    Returns [C, Hq, D].
    """
    q = _f64(q)
    C = q.shape[0]
    n = K.shape[0]
    if C > n:
        raise ValueError("chunk longer than the context")
    out = np.empty_like(q)
    for i in range(C):
        visible = n - C + i + 1
        out[i] = dense_decode(q[i], K[:visible], V[:visible], scale)
    return out


def paged_chunk_attend(q, k_cache, v_cache, block_tables, ctx_lens, block_size: int,
                       scale: float) -> np.ndarray:
    """``chunk_attend`` for a batch through block tables; q: [S, C, Hq, D]."""
    q = _f64(q)
    out = np.empty_like(q)
    for s in range(q.shape[0]):
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], int(ctx_lens[s]),
                               block_size)
        out[s] = chunk_attend(q[s], K, V, scale)
    return out


# -- split-K partitions and their merge ---------------------------------------
#
# The KV-cache chapter ("Common misconception") notes that serving kernels run
# FlashAttention-style tiled compute on the paged layout.  Tiling the context
# into partitions gives, per partition p, its own max m_p, weight sum l_p and
# normalised output o_p; the exact result is recovered by rescaling each
# partition to the common max.  These two functions state that identity so the
# tests can pin it (merge of any split == unsplit attention).

def partition_state(q_row, K_head, V_head, scale: float):
    """(m, l, o) of one partition: max score, sum of exp(x - m), normalised output."""
    x = scale * (_f64(K_head) @ _f64(q_row))
    m = x.max()
    w = np.exp(x - m)
    l = w.sum()
    return m, l, (w @ _f64(V_head)) / l


def merge_partitions(ms, ls, os) -> np.ndarray:
    """Combine partition states: weights l_p e^(m_p - m) with m = max_p m_p."""
    ms, ls, os = _f64(ms), _f64(ls), _f64(os)
    m = ms.max()
    a = ls * np.exp(ms - m)
    return (a[:, None] * os).sum(axis=0) / a.sum()
