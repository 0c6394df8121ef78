"""Seeded synthetic workloads shaped like the pages' serving scenarios.

This module only draws random inputs and describes, as a script of block-manager
operations, how a workload's state is built; it computes nothing the paged path
computes.  Both sides of a parity test consume it: the library (through its block
manager and kernels) and the oracle (through the recorded value rows of each
sequence).

A workload holds:

* shapes: query/kv heads, head_dim, block size, dtype, pool size, softmax scale;
* ``free_order``: the initial order of the free pool (a seeded shuffle, so
  physical blocks are scattered: "Taming the Tail", "How the Architecture Works");
* ``script``: operations that build the pool state before the timed step
  (prefills, forks, frees and -- for the fragmented pool -- churn by "ghost"
  sequences whose admissions/appends are skipped when the pool is full);
* ``step_ids`` / ``step_tokens``: the batch of the timed step, in batch order;
  each appends ``step_tokens`` tokens (1 = decode, C = a chunk);
* ``segments``: for every sequence of the timed batch, the rows of the value
  tensors that make up its K/V in logical order (after the step).  The oracle
  builds contiguous K/V from these directly.

Value tensors (named ``k_<x>``, ``v_<x>``; ``q``) are N(0, 1) draws rounded to the
workload dtype, made with a seeded torch generator on the requested device.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

GHOST_BASE = 1 << 40   # ids of churn sequences


@dataclass
class Workload:
    name: str
    dtype: str                  # "f32" | "bf16"
    hq: int
    hkv: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    seed: int
    free_order: np.ndarray
    script: list
    step_ids: list
    step_tokens: int
    rows: dict                  # value tensor name -> number of rows
    segments: dict              # seq id -> [(tensor name, first row, count), ...]
    meta: dict = field(default_factory=dict)
    chunk: bool = False         # the step is a chunked query (q is [S, C, Hq, D])

    @property
    def num_seqs(self) -> int:
        return len(self.step_ids)

    def ctx_len(self, sid) -> int:
        return sum(c for _, _, c in self.segments[sid])

    def ctx_lens(self) -> list:
        return [self.ctx_len(s) for s in self.step_ids]

    def max_blocks(self) -> int:
        B = self.block_size
        return max((n + B - 1) // B for n in self.ctx_lens())


# -- value tensors ----------------------------------------------------------------------

_TENSOR_IDS = {"q": 1, "k_prefill": 2, "v_prefill": 3, "k_step": 4, "v_step": 5}


def torch_dtype(w: Workload):
    import torch
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def value_tensor(w: Workload, name: str, device="cpu"):
    """N(0,1) values of tensor ``name`` ([rows, Hkv, D], or q) in the workload dtype."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed * 1000 + _TENSOR_IDS[name])
    if name == "q":
        shape = (w.num_seqs, w.step_tokens, w.hq, w.head_dim) if w.chunk else \
                (w.num_seqs, w.hq, w.head_dim)
    else:
        shape = (w.rows[name[2:]], w.hkv, w.head_dim)
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(torch_dtype(w))


# -- replay of the script on any block manager -------------------------------------------

def replay(w: Workload, bm, out_of_blocks, write=None) -> None:
    """Apply ``w.script`` to ``bm``.

    ``bm`` offers add_seq(id, n) -> slots, append_slots(ids, k) -> (slots, pairs),
    fork(parent, child) and free_seq(id); ``out_of_blocks`` is the exception type it
    raises when the pool is full (churn operations that hit it are skipped).
    ``write(name, row0, slots, pairs)`` is called after every operation that stores
    values: rows [row0, row0 + len(slots)) of tensors k_<name>/v_<name> go to ``slots``
    after the block copies ``pairs`` are applied.
    """
    ghosts: list = []
    for op in w.script:
        kind = op[0]
        if kind == "add":
            _, sid, n, vals = op
            slots = bm.add_seq(sid, n)
            if write is not None and vals is not None and n:
                write(vals[0], vals[1], slots, [])
        elif kind == "append":
            _, ids, k, vals = op
            slots, pairs = bm.append_slots(ids, k)
            if write is not None and vals is not None:
                write(vals[0], vals[1], slots, pairs)
            elif len(pairs):
                raise RuntimeError("copy-on-write during a value-less append")
        elif kind == "fork":
            bm.fork(op[1], op[2])
        elif kind == "free":
            bm.free_seq(op[1])
        elif kind == "ghost_add":
            try:
                bm.add_seq(op[1], op[2])
                ghosts.append(op[1])
            except out_of_blocks:
                pass
        elif kind == "ghost_append":
            if ghosts:
                try:
                    bm.append_slots([ghosts[op[1] % len(ghosts)]], op[2])
                except out_of_blocks:
                    pass
        elif kind == "ghost_free":
            if ghosts:
                bm.free_seq(ghosts.pop(op[1] % len(ghosts)))
        elif kind == "ghost_free_all":
            order = np.random.default_rng(op[1]).permutation(len(ghosts))
            for i in order:
                bm.free_seq(ghosts[i])
            ghosts.clear()
        else:
            raise ValueError(f"unknown script op {kind!r}")


# -- workload builders ----------------------------------------------------------------------

def _blocks(n: int, B: int) -> int:
    return (n + B - 1) // B


def _decode_workload(name, seed, lens, hq, hkv, D, B, dtype, pool_factor=1.25,
                     churn_steps=0, churn_law=None, rng=None, extra_blocks=0) -> Workload:
    """Independent sequences: prefill n-1 tokens each, then the decode step writes token n."""
    rng = np.random.default_rng(seed) if rng is None else rng
    lens = [int(n) for n in lens]
    need = sum(_blocks(n, B) for n in lens) + extra_blocks
    num_blocks = int(math.ceil(pool_factor * need))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    script = []
    if churn_steps:
        # Alloc/free churn by ghost sequences: admit (p=0.4) a ghost with a length from
        # the workload's law when it fits, grow a random ghost by 1..64 tokens (p=0.4),
        # or retire one (p=0.2); finally retire every ghost in random order.
        gid = GHOST_BASE
        for _ in range(churn_steps):
            u = rng.random()
            if u < 0.4:
                script.append(("ghost_add", gid, int(churn_law(rng))))
                gid += 1
            elif u < 0.8:
                script.append(("ghost_append", int(rng.integers(1 << 31)), int(rng.integers(1, 65))))
            else:
                script.append(("ghost_free", int(rng.integers(1 << 31))))
        script.append(("ghost_free_all", int(rng.integers(1 << 31))))
    row = 0
    segments = {}
    for sid, n in enumerate(lens):
        script.append(("add", sid, n - 1, ("prefill", row)))
        segments[sid] = [("prefill", row, n - 1), ("step", sid, 1)]
        row += n - 1
    return Workload(name=name, dtype=dtype, hq=hq, hkv=hkv, head_dim=D, block_size=B,
                    num_blocks=num_blocks, scale=1.0 / math.sqrt(D), seed=seed,
                    free_order=free_order, script=script, step_ids=list(range(len(lens))),
                    step_tokens=1, rows={"prefill": row, "step": len(lens)}, segments=segments)


def tiny(seed: int = 1) -> Workload:
    """Four requests of the KV-cache chapter's Worked Example 1 (47/612/130/1,900 tokens),
    4 query = 4 kv heads, head_dim 64, fp32, B = 16, a 256-block shuffled pool."""
    rng = np.random.default_rng(seed)
    w = _decode_workload("tiny_fp32", seed, [47, 612, 130, 1900], 4, 4, 64, 16, "f32",
                         rng=rng)
    # fixed pool of 256 blocks (the worked example needs 170)
    w.num_blocks = 256
    w.free_order = rng.permutation(256).astype(np.int32)
    return w


def mistral(seed: int = 2, S: int = 64, max_len: int = 4096) -> Workload:
    """Mistral-7B-shaped decode layer: 32/8 heads, D=128, bf16, B=16, lengths U[128, max]."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(128, max_len + 1, size=S)
    return _decode_workload(f"mistral7b_b{S}", seed, lens, 32, 8, 128, 16, "bf16", rng=rng)


def llama70b(seed: int = 3, S: int = 256, churn_steps: int = 10_000, max_len: int = 8192,
             median: float = 1024.0, sigma: float = 1.0, B: int = 16) -> Workload:
    """Llama-3-70B-shaped decode layer: 64/8 heads, D=128, bf16, B=16 (other block sizes for
    the block-size trade-off), log-normal lengths (median 1,024, clipped to [16, 8,192]) over
    a pool fragmented by alloc/free churn."""
    rng = np.random.default_rng(seed)

    def law(r):
        return int(np.clip(np.rint(np.exp(r.normal(math.log(median), sigma))), 16, max_len))

    lens = [law(rng) for _ in range(S)]
    name = f"llama3_70b_b{S}" + ("" if B == 16 else f"_B{B}")
    w = _decode_workload(name, seed, lens, 64, 8, 128, B, "bf16",
                         churn_steps=churn_steps, churn_law=law, rng=rng)
    w.meta["churn_steps"] = churn_steps
    return w


def long_context(seed: int = 6, S: int = 32, n: int = 32768) -> Workload:
    """Long-context decode: S sequences of n tokens, 64/8 heads, D=128, bf16, B=32."""
    return _decode_workload(f"long_decode_b{S}_n{n}", seed, [n] * S, 64, 8, 128, 32, "bf16")


def shared_prefix(seed: int = 4, B: int = 16, n_seqs: int = 128, prefix: int = 1024,
                  n_families: int = 32, children: int = 3, suffix_range=(16, 2048),
                  hq: int = 32, hkv: int = 8) -> Workload:
    """Shared system prompt + copy-on-write forks.

    A template sequence of ``prefix`` tokens is forked into ``n_seqs`` sequences and then
    dropped (its blocks stay, shared n_seqs ways); each sequence prefills a private suffix
    of U[suffix_range] tokens; the first ``n_families`` sequences are each forked into
    ``children`` more samples (sharing every block, including a partly filled last block).
    The timed step appends one token to all of them, in order: the shared last blocks are
    copied on first write.
    """
    rng = np.random.default_rng(seed)
    T = -1
    suf = rng.integers(suffix_range[0], suffix_range[1] + 1, size=n_seqs)
    script = [("add", T, prefix, ("prefill", 0)), *[("fork", T, i) for i in range(n_seqs)],
              ("free", T)]
    row = prefix
    segs = {}
    for i in range(n_seqs):
        script.append(("append", [i], int(suf[i]), ("prefill", row)))
        segs[i] = [("prefill", 0, prefix), ("prefill", row, int(suf[i]))]
        row += int(suf[i])
    ids = list(range(n_seqs))
    nid = n_seqs
    for f in range(n_families):
        for _ in range(children):
            script.append(("fork", f, nid))
            segs[nid] = list(segs[f])
            ids.append(nid)
            nid += 1
    for j, sid in enumerate(ids):
        segs[sid] = segs[sid] + [("step", j, 1)]
    need = _blocks(prefix, B) + sum(_blocks(int(s), B) for s in suf) + len(ids) * 2
    num_blocks = int(math.ceil(1.25 * need))
    return Workload(name=f"shared_prefix_B{B}", dtype="bf16", hq=hq, hkv=hkv, head_dim=128,
                    block_size=B, num_blocks=num_blocks, scale=1 / math.sqrt(128), seed=seed,
                    free_order=rng.permutation(num_blocks).astype(np.int32), script=script,
                    step_ids=ids, step_tokens=1, rows={"prefill": row, "step": len(ids)},
                    segments=segs)


def chunked(seed: int = 5, S: int = 8, cached: int = 4096, C: int = 512, B: int = 32,
            hq: int = 64, hkv: int = 8, D: int = 128) -> Workload:
    """Chunked query: S sequences with ``cached`` tokens in the pool each receive C new
    tokens (written, then attended causally over the whole context)."""
    rng = np.random.default_rng(seed)
    need = S * _blocks(cached + C, B)
    num_blocks = int(math.ceil(1.25 * need))
    script = []
    segs = {}
    for s in range(S):
        script.append(("add", s, cached, ("prefill", s * cached)))
        segs[s] = [("prefill", s * cached, cached), ("step", s * C, C)]
    return Workload(name=f"chunk_b{S}_c{C}_ctx{cached}", dtype="bf16", hq=hq, hkv=hkv,
                    head_dim=D, block_size=B, num_blocks=num_blocks, scale=1 / math.sqrt(D),
                    seed=seed, free_order=rng.permutation(num_blocks).astype(np.int32),
                    script=script, step_ids=list(range(S)), step_tokens=C,
                    rows={"prefill": S * cached, "step": S * C}, segments=segs, chunk=True)


def logical_kv(w: Workload, sid, tensors: dict):
    """Contiguous K and V of sequence ``sid`` (after the step) from its value rows.

    ``tensors`` maps "k_prefill", "v_prefill", "k_step", "v_step" to array-likes
    supporting row slicing.  Returns (K, V) as lists of row blocks, to be concatenated by
    the caller in its own array library.
    """
    ks, vs = [], []
    for name, r0, cnt in w.segments[sid]:
        ks.append(tensors["k_" + name][r0:r0 + cnt])
        vs.append(tensors["v_" + name][r0:r0 + cnt])
    return ks, vs


def custom_decode(name: str, seed: int, lens, hq: int, hkv: int, D: int, B: int, dtype: str,
                  churn_steps: int = 0, extra_blocks: int = 0) -> Workload:
    """Independent sequences of the given lengths (a decode step over a shuffled pool);
    ``extra_blocks`` enlarges the pool for appends beyond the workload's own step."""
    rng = np.random.default_rng(seed)
    law = None
    if churn_steps:
        lo, hi = int(min(lens)), int(max(lens))

        def law(r):
            return int(r.integers(lo, hi + 1))
    return _decode_workload(name, seed, lens, hq, hkv, D, B, dtype, churn_steps=churn_steps,
                            churn_law=law, rng=rng, extra_blocks=extra_blocks)
