"""Integer model of the paged block manager.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix:

* Taming the Tail, "How the Architecture Works": each sequence has a block
  table mapping its logical blocks (contiguous from the model's point of view)
  to physical blocks anywhere in the pool; when the current block is full a
  new one is taken from the free block pool.
* vLLM PagedAttention (tinycto), "1. Underlying Mechanism": blocks of B=16
  tokens; the token that no longer fits (token 17) takes a new block on the
  fly; a forked child shares the parent's blocks (zero copy) and copy-on-write
  gives it private copies only where it writes.
* KV-cache chapter, "PagedAttention: borrowing virtual memory": a reference
  count per physical block; a block goes back to the free pool only when its
  count reaches zero; a sequence about to write into a shared block first gets
  a private copy of it (copy-on-write).  Answer A6: tearing down one of two
  tables that share a block leaves the block live with count 1.
* Taming the Tail, "The Kernel Engineering" snippet: a token's physical address
  is the physical block times the block size plus its offset in the block.

Where the pages leave the policy open, this model fixes it (the same policy is
the specification of the C++ block manager, which must match it bit for bit):

* the free pool is a FIFO queue: blocks are taken from the front and freed
  blocks are appended at the back, a freed sequence's blocks in logical order;
* in a batched append the sequences are served in batch order; a sequence
  copies its last block iff that block's count is above one at its turn (so
  of k sharers writing in one step, the first k-1 copy and the last writes in
  place); a copy duplicates the whole block;
* a batch may name a sequence only once;
* every call is all-or-nothing: on any error nothing changes.

Preemption (Taming the Tail, "Infrastructure Scale": when the pool runs out of
physical blocks, a request can be paused and its KV-cache moved to CPU RAM) and
truncation, read plainly:

* swapping a sequence out hands back its physical blocks in logical order (their
  contents are what goes to host memory), then drops its references as freeing
  it would; the sequence keeps its id and length and holds no blocks;
* swapping it back in takes ceil(n / B) fresh blocks from the front of the pool,
  each with count 1 (blocks shared before the swap come back as private copies
  of the same contents);
* truncating to n_keep tokens drops the references of the blocks past
  ceil(n_keep / B), in logical order; a shared kept block stays shared until
  the next write copies it.

Prefix cache (KV-cache chapter, "RadixAttention": cached token sequences form a
radix tree; a new request reuses the blocks of its longest cached prefix and
prefills only the rest; when memory runs low the least recently used leaves are
evicted, and reference counting protects branches running requests still use;
answer A3: only whole blocks that are entirely prefix can be shared), read at
block granularity:

* a tree node is one full block of B tokens, keyed by those token ids under its
  parent; the tree holds one reference to each node's block;
* inserting a live sequence's first k full blocks walks the tree by content,
  keeps the node that already exists for a content, else adds one holding the
  sequence's block;
* a cached add matches the longest chain of full blocks from the root, takes a
  reference to each matched block (before anything is evicted, so they are
  safe), and allocates the rest like a plain add;
* every call that allocates first evicts, if the free pool is short, exactly the
  shortfall: each time the leaf with the oldest use (ties: oldest node) among
  those only the tree references; its block rejoins the pool; if the tree
  cannot cover the shortfall the call fails and nothing changes;
* an insert or a cached add marks every node it passes as used at one tick.
"""

from __future__ import annotations

import copy
from collections import deque


class BlockManagerError(Exception):
    status = -1


class InvalidArg(BlockManagerError):
    status = -1


class OutOfBlocks(BlockManagerError):
    status = -2


class UnknownSeq(BlockManagerError):
    status = -3


class SeqExists(BlockManagerError):
    status = -4


class Swapped(BlockManagerError):
    status = -8


class _Node:
    __slots__ = ("block", "key", "parent", "children", "last_use", "nid")

    def __init__(self, block, key, parent, last_use, nid):
        self.block = block
        self.key = key
        self.parent = parent          # parent _Node or None (child of the root)
        self.children: dict = {}      # token tuple -> _Node
        self.last_use = last_use
        self.nid = nid


class _Seq:
    __slots__ = ("blocks", "n")

    def __init__(self):
        self.blocks: list[int] = []
        self.n = 0


class BlockManagerModel:
    """Free pool + per-block reference counts + per-sequence block tables."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise InvalidArg("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArg("free_order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.seqs: dict[int, _Seq] = {}
        self.swapped: dict[int, int] = {}  # swapped-out sequence -> its length
        self.forks = 0
        self.cow_copies = 0
        self.swap_outs = 0
        self.swap_ins = 0
        self.root: dict = {}          # token tuple -> _Node
        self.nodes: list = []         # live tree nodes
        self.tick = 0
        self.next_nid = 0
        self.cache_hit_blocks = 0
        self.cache_evictions = 0

    # -- prefix-cache helpers ---------------------------------------------
    def _evictable(self) -> int:
        """Nodes whose whole subtree is referenced by the tree only."""
        def count(children) -> tuple:
            total, all_free = 0, True
            for node in children.values():
                sub, sub_free = count(node.children)
                total += sub
                if sub_free and self.ref[node.block] == 1:
                    total += 1
                else:
                    all_free = False
            return total, all_free
        return count(self.root)[0]

    def _evict_one(self) -> bool:
        best = None
        for node in self.nodes:
            if not node.children and self.ref[node.block] == 1:
                if best is None or (node.last_use, node.nid) < (best.last_use, best.nid):
                    best = node
        if best is None:
            return False
        (best.parent.children if best.parent else self.root).pop(best.key)
        self.nodes.remove(best)
        self._release(best.block)
        self.cache_evictions += 1
        return True

    def _make_room(self, need: int) -> None:
        short = need - len(self.free)
        if short <= 0:
            return
        if self._evictable() < short:
            raise OutOfBlocks("free pool and evictable cache too small")
        for _ in range(short):
            self._evict_one()

    def _append_need(self, ids, tokens_each: int) -> int:
        B, need, dec = self.block_size, 0, {}
        for s in ids:
            seq = self.seqs[s]
            if tokens_each == 0:
                continue
            if seq.n % B:
                last = seq.blocks[-1]
                if self.ref[last] - dec.get(last, 0) > 1:
                    dec[last] = dec.get(last, 0) + 1
                    need += 1
            first = -(-seq.n // B)
            lastm = (seq.n + tokens_each - 1) // B
            need += lastm - first + 1
        return need

    # -- internal helpers -------------------------------------------------
    def _take(self) -> int:
        if not self.free:
            raise OutOfBlocks("free pool is empty")
        b = self.free.popleft()
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        assert self.ref[b] >= 0
        if self.ref[b] == 0:
            self.free.append(b)

    def _write_one(self, seq: _Seq, pairs: list) -> int:
        """Give the next position of ``seq`` a slot; returns the slot."""
        B = self.block_size
        pos = seq.n
        if pos % B == 0:
            seq.blocks.append(self._take())
        else:
            last = seq.blocks[-1]
            if self.ref[last] > 1:
                fresh = self._take()
                pairs.append((last, fresh))
                self.ref[last] -= 1
                seq.blocks[-1] = fresh
                self.cow_copies += 1
        seq.n = pos + 1
        return seq.blocks[pos // B] * B + pos % B

    def _transaction(self, fn):
        """Run ``fn`` on the live state; restore everything if it raises."""
        saved = copy.deepcopy((self.seqs, self.ref, self.free, self.forks, self.cow_copies,
                               self.swapped, self.root, self.nodes, self.tick, self.next_nid,
                               self.cache_hit_blocks, self.cache_evictions))
        try:
            return fn()
        except BlockManagerError:
            (self.seqs, self.ref, self.free, self.forks, self.cow_copies, self.swapped, self.root,
             self.nodes, self.tick, self.next_nid, self.cache_hit_blocks,
             self.cache_evictions) = saved
            raise

    def _live(self, seq_id: int) -> _Seq:
        if seq_id in self.seqs:
            return self.seqs[seq_id]
        if seq_id in self.swapped:
            raise Swapped(seq_id)
        raise UnknownSeq(seq_id)

    # -- API ----------------------------------------------------------------
    def add_seq(self, seq_id: int, n_tokens: int) -> list[int]:
        """New sequence holding ``n_tokens`` tokens (a prefill); returns their slots."""
        if seq_id in self.seqs or seq_id in self.swapped:
            raise SeqExists(seq_id)
        if n_tokens < 0:
            raise InvalidArg("n_tokens < 0")

        def run():
            self._make_room(-(-n_tokens // self.block_size))
            seq = _Seq()
            self.seqs[seq_id] = seq
            pairs: list = []
            return [self._write_one(seq, pairs) for _ in range(n_tokens)]

        return self._transaction(run)

    def append_slots(self, seq_ids, tokens_each: int):
        """Append ``tokens_each`` tokens to every listed sequence, in batch order.

        Returns (slots, copy_pairs): slots in batch order (sequence-major) and
        the (src, dst) block copies copy-on-write requires, in the order made.
        """
        ids = [int(s) for s in seq_ids]
        if tokens_each < 0:
            raise InvalidArg("tokens_each < 0")
        seen = set()
        for s in ids:  # in batch order: the first unknown, swapped or repeated id decides
            self._live(s)
            if s in seen:
                raise InvalidArg("a batch may name a sequence only once")
            seen.add(s)

        def run():
            self._make_room(self._append_need(ids, tokens_each))
            slots: list[int] = []
            pairs: list = []
            for s in ids:
                seq = self.seqs[s]
                for _ in range(tokens_each):
                    slots.append(self._write_one(seq, pairs))
            return slots, pairs

        return self._transaction(run)

    def fork(self, parent: int, child: int) -> None:
        """Child shares every block of the parent (no copy); counts go up by one."""
        src = self._live(parent)
        if child in self.seqs or child in self.swapped:
            raise SeqExists(child)
        seq = _Seq()
        seq.blocks = list(src.blocks)
        seq.n = src.n
        for b in seq.blocks:
            self.ref[b] += 1
        self.seqs[child] = seq
        self.forks += 1

    def free_seq(self, seq_id: int) -> None:
        """Drop a sequence; blocks whose count reaches zero rejoin the pool."""
        if seq_id in self.swapped:  # holds no blocks
            del self.swapped[seq_id]
            return
        if seq_id not in self.seqs:
            raise UnknownSeq(seq_id)
        seq = self.seqs.pop(seq_id)
        for b in seq.blocks:
            self._release(b)

    def block_tables(self, seq_ids, max_blocks: int):
        """Per-sequence rows of physical block ids, padded with -1, and lengths."""
        rows, lens = [], []
        for s in seq_ids:
            seq = self._live(s)
            if len(seq.blocks) > max_blocks:
                raise InvalidArg("sequence needs more than max_blocks blocks")
            rows.append(seq.blocks + [-1] * (max_blocks - len(seq.blocks)))
            lens.append(seq.n)
        return rows, lens

    def seq_len(self, seq_id: int) -> int:
        if seq_id in self.swapped:
            return self.swapped[seq_id]
        if seq_id not in self.seqs:
            raise UnknownSeq(seq_id)
        return self.seqs[seq_id].n

    def swap_out(self, seq_id: int) -> list[int]:
        """Pause a sequence: returns its physical blocks in logical order (the contents
        to keep in host memory) and drops its references as freeing it would."""
        if seq_id in self.swapped:
            raise Swapped(seq_id)
        if seq_id not in self.seqs:
            raise UnknownSeq(seq_id)
        seq = self.seqs.pop(seq_id)
        for b in seq.blocks:
            self._release(b)
        self.swapped[seq_id] = seq.n
        self.swap_outs += 1
        return list(seq.blocks)

    def swap_in(self, seq_id: int) -> list[int]:
        """Resume a swapped sequence on ceil(n / B) fresh private blocks; returns them in
        logical order (where its saved contents go back)."""
        if seq_id in self.seqs:
            raise InvalidArg("sequence is not swapped out")
        if seq_id not in self.swapped:
            raise UnknownSeq(seq_id)
        n = self.swapped[seq_id]
        k = -(-n // self.block_size)

        def run():
            self._make_room(k)
            seq = _Seq()
            seq.blocks = [self._take() for _ in range(k)]
            seq.n = n
            del self.swapped[seq_id]
            self.seqs[seq_id] = seq
            self.swap_ins += 1
            return list(seq.blocks)

        return self._transaction(run)

    def truncate(self, seq_id: int, n_keep: int) -> None:
        """Keep the first ``n_keep`` tokens; blocks past them lose this reference."""
        seq = self._live(seq_id)
        if not 0 <= n_keep <= seq.n:
            raise InvalidArg("n_keep outside [0, n]")
        keep = -(-n_keep // self.block_size)
        for b in seq.blocks[keep:]:
            self._release(b)
        del seq.blocks[keep:]
        seq.n = n_keep

    def add_seq_cached(self, seq_id: int, tokens) -> tuple[list[int], int]:
        """New sequence of the given token ids reusing its longest cached prefix of full
        blocks; returns (slots of every position, number of cached tokens)."""
        if seq_id in self.seqs or seq_id in self.swapped:
            raise SeqExists(seq_id)
        toks = [int(t) for t in tokens]
        B = self.block_size
        matched, children = [], self.root
        for j in range(len(toks) // B):
            node = children.get(tuple(toks[j * B:(j + 1) * B]))
            if node is None:
                break
            matched.append(node)
            children = node.children
        need = -(-len(toks) // B) - len(matched)
        # the matched blocks are referenced first, so eviction cannot take them
        for node in matched:
            self.ref[node.block] += 1
        short = need - len(self.free)
        if short > 0 and self._evictable() < short:
            for node in matched:
                self.ref[node.block] -= 1
            raise OutOfBlocks("free pool and evictable cache too small")
        for node in matched:
            node.last_use = self.tick
        self.tick += 1
        self._make_room(need)
        seq = _Seq()
        seq.blocks = [node.block for node in matched]
        seq.n = len(matched) * B
        self.seqs[seq_id] = seq
        pairs: list = []
        for _ in range(len(toks) - seq.n):
            self._write_one(seq, pairs)
        self.cache_hit_blocks += len(matched)
        slots = [seq.blocks[j // B] * B + j % B for j in range(len(toks))]
        return slots, len(matched) * B

    def cache_insert(self, seq_id: int, tokens) -> int:
        """Cache the full blocks of a live sequence's first len(tokens) tokens (the caller
        vouches that they are its tokens); returns the number of nodes added."""
        seq = self._live(seq_id)
        toks = [int(t) for t in tokens]
        if len(toks) > seq.n:
            raise InvalidArg("more tokens than the sequence holds")
        B = self.block_size
        children, parent, added = self.root, None, 0
        for j in range(len(toks) // B):
            key = tuple(toks[j * B:(j + 1) * B])
            node = children.get(key)
            if node is None:
                node = _Node(seq.blocks[j], key, parent, self.tick, self.next_nid)
                self.next_nid += 1
                self.ref[node.block] += 1
                children[key] = node
                self.nodes.append(node)
                added += 1
            node.last_use = self.tick
            children, parent = node.children, node
        self.tick += 1
        return added

    def cache_evict(self, n_blocks: int) -> int:
        """Evict up to n_blocks least recently used unreferenced leaves; returns how many."""
        if n_blocks < 0:
            raise InvalidArg("n_blocks < 0")
        done = 0
        while done < n_blocks and self._evict_one():
            done += 1
        return done

    def refcount(self, block: int) -> int:
        if not 0 <= block < self.num_blocks:
            raise InvalidArg("block id out of range")
        return self.ref[block]

    def stats(self) -> dict:
        B = self.block_size
        used = sum(1 for r in self.ref if r > 0)
        logical_blocks = sum(len(s.blocks) for s in self.seqs.values())
        tokens = sum(s.n for s in self.seqs.values())
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": len(self.free),
            "used_blocks": used,
            "shared_blocks": sum(1 for r in self.ref if r > 1),
            "num_seqs": len(self.seqs),
            "logical_blocks": logical_blocks,
            "live_tokens": tokens,
            "tail_waste_slots": logical_blocks * B - tokens,
            "forks": self.forks,
            "cow_copies": self.cow_copies,
            "swapped_seqs": len(self.swapped),
            "swapped_tokens": sum(self.swapped.values()),
            "swap_outs": self.swap_outs,
            "swap_ins": self.swap_ins,
            "cached_blocks": len(self.nodes),
            "cache_hit_blocks": self.cache_hit_blocks,
            "cache_evictions": self.cache_evictions,
        }
