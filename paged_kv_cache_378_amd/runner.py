"""Drive a workload through libpa: build the pool state, then run timed steps.

Only sequences library calls (block manager on the host, kernels on the device);
every number the path produces comes from libpa.

A decode step is the hot path of one serving iteration:
  1. host: ``pa_bm_append_slots`` (one token per sequence, copy-on-write decisions),
     ``pa_bm_block_tables`` into a pinned staging buffer;
  2. one async host->device copy of slots, copy pairs, block tables and lengths;
  3. device: ``pa_copy_blocks`` -> ``pa_cache_write`` -> ``pa_decode`` (split-K + merge),
     or ``pa_chunk_attend`` for a chunk step.
"""

from __future__ import annotations

import numpy as np
import torch

from . import _lib
from .workloads import Workload, replay, torch_dtype, value_tensor

NAN_BITS = {torch.float32: (torch.int32, 0x7FC00000), torch.bfloat16: (torch.int16, 0x7FC0)}


def poison_(t: torch.Tensor) -> torch.Tensor:
    """Fill a pool with a quiet-NaN bit pattern (memory that must never reach an output)."""
    it, bits = NAN_BITS[t.dtype]
    t.view(it).fill_(bits)
    return t


class PagedState:
    """Pool, block manager and value tensors of one workload on one device."""

    def __init__(self, w: Workload, device="cuda", poison: bool = True, values=None,
                 free_order=None):
        self.w = w
        self.device = torch.device(device)
        dt = torch_dtype(w)
        NB, H, B, D = w.num_blocks, w.hkv, w.block_size, w.head_dim
        self.k_cache = torch.empty((NB, H, B, D), dtype=dt, device=self.device)
        self.v_cache = torch.empty((NB, H, D, B), dtype=dt, device=self.device)
        if poison:
            poison_(self.k_cache)
            poison_(self.v_cache)
        else:
            self.k_cache.zero_()
            self.v_cache.zero_()
        if values is None:
            values = {n: value_tensor(w, n, self.device)
                      for n in ("q", "k_prefill", "v_prefill", "k_step", "v_step")}
        self.vals = values
        order = w.free_order if free_order is None else free_order
        self.bm = _lib.BlockManager(NB, B, order)
        replay(w, self.bm, _lib.OutOfBlocks, write=self._write)
        self.max_blocks = self._max_blocks_after_step()
        self.max_ctx = max(w.ctx_lens())

    def _max_blocks_after_step(self) -> int:
        B = self.w.block_size
        return max((n + B - 1) // B for n in self.w.ctx_lens())

    def _write(self, name, row0, slots, pairs):
        dev = self.device
        if len(pairs):
            _lib.pa_copy_blocks(self.k_cache, self.v_cache,
                                torch.from_numpy(np.ascontiguousarray(pairs)).to(dev))
        n = len(slots)
        _lib.pa_cache_write(self.vals["k_" + name][row0:row0 + n],
                            self.vals["v_" + name][row0:row0 + n], self.k_cache, self.v_cache,
                            torch.from_numpy(np.ascontiguousarray(slots)).to(dev))

    # -- one step ---------------------------------------------------------------------
    def host_step(self):
        """Block-manager half of the step: slots, copy pairs, tables and lengths (host)."""
        w = self.w
        slots, pairs = self.bm.append_slots(w.step_ids, w.step_tokens)
        tables, lens = self.bm.block_tables(w.step_ids, self.max_blocks)
        return slots, pairs, tables, lens

    def upload(self, slots, pairs, tables, lens):
        dev = self.device
        return (torch.from_numpy(slots).to(dev), torch.from_numpy(np.ascontiguousarray(pairs)).to(dev),
                torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev))

    def device_step(self, slots_d, pairs_d, tables_d, lens_d, out, workspace=None,
                    partition_tokens: int = 0, max_ctx=None):
        w = self.w
        if pairs_d.numel():
            _lib.pa_copy_blocks(self.k_cache, self.v_cache, pairs_d)
        _lib.pa_cache_write(self.vals["k_step"], self.vals["v_step"], self.k_cache, self.v_cache,
                            slots_d)
        if not w.chunk:
            _lib.pa_decode(out, self.vals["q"], self.k_cache, self.v_cache, tables_d, lens_d,
                           max_ctx or self.max_ctx, w.scale, partition_tokens, workspace)
        else:
            _lib.pa_chunk_attend(out, self.vals["q"], self.k_cache, self.v_cache, tables_d,
                                 lens_d, w.scale)

    def workspace(self, partition_tokens: int = 0):
        w = self.w
        nbytes = _lib.pa_decode_workspace_size(w.num_seqs, w.hq, w.head_dim, self.max_ctx,
                                               partition_tokens)
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=self.device)

    def new_out(self):
        return torch.empty_like(self.vals["q"])

    def run_step(self, partition_tokens: int = 0):
        """Host step + upload + device step; returns (out, (slots, pairs, tables, lens))."""
        host = self.host_step()
        dev = self.upload(*host)
        out = self.new_out()
        ws = None if self.w.chunk else self.workspace(partition_tokens)
        self.device_step(*dev, out, ws, partition_tokens)
        return out, host
