#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV-cache hot path on one MI355X.

Workload: the Llama-3-70B-shaped decode layer -- batch 256, 64 query / 8 kv heads,
head_dim 128, bf16, block size 16, log-normal context lengths (median 1,024, clipped to
[16, 8,192]) in a pool fragmented by 10,000 steps of alloc/free churn.  Synthetic, seeded
values (N(0,1) rounded to bf16).

One step = the whole hot path for one batch:
  host  : pa_bm_append_step (one token per sequence: slots, copy-on-write decisions and the
          new lengths in one pass) into pinned host buffers (2 KB);
  device: pa_copy_blocks (if any pairs) -> pa_decode_step: one launch that reads the pinned
          slots and lengths directly and does the cache write + the block-table entries the
          step created (on the device-resident tables) together with the decode planning,
          then the split-K decode and the merge.
The block tables are uploaded once before the timed steps and from then on live on the device.

Prints one JSON line.  ``value`` is the step's algorithmic HBM traffic divided by the step
time (GB/s); tokens/s is the batch size over the step time.  ``roofline`` reports the
pa_decode_step call (cache write + plan, split-K kernel, merge): HIP events on the stream it runs
on bracket the timed region, and the region's time over the steps is the call's average
duration.
"""

from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "pa_decode_step_llama70b_b256.md")


def measured_traffic():
    """HBM bytes per pa_decode_step call from the committed rocprofv3 counter summary (FETCH_SIZE and
    WRITE_SIZE passes, scaled by a plain copy of known size), or None when the summary is
    missing or was taken on kernel sources other than the current ones."""
    import hashlib
    try:
        text = open(COUNTER_SUMMARY).read()
    except OSError:
        return None
    fields = dict(l.split(": ", 1) for l in text.splitlines()
                  if l.startswith(("kernel_sources", "traffic_bytes_per_call")) and ": " in l)
    try:
        srcs = fields["kernel_sources"].split()
        digest = hashlib.sha256(b"".join(open(os.path.join(ROOT, p), "rb").read()
                                         for p in srcs)).hexdigest()
        if digest != fields["kernel_sources_sha256"].strip():
            return None
        return int(fields["traffic_bytes_per_call"])
    except (KeyError, OSError, ValueError):
        return None


def algorithmic_bytes(lens, w, T, with_write=True):
    """Bytes the decode step must move (exact token counts):
    K and V of every context token, q and out, table entries in use and lengths, and the
    cache write of the T new tokens (read + write)."""
    elt = 2 if w.dtype == "bf16" else 4
    B = w.block_size
    lens = np.asarray(lens, np.int64)
    S = len(lens)
    kv = int(lens.sum()) * w.hkv * w.head_dim * 2 * elt
    qo = 2 * S * w.hq * w.head_dim * elt
    meta = 4 * int(((lens + B - 1) // B).sum()) + 4 * S
    write = T * w.hkv * w.head_dim * 2 * elt * 2 if with_write else 0
    return kv + qo + meta, write


WORKLOADS = {
    "llama70b": "llama3-70b-shaped decode layer, batch 256, 64/8 heads, D=128, B=16, log-normal "
                "ctx (median 1024, [16, 8192])",
    "mistral7b": "mistral-7b-shaped decode layer, batch 64, 32/8 heads, D=128, B=16, "
                 "ctx U[128, 4096]",
    "long32k": "long-context decode, batch 32 x 32768 tokens, 64/8 heads, D=128, B=32",
    "shared16": "shared 1024-token prefix + copy-on-write forks, 224 sequences, 32/8 heads, "
                "D=128, B=16",
    "shared32": "shared 1024-token prefix + copy-on-write forks, 224 sequences, 32/8 heads, "
                "D=128, B=32",
    "chunk": "chunked-query prefill, 8 sequences x 512 new tokens over 4096 cached, 64/8 heads, "
             "D=128, B=32, causal inside the chunk",
    "swap": "preemption by swapping: every 8th sequence of the llama3-70b-shaped batch (32 of "
            "256) swapped out to pinned host memory and back in",
}
PCIE_PEAK_GBS = 63.0  # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes x 128/130 / 8


def make_workload(wl, name, pool, block_size=16, batch=0):
    if name in ("llama70b", "swap"):
        kw = {"S": batch} if batch else {}
        if pool == "churned":
            return wl.llama70b(B=block_size, **kw)
        w = wl.llama70b(churn_steps=0, B=block_size, **kw)
    elif name == "mistral7b":
        w = wl.mistral()
    elif name == "long32k":
        w = wl.long_context(**({"S": batch} if batch else {}))
    elif name == "shared16":
        w = wl.shared_prefix(B=16)
    elif name == "shared32":
        w = wl.shared_prefix(B=32)
    else:
        w = wl.chunked()
    if pool == "contiguous":
        w.free_order = np.arange(w.num_blocks, dtype=np.int32)
    return w


def unique_kv_bytes(tables, lens, w):
    """K/V bytes of the distinct physical blocks a batch reads (each block counted once, with
    the largest number of its slots any sequence uses)."""
    B = w.block_size
    used = {}
    for row, n in zip(tables, lens):
        for j in range((int(n) + B - 1) // B):
            p = int(row[j])
            used[p] = max(used.get(p, 0), min(B, int(n) - j * B))
    elt = 2 if w.dtype == "bf16" else 4
    return sum(used.values()) * w.hkv * w.head_dim * 2 * elt


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="llama70b",
                    help="llama70b (default, the headline batch); the others are the remaining "
                         "configurations of the path, measured the same way")
    ap.add_argument("--partition", type=int, default=0, help="split-K partition tokens (0 = auto)")
    ap.add_argument("--cpu-seqs", type=int, default=256,
                    help="sequences of the batch the CPU oracle baseline runs (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum oracle time for the CPU baseline (the sample is repeated)")
    ap.add_argument("--pool", choices=["churned", "contiguous"], default="churned",
                    help="churned: the workload's scattered pool (the llama70b pool is also "
                         "fragmented by 10,000 alloc/free steps); contiguous: identity free order "
                         "and no churn, so each sequence's blocks are physically consecutive (the "
                         "contiguous-cache comparison)")
    ap.add_argument("--block-size", type=int, choices=[16, 32, 64], default=16,
                    help="block size of the llama70b / swap batch (the block-size trade-off: "
                         "table entries, tail waste, kernel rate)")
    ap.add_argument("--batch", type=int, default=0,
                    help="llama70b / long32k: number of sequences (0 = the workload's own: 256 / "
                         "32); e.g. 1 for the batch-1 paging-overhead comparison with --pool")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before the timed steps, run one device-to-device copy of this many MiB "
                         "(a plain copy of known size that calibrates the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the decode path needs no "
                          "collective; run with --gpus 1"}), flush=True)
        return 2

    import torch

    from paged_kv_cache_378_amd import workloads as wl
    from paged_kv_cache_378_amd.runner import PagedState

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.block_size != 16 and args.workload not in ("llama70b", "swap"):
        print(json.dumps({"error": "--block-size applies to the llama70b and swap workloads"}))
        return 2
    if args.batch and args.workload not in ("llama70b", "long32k"):
        print(json.dumps({"error": "--batch applies to the llama70b and long32k workloads"}))
        return 2
    w = make_workload(wl, args.workload, args.pool, args.block_size, args.batch)
    t_setup = time.perf_counter()
    st = PagedState(w, dev, poison=True)
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup
    if args.calib_copy_mib > 0:
        src_buf = torch.ones(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst_buf = torch.empty_like(src_buf)
        torch.cuda.synchronize()
        dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf
    run = run_chunk if w.chunk else (run_swap if args.workload == "swap" else run_decode)
    line = run(args, w, st, t_setup)
    print(json.dumps(line), flush=True)
    return 0 if "error" not in line else 1


SPREAD_BLOCKS = 5  # blocks of steps timed after the main region, for the per-step spread


def timed_loop(args, step, spread=False, on_timed_end=None):
    """Warm-up, then exactly args.steps timed steps between two device synchronisations, with
    the set-up's Python objects frozen and the cyclic GC off (a collection over the workload
    script once stalled one step for tens of milliseconds).  Returns the wall-clock seconds of
    the timed steps and the milliseconds between two HIP events recorded on the launch stream
    at the start and the end of the timed region.  With `spread`, SPREAD_BLOCKS more blocks of
    spread_steps(args) steps follow the timed region, each between its own pair of events (an
    event per step would add its own gap to every step), and a third value lists their
    per-step milliseconds."""
    import torch
    gc.collect()
    gc.freeze()
    gc.disable()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    try:
        for i in range(args.warmup):
            step(i, False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record()
        for i in range(args.warmup, args.warmup + args.steps):
            step(i, True)
        ev1.record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        if on_timed_end:
            on_timed_end()
        blocks = []
        if spread:
            # the blocks follow each other with no synchronisation between them, so the stream
            # never runs dry; the events are read once all have completed
            n = spread_steps(args)
            i = args.warmup + args.steps
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(SPREAD_BLOCKS)]
            for e0, e1 in evs:
                e0.record()
                for _ in range(n):
                    step(i, False)
                    i += 1
                e1.record()
            torch.cuda.synchronize()
            blocks = [e0.elapsed_time(e1) / n for e0, e1 in evs]
        if spread:
            return elapsed, ev0.elapsed_time(ev1), blocks
        return elapsed, ev0.elapsed_time(ev1)
    finally:
        gc.enable()


def spread_steps(args):
    return max(1, args.steps // SPREAD_BLOCKS)


def spread_summary(blocks):
    """Per-step milliseconds of the spread blocks: p10, median, p90."""
    b = np.asarray(blocks, np.float64)
    return {"p10_ms": round(float(np.percentile(b, 10)), 4),
            "median_ms": round(float(np.median(b)), 4),
            "p90_ms": round(float(np.percentile(b, 90)), 4),
            "blocks": len(blocks), "steps_per_block": None}


def base_line(args, w, ms_step):
    return {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
            "data": "synthetic"}


def run_decode(args, w, st, t_setup):
    """One decode step of the whole path per iteration (host block manager, copy-on-write
    copies, cache write + table patch, plan + split-K decode + merge)."""
    import torch

    from paged_kv_cache_378_amd import _lib

    dev = st.device
    S, B = w.num_seqs, w.block_size
    total = args.warmup + args.steps + SPREAD_BLOCKS * spread_steps(args)
    max_ctx = st.max_ctx + total
    max_blocks = (max_ctx + B - 1) // B
    nbytes = _lib.pa_decode_workspace_size(S, w.hq, w.head_dim, max_ctx, args.partition)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    out = st.new_out()
    ids = np.asarray(w.step_ids, np.int64)

    # Block tables and lengths live on the device.  Each step's slots and lengths (2 KB) are
    # written into a ring of pinned host buffers that pa_decode_step's first kernel reads
    # directly, so there is no upload.  A buffer is rewritten RING steps after its last use; the
    # host checks that use is over on an event recorded once every MARK steps (long complete by
    # then), never on the step just enqueued.
    tables0, lens0 = st.bm.block_tables(ids, max_blocks)
    tables_d = torch.from_numpy(tables0).to(dev)
    lens_d = torch.from_numpy(lens0).to(dev)
    RING, MARK = 16, 8
    pin_slots = [torch.empty(S, dtype=torch.int32).pin_memory() for _ in range(RING)]
    pin_lens = [torch.empty(S, dtype=torch.int32).pin_memory() for _ in range(RING)]
    pairs_h = np.empty((S, 2), np.int32)
    # the host half of the step: one pa_bm_append_step call (slots, copy-on-write pairs and the
    # new lengths in one pass) straight into the pinned buffers, its arguments marshalled once
    append_step = st.bm.prepare_append_step(ids, 1, [t.numpy() for t in pin_slots],
                                            [t.numpy() for t in pin_lens], pairs_h)
    marks = [torch.cuda.Event() for _ in range(4)]
    stream = torch.cuda.current_stream()
    host_s, step_lens, n_pairs = [], [], []

    def step(i, timed):
        r = i % RING
        if i >= RING:
            # step i - RING read buffer r; the mark of its group of MARK steps was recorded
            # after step i - RING + MARK - 1 < i at the latest, and is not yet re-recorded
            marks[((i - RING) // MARK) % len(marks)].synchronize()
        slots_h, lens_h = pin_slots[r], pin_lens[r]
        h0 = time.perf_counter()
        np_ = append_step(r)
        if timed:
            host_s.append(time.perf_counter() - h0)
            step_lens.append(lens_h.numpy().copy())
        n_pairs.append(np_)
        if np_:
            _lib.pa_copy_blocks(st.k_cache, st.v_cache, torch.from_numpy(pairs_h[:np_]).to(dev))
        _lib.pa_decode_step(out, st.vals["q"], st.vals["k_step"], st.vals["v_step"], st.k_cache,
                            st.v_cache, slots_h, tables_d, lens_d, max_ctx, w.scale,
                            args.partition, ws, new_ctx_lens=lens_h)
        if i % MARK == MARK - 1:
            marks[(i // MARK) % len(marks)].record(stream)

    pool_end, tables_end = {}, []

    def at_timed_end():  # pool statistics and tables as the last timed step left them
        pool_end.update(st.bm.stats())
        tables_end.extend(st.bm.block_tables(ids, max_blocks))

    elapsed, region_ms, blocks = timed_loop(args, step, spread=True, on_timed_end=at_timed_end)
    if not torch.isfinite(out.float()).all():
        return {"error": "non-finite decode output"}
    # the device-resident tables and lengths must still mirror the block manager's exactly
    final_tables, final_lens = st.bm.block_tables(ids, max_blocks)
    if not np.array_equal(tables_d.cpu().numpy(), final_tables) or \
            not np.array_equal(lens_d.cpu().numpy(), final_lens):
        return {"error": "device block tables diverged from the block manager"}

    ms_step = 1e3 * elapsed / args.steps
    # Each step puts one pa_decode_step call on the stream (plus pa_copy_blocks where a step
    # has copy-on-write pairs), so the event time of the region over the steps is the call's
    # average duration, launch gaps between calls included.
    dec_avg_ms = region_ms / args.steps
    dec_bytes, write_bytes = zip(*[algorithmic_bytes(l, w, S) for l in step_lens])
    # the timed call is pa_decode_step: decode bytes plus the new tokens' cache write
    dec_bytes_avg = float(np.mean(dec_bytes)) + float(np.mean(write_bytes))
    step_bytes_avg = dec_bytes_avg
    tokens = int(np.mean([l.sum() for l in step_lens]))
    shared = args.workload.startswith("shared")
    extra = {}
    if shared:
        # shared prefix blocks are read once per sequence but live once in HBM: the roofline
        # counts each physical block once; the logical (per-sequence) rate is "effective"
        elt = 2
        logical_kv = tokens * w.hkv * w.head_dim * 2 * elt
        uniq = unique_kv_bytes(tables_end[0], tables_end[1], w)
        extra = {"effective_logical_GBps": round(dec_bytes_avg / (dec_avg_ms * 1e-3) / 1e9, 1),
                 "unique_kv_bytes": uniq, "logical_kv_bytes": logical_kv,
                 "cow_pairs_first_step": n_pairs[0], "cow_pairs_later_steps": sum(n_pairs[1:])}
        dec_bytes_avg = dec_bytes_avg - logical_kv + uniq
        step_bytes_avg = step_bytes_avg - logical_kv + uniq
    achieved = dec_bytes_avg / (dec_avg_ms * 1e-3) / 1e9
    value = step_bytes_avg / (ms_step * 1e-3) / 1e9
    headline = args.workload == "llama70b" and not args.batch
    cpu = None
    if args.cpu_seqs > 0 and headline:
        cpu = cpu_baseline(w, st, args.cpu_seqs, args.cpu_seconds)
    line = {"metric": "paged decode attention: HBM GB/s (% of peak) + decode tokens/s at batch 256",
            "value": round(value, 1), "unit": "GB/s"}
    line.update(base_line(args, w, ms_step))
    line.update({
        "config": {"workload": WORKLOADS[args.workload] + ", %s pool" % args.pool,
                   "global_batch": S, "seq_len": "mean %d" % (tokens // S),
                   "context_tokens": tokens, "partition_tokens": args.partition or "auto",
                   "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(S / (ms_step * 1e-3), 1),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "host_block_manager_us": round(1e6 * float(np.median(host_s)), 1),
        "block_size": w.block_size,
        "pool": {k: pool_end[k] for k in ("logical_blocks", "live_tokens", "tail_waste_slots",
                                          "used_blocks", "num_blocks")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic()
                     if headline and args.pool == "churned" and w.block_size == 16 else None,
                     "kernel": "pa_decode_step (cache write + plan, persistent split-K decode, "
                               "merge); avg_ms = HIP-event time of the timed region / steps",
                     "avg_ms": round(dec_avg_ms, 4), "algorithmic_bytes": int(dec_bytes_avg)},
        "cpu_baseline": cpu,
        "step_ms_spread": dict(spread_summary(blocks), steps_per_block=spread_steps(args),
                               note="per-step time of %d further blocks of steps after the "
                                    "timed region, each between its own HIP events"
                                    % SPREAD_BLOCKS),
        "setup_s": round(t_setup, 1),
    })
    line.update(extra)
    return line


def chunk_flops(lens, C, w):
    """Causal-exact attention flops of a chunk step: 4 D Hq per (query, visible key) pair."""
    pairs = sum(sum(int(n) - C + i + 1 for i in range(C)) for n in lens)
    return 4 * w.head_dim * w.hq * pairs


def run_chunk(args, w, st, t_setup):
    """The chunk step: the block manager appends C tokens to every sequence (once, before the
    timing), then each timed iteration replays the step's device work on the same slots and
    values -- cache write + table patch of the S*C new tokens, then chunked-query attention --
    so the pool does not grow from iteration to iteration."""
    import torch

    from paged_kv_cache_378_amd import _lib

    dev = st.device
    S, B, C = w.num_seqs, w.block_size, w.step_tokens
    ids = np.asarray(w.step_ids, np.int64)
    max_ctx = max(w.ctx_lens())
    max_blocks = (max_ctx + B - 1) // B
    tables0, lens_before = st.bm.block_tables(ids, max_blocks)
    slots, pairs = st.bm.append_slots(ids, C)
    lens = st.bm.seq_lens(ids)
    assert not len(pairs)
    tables_d = torch.from_numpy(tables0).to(dev)
    lens_d = torch.from_numpy(lens).to(dev)
    slots_d = torch.from_numpy(slots).to(dev)
    out = st.new_out()
    stream = torch.cuda.current_stream()
    ev_pool = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    events = []

    def step(i, timed):
        _lib.pa_cache_append(st.vals["k_step"], st.vals["v_step"], st.k_cache, st.v_cache, slots_d,
                             tables_d, lens_d, C)
        if timed:
            e0, e1 = ev_pool[len(events)]
            e0.record(stream)
        _lib.pa_chunk_attend(out, st.vals["q"], st.k_cache, st.v_cache, tables_d, lens_d, w.scale)
        if timed:
            e1.record(stream)
            events.append((e0, e1))

    elapsed, _ = timed_loop(args, step)
    if not torch.isfinite(out.float()).all():
        return {"error": "non-finite chunk output"}
    if not np.array_equal(tables_d.cpu().numpy(), st.bm.block_tables(ids, max_blocks)[0]):
        return {"error": "device block tables diverged from the block manager"}
    ms_step = 1e3 * elapsed / args.steps
    att_ms = float(np.mean([a.elapsed_time(b) for a, b in events]))
    flops = chunk_flops(lens, C, w)
    elt = 2
    kv = int(np.sum(lens)) * w.hkv * w.head_dim * 2 * elt
    qo = 2 * S * C * w.hq * w.head_dim * elt
    write = S * C * w.hkv * w.head_dim * 2 * elt * 2
    achieved = flops / (att_ms * 1e-3) / 1e12
    value = flops / (ms_step * 1e-3) / 1e12
    line = {"metric": "chunked-query paged attention: TFLOP/s (causal-exact flops)",
            "value": round(value, 1), "unit": "TFLOP/s"}
    line.update(base_line(args, w, ms_step))
    line.update({
        "config": {"workload": WORKLOADS["chunk"] + ", %s pool" % args.pool, "global_batch": S,
                   "chunk_tokens": C, "context_tokens": int(np.sum(lens)),
                   "parallelism": "none (1 GPU)"},
        "prefill_tokens_per_s": round(S * C / (ms_step * 1e-3), 1),
        "step_bytes": kv + qo + write,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "pa_chunk_attend (chunk_kernel)",
                     "avg_ms": round(att_ms, 4), "algorithmic_flops": flops},
        "cpu_baseline": None,
        "setup_s": round(t_setup, 1),
    })
    return line


def run_swap(args, w, st, t_setup):
    """One step = pause 32 sequences (pa_bm_swap_out, then one pa_swap_blocks copy of all their
    blocks to pinned host memory) and resume them (pa_bm_swap_in onto fresh blocks, one copy
    back).  Each copy is timed with HIP events on its stream; the decode of the whole batch
    after the last step must equal the decode before the first, bit for bit."""
    import torch

    from paged_kv_cache_378_amd import _lib

    dev = st.device
    S, B, H, D = w.num_seqs, w.block_size, w.hkv, w.head_dim
    ids = [int(i) for i in w.step_ids]
    victims = ids[::8]
    max_ctx = max(w.ctx_lens())
    max_blocks = (max_ctx + B - 1) // B
    ws = torch.empty(_lib.pa_decode_workspace_size(S, w.hq, D, max_ctx, 0), dtype=torch.uint8,
                     device=dev)

    def decode():
        t, l = (torch.from_numpy(x).to(dev) for x in st.bm.block_tables(ids, max_blocks))
        out = st.new_out()
        _lib.pa_decode(out, st.vals["q"], st.k_cache, st.v_cache, t, l, max_ctx, w.scale, 0, ws)
        torch.cuda.synchronize()
        return out

    before = decode()
    nblk = sum(-(-st.bm.seq_len(v) // B) for v in victims)
    slab = H * B * D
    host = torch.empty(nblk * 2 * slab, dtype=st.k_cache.dtype).pin_memory()
    out_list = torch.empty(nblk, dtype=torch.int32).pin_memory()
    in_list = torch.empty(nblk, dtype=torch.int32).pin_memory()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    times = []

    def step(i, timed):
        o = 0
        for v in victims:
            b = st.bm.swap_out(v)
            out_list.numpy()[o:o + len(b)] = b
            o += len(b)
        e = ev[len(times)] if timed else None
        if timed:
            e[0].record(stream)
        _lib.pa_swap_blocks(st.k_cache, st.v_cache, host, out_list, to_host=True)
        if timed:
            e[1].record(stream)
        o = 0
        for v in victims:
            b = st.bm.swap_in(v)
            in_list.numpy()[o:o + len(b)] = b
            o += len(b)
        if timed:
            e[2].record(stream)
        _lib.pa_swap_blocks(st.k_cache, st.v_cache, host, in_list, to_host=False)
        if timed:
            e[3].record(stream)
            times.append(e)
        # the block lists and the host buffer are reused next step: wait for this one
        torch.cuda.synchronize()

    elapsed, _ = timed_loop(args, step)
    after = decode()
    it = torch.int16 if w.dtype == "bf16" else torch.int32
    if not torch.equal(before.view(it), after.view(it)):
        return {"error": "decode changed across swap-out / swap-in"}
    ms_step = 1e3 * elapsed / args.steps
    d2h_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in times]))
    h2d_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in times]))
    nbytes = nblk * 2 * slab * st.k_cache.element_size()
    achieved = 2 * nbytes / ((d2h_ms + h2d_ms) * 1e-3) / 1e9
    line = {"metric": "swap: host-link GB/s (paused sequences' blocks out to pinned host memory "
                      "and back)",
            "value": round(2 * nbytes / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s"}
    line.update(base_line(args, w, ms_step))
    line.update({
        "config": {"workload": WORKLOADS["swap"], "swapped_sequences": len(victims),
                   "blocks": nblk, "bytes_each_way": nbytes, "parallelism": "none (1 GPU)"},
        "d2h_GBps": round(nbytes / (d2h_ms * 1e-3) / 1e9, 2),
        "h2d_GBps": round(nbytes / (h2d_ms * 1e-3) / 1e9, 2),
        "roofline": {"bound": "pcie", "achieved": round(achieved, 2), "peak": PCIE_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / PCIE_PEAK_GBS, 4), "traffic": None,
                     "kernel": "pa_swap_blocks (both directions; one direction at a time)",
                     "avg_ms": round(d2h_ms + h2d_ms, 4), "algorithmic_bytes": 2 * nbytes},
        "cpu_baseline": None,
        "setup_s": round(t_setup, 1),
    })
    return line


def cpu_baseline(w, st, n_seqs, min_seconds):
    """The fp64 oracle on the first n_seqs sequences of the batch, one thread, repeated until it
    has run for min_seconds (the batch's K/V are copied to the host once, outside the timing)."""
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import attention as att
    from paged_kv_cache_378_amd import workloads as wl

    n_seqs = min(n_seqs, w.num_seqs)
    q = st.vals["q"]
    batch = []
    tokens = 0
    for i in range(n_seqs):
        ks, vs = wl.logical_kv(w, w.step_ids[i], st.vals)
        K = torch.cat(ks).to("cpu", torch.float64).numpy()
        V = torch.cat(vs).to("cpu", torch.float64).numpy()
        batch.append((q[i].to("cpu", torch.float64).numpy(), K, V))
        tokens += K.shape[0]
    busy = 0.0
    done = 0
    with threadpool_limits(limits=1):
        torch_threads = torch.get_num_threads()
        torch.set_num_threads(1)
        try:
            while busy < min_seconds:
                for qi, K, V in batch:
                    t0 = time.perf_counter()
                    att.dense_decode(qi, K, V, w.scale)
                    busy += time.perf_counter() - t0
                    done += 1
        finally:
            torch.set_num_threads(torch_threads)
    return {"value": round(done / busy, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the first {n_seqs} of {w.num_seqs} sequences of one decode step "
                      f"({tokens} context tokens, all {w.hq} heads), numpy fp64, 1 thread, run "
                      f"{done // n_seqs}x ({done} sequence-steps in {busy:.1f} s of oracle time; "
                      f"the host copy of K/V is not timed)",
            "oracle_s": round(busy, 2)}


if __name__ == "__main__":
    sys.exit(main())
