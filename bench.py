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
    "ceilings": "HBM read ceilings: a streaming read of 4 GiB and a gather of 4 GiB as 4 KiB chunks "
                "in shuffled and in sequential order, swept over launch shapes; and the matrix "
                "cores' sustained bf16 rate (independent back-to-back instructions, fixed and "
                "random operands) with the shader clock they ran at",
    "paging_cost": "paging cost at small batch: the long-context decode step (32,768 tokens, "
                   "64/8 heads, D=128, B=32) over a scattered pool vs physically consecutive "
                   "blocks, alternating",
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
    ap.add_argument("--no-share-groups", action="store_true",
                    help="shared16 / shared32: decode without share groups (by default the "
                         "batch's groups from pa_bm_share_groups, taken once before the steps, are "
                         "passed to pa_decode_step_shared)")
    ap.add_argument("--flush", action="store_true",
                    help="decode workloads: write 1 GiB and read another 1 GiB before every step "
                         "and time each call by its own HIP events (no byte of the step's data "
                         "left in any cache, no dirty line to write back)")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="processes of the all-core CPU oracle leg (at most os.cpu_count(); 0 = "
                         "skip that leg)")
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
    if args.workload in ("ceilings", "paging_cost"):
        line = (run_ceilings if args.workload == "ceilings" else run_paging_cost)(args, dev)
        print(json.dumps(line), flush=True)
        return 0 if "error" not in line else 1
    if args.block_size != 16 and args.workload not in ("llama70b", "swap"):
        print(json.dumps({"error": "--block-size applies to the llama70b and swap workloads"}))
        return 2
    if args.batch and args.workload not in ("llama70b", "long32k", "paging_cost"):
        print(json.dumps({"error": "--batch applies to the llama70b, long32k and paging_cost "
                                   "workloads"}))
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


SPREAD_BLOCKS = 20  # blocks of steps timed after the main region, for the per-step spread


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
    # a few steps per block: an event pair around every step would add its own gap to each
    return max(1, args.steps // 5)


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
    ids = np.asarray(w.step_ids, np.int64)
    # the longest context the steps reach (from the current lengths: a state may have run steps)
    max_ctx = max(st.max_ctx - 1, int(st.bm.seq_lens(ids).max())) + total
    max_blocks = (max_ctx + B - 1) // B
    nbytes = _lib.pa_decode_workspace_size(S, w.hq, w.head_dim, max_ctx, args.partition)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    out = st.new_out()

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
    host_s, step_lens, n_pairs, all_lens = [], [], [], []
    # Share groups (shared-prefix workloads): the host helper's groups, taken once from the
    # batch's tables before the steps; they stay valid through the steps' copy-on-write (the
    # copies hold the same K/V at the shared positions)
    groups_d, share = None, None
    if args.workload.startswith("shared") and not args.no_share_groups:
        g = w.hq // w.hkv
        groups = st.bm.share_groups(ids, max(2, min(4, 16 // g)), 32)
        groups_d = torch.from_numpy(groups).to(dev)
        lens_now = st.bm.seq_lens(ids)
        gm = min(4, 16 // g)
        reads = int(lens_now.sum()) - sum(
            (int((r[1:] >= 0).sum()) - -(-int((r[1:] >= 0).sum()) // gm)) * (int(r[0]) // 32 * 32)
            for r in groups)
        share = {"groups": int(len(groups)),
                 "sequences_in_groups": int(sum((r[1:] >= 0).sum() for r in groups)),
                 "tokens_read_per_step": reads, "tokens_logical": int(lens_now.sum()),
                 "note": "pa_bm_share_groups once before the steps; each group's shared tokens "
                         "(rounded down to 32) are read once per item of %d members" % gm}
    # --flush: before every step, outside per-call events, a 1 GiB write and then an ordinary
    # read of another 1 GiB, so no byte of the step's data is left in the 256 MB Infinity Cache
    # or the L2s, and no dirty line either (a write alone would leave up to 256 MB of them for
    # the step to write back)
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if args.flush else None
    flush_rd = torch.ones(1 << 28, dtype=torch.int32, device=dev) if args.flush else None
    call_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)] if args.flush else []
    timed_calls = []

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
        if flush_buf is not None:
            flush_buf.fill_(i & 0xFF)
            flush_rd.amax()
            if timed:
                e0, e1 = call_ev[len(timed_calls)]
                e0.record(stream)
        if np_:
            _lib.pa_copy_blocks(st.k_cache, st.v_cache, torch.from_numpy(pairs_h[:np_]).to(dev))
        if groups_d is None:
            _lib.pa_decode_step(out, st.vals["q"], st.vals["k_step"], st.vals["v_step"],
                                st.k_cache, st.v_cache, slots_h, tables_d, lens_d, max_ctx,
                                w.scale, args.partition, ws, new_ctx_lens=lens_h)
        else:
            _lib.pa_decode_step_shared(out, st.vals["q"], st.vals["k_step"], st.vals["v_step"],
                                       st.k_cache, st.v_cache, slots_h, tables_d, lens_d, max_ctx,
                                       w.scale, groups_d, args.partition, ws,
                                       new_ctx_lens=lens_h)
        if flush_buf is not None and timed:
            e1.record(stream)
            timed_calls.append((e0, e1))
        all_lens.append(lens_h.numpy().copy())
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
    # average duration, launch gaps between calls included.  With --flush the region also holds
    # the flushes: the call's duration is then the mean of its own event pairs.
    dec_avg_ms = region_ms / args.steps
    flushed = None
    if flush_buf is not None:
        per_call = np.array([a.elapsed_time(b) for a, b in timed_calls])
        dec_avg_ms = float(per_call.mean())
        flushed = {"flush_bytes_written": flush_buf.numel(),
                   "flush_bytes_read": flush_rd.numel() * 4, "call_ms_mean": round(dec_avg_ms, 4),
                   "call_ms_p10": round(float(np.percentile(per_call, 10)), 4),
                   "call_ms_median": round(float(np.median(per_call)), 4),
                   "call_ms_p90": round(float(np.percentile(per_call, 90)), 4),
                   "note": "a 1 GiB device write and a 1 GiB read of another buffer before "
                           "every step; the call (copy-on-write copies if any + "
                           "pa_decode_step) timed by its own HIP event pair"}
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
    if flushed is not None:  # the wall clock holds the flushes: the call time is the step
        value = achieved
        ms_step = dec_avg_ms
    all_bytes = [sum(algorithmic_bytes(l, w, S)) for l in all_lens]
    headline = args.workload == "llama70b" and not args.batch and flushed is None
    cpu = None
    if args.cpu_seqs > 0 and headline:
        cpu = cpu_baseline(w, st, args.cpu_seqs, args.cpu_seconds, args.cpu_workers)
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
                     "traffic_source": "profiles/pa_decode_step_llama70b_b256.md: FETCH_SIZE + "
                                       "WRITE_SIZE per call from rocprofv3 counter runs of the "
                                       "same kernel sources (null once the sources differ); not "
                                       "measured in this run",
                     "kernel": "pa_decode_step (cache write + plan, persistent split-K decode, "
                               "merge); avg_ms = HIP-event time of the timed region / steps",
                     "avg_ms": round(dec_avg_ms, 4), "algorithmic_bytes": int(dec_bytes_avg)},
        "cpu_baseline": cpu,
        "step_ms_spread": dict(spread_summary(blocks), steps_per_block=spread_steps(args),
                               note="per-step time of %d further blocks of steps after the "
                                    "timed region, each between its own HIP events"
                                    % SPREAD_BLOCKS),
        "calls": {"count": len(all_bytes),
                  "algorithmic_bytes_mean": int(np.mean(all_bytes)),
                  "note": "every pa_decode_step call of this run (warm-up, timed, spread "
                          "blocks): a counter run of this command divides its per-dispatch "
                          "bytes by this mean"},
        "setup_s": round(t_setup, 1),
    })
    if flushed is not None:
        line["flushed"] = flushed
    if share is not None:
        line["share_groups"] = share
    line.update(extra)
    return line


def run_ceilings(args, dev):
    """Achievable HBM read rates on this GPU (libpa_probe.so): the best streaming read and the
    best gather of shuffled (and of sequential) 4 KiB chunks over a sweep of launch shapes, each
    shape timed over 10 launches after 2 warm-ups."""
    import ctypes as C

    import torch

    lib = C.CDLL(os.path.join(ROOT, "paged_kv_cache_378_amd", "libpa_probe.so"))
    lib.pa_probe_read_stream.argtypes = [C.c_void_p, C.c_size_t, C.c_int32, C.c_int32, C.c_void_p,
                                         C.POINTER(C.c_size_t), C.c_void_p]
    lib.pa_probe_read_gather.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                         C.c_void_p, C.c_void_p]
    lib.pa_probe_mfma.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                  C.c_void_p, C.c_void_p, C.POINTER(C.c_double), C.c_void_p]
    nbytes = 4 << 30
    nchunks = nbytes // 4096
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    grids = (256, 384, 512, 768, 1024, 2048)
    sink = torch.empty(max(grids) * 256, dtype=torch.int32, device=dev)
    g = torch.Generator().manual_seed(7)
    orders = {"shuffled": torch.randperm(nchunks, generator=g).to(torch.int32).to(dev),
              "sequential": torch.arange(nchunks, dtype=torch.int32, device=dev)}
    stream = torch.cuda.current_stream()
    s_ptr = stream.cuda_stream

    def timed(launch, reps=10):
        for _ in range(2):
            launch()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    stream_rows, gather_rows = [], []
    for wg in grids:
        for loads in (1, 2, 4, 8):
            got = C.c_size_t()
            st = lib.pa_probe_read_stream(buf.data_ptr(), nbytes, wg, loads, sink.data_ptr(),
                                          C.byref(got), s_ptr)
            if st:
                return {"error": f"pa_probe_read_stream({wg}, {loads}) returned {st}"}
            ms = timed(lambda: lib.pa_probe_read_stream(buf.data_ptr(), nbytes, wg, loads,
                                                        sink.data_ptr(), C.byref(got), s_ptr))
            stream_rows.append({"workgroups": wg, "loads_in_flight": loads,
                                "GBps": round(got.value / (ms * 1e-3) / 1e9, 1)})
    for name, order in orders.items():
        for wg in grids[:5]:
            for per_wave in (1, 2, 4):
                ms = timed(lambda: lib.pa_probe_read_gather(buf.data_ptr(), order.data_ptr(),
                                                            nchunks, per_wave, wg,
                                                            sink.data_ptr(), s_ptr))
                gather_rows.append({"order": name, "workgroups": wg, "chunks_per_wave": per_wave,
                                    "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)})
    # matrix cores: back-to-back independent bf16 instructions, register operands, with a fixed
    # sparse operand pattern and with random operands (the clock drops under the heavier draw)
    mfma_rows = []
    msink = torch.empty(2048 * 512, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2 * 2048, dtype=torch.int64, device=dev)
    for operands, kind in ((0, "fixed"), (1, "random")):
        for shape in (16, 32):
            for wg, waves in ((256, 4), (512, 4), (1024, 4), (512, 8), (1024, 8), (2048, 8)):
                fl = C.c_double()
                st = lib.pa_probe_mfma(shape, operands, wg, waves, 20000, msink.data_ptr(),
                                       clocks.data_ptr(), C.byref(fl), s_ptr)
                if st:
                    return {"error": f"pa_probe_mfma({shape}, {operands}, {wg}, {waves}) returned {st}"}
                ms = timed(lambda: lib.pa_probe_mfma(shape, operands, wg, waves, 20000,
                                                     msink.data_ptr(), clocks.data_ptr(),
                                                     C.byref(fl), s_ptr), reps=5)
                ck = clocks[:2 * wg].view(wg, 2).double().sum(0).tolist()
                mfma_rows.append({"shape": f"{shape}x{shape}x{512 // shape}", "operands": kind,
                                  "workgroups": wg, "waves_per_workgroup": waves,
                                  "TFLOPs": round(fl.value / (ms * 1e-3) / 1e12, 1),
                                  "clock_MHz": round(100.0 * ck[0] / ck[1]) if ck[1] else None})
    best_mfma = {f"{r0} {kind}": max((r for r in mfma_rows if r["shape"] == r0 and r["operands"] == kind),
                                     key=lambda r: r["TFLOPs"])
                 for kind in ("fixed", "random") for r0 in ("16x16x32", "32x32x16")}
    best_stream = max(stream_rows, key=lambda r: r["GBps"])
    best = {n: max((r for r in gather_rows if r["order"] == n), key=lambda r: r["GBps"])
            for n in orders}
    line = {"metric": "HBM read ceiling (best streaming read)", "value": best_stream["GBps"],
            "unit": "GB/s", "n_gpus": 1, "steps": 10, "warmup": 2, "higher_is_better": True,
            "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": WORKLOADS["ceilings"], "parallelism": "none (1 GPU)"},
            "pct_of_hbm_peak": round(100 * best_stream["GBps"] / HBM_PEAK_GBS, 2),
            "best_stream": best_stream, "best_gather_shuffled": best["shuffled"],
            "best_gather_sequential": best["sequential"],
            "gather_shuffled_pct_of_hbm_peak": round(100 * best["shuffled"]["GBps"] / HBM_PEAK_GBS, 2),
            "stream_sweep": stream_rows, "gather_sweep": gather_rows,
            "best_mfma_bf16": {k: dict(v, pct_of_bf16_peak=round(100 * v["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 2))
                               for k, v in best_mfma.items()},
            "mfma_sweep": mfma_rows}
    return line


def run_paging_cost(args, dev):
    """The contiguous-vs-paged comparison at small batch ("Taming the Tail", "Deep-Dive
    Curiosity: The Performance Trade-off": a contiguous kernel is 1-2% faster at batch 1): the
    same long-context decode step (args.batch sequences, default 1, of 32,768 tokens) over the
    workload's scattered pool and over physically consecutive blocks, run as decode-step
    benchmarks in alternation (four of each) so drift hits both the same."""
    from paged_kv_cache_378_amd import workloads as wl
    from paged_kv_cache_378_amd.runner import PagedState

    S = args.batch or 1
    states = {}
    for pool in ("churned", "contiguous"):
        w = wl.long_context(S=S)
        if pool == "contiguous":
            w.free_order = np.arange(w.num_blocks, dtype=np.int32)
        states[pool] = (w, PagedState(w, dev, poison=True))
    runs = {"churned": [], "contiguous": []}
    sub = argparse.Namespace(**vars(args))
    sub.cpu_seqs = 0
    sub.flush = False
    for _ in range(4):
        for pool in ("churned", "contiguous"):
            w, st = states[pool]
            r = run_decode(sub, w, st, 0.0)
            if "error" in r:
                return r
            runs[pool].append(r)
    med = {p: float(np.median([r["ms_per_step"] for r in rs])) for p, rs in runs.items()}
    call = {p: float(np.median([r["roofline"]["avg_ms"] for r in rs])) for p, rs in runs.items()}
    ratio = med["churned"] / med["contiguous"]
    return {"metric": "paging cost: decode step time over a scattered pool / over physically "
                      "consecutive blocks", "value": round(ratio, 4), "unit": "ratio",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": False, "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": WORKLOADS["paging_cost"], "global_batch": S,
                       "seq_len": 32768, "parallelism": "none (1 GPU)"},
            "step_ms_median": {p: round(v, 4) for p, v in med.items()},
            "call_ms_median": {p: round(v, 4) for p, v in call.items()},
            "step_ms_runs": {p: [r["ms_per_step"] for r in rs] for p, rs in runs.items()},
            "paging_overhead_pct": round(100 * (ratio - 1), 2),
            "page_claim": "a contiguous kernel is 1-2% faster at batch 1"}


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


def _oracle_batch_loop(batch, scale, min_seconds):
    """The oracle's decode over `batch` [(q, K, V) in fp64] on this thread, repeated until it
    has run for min_seconds; returns (sequence-steps done, their context tokens, seconds of
    oracle time)."""
    from oracle import attention as att
    busy, done, ctx = 0.0, 0, 0
    while busy < min_seconds:
        for qi, K, V in batch:
            t0 = time.perf_counter()
            att.dense_decode(qi, K, V, scale)
            busy += time.perf_counter() - t0
            done += 1
            ctx += K.shape[0]
    return done, ctx, busy


def _oracle_worker(job):
    """One process of the all-core leg: bf16 bit patterns in, the oracle at one thread."""
    bits, scale, min_seconds = job
    from threadpoolctl import threadpool_limits

    from oracle import attention as att
    batch = [tuple(att.bf16_bits_to_f64(x) for x in seq) for seq in bits]
    with threadpool_limits(limits=1):
        return _oracle_batch_loop(batch, scale, min_seconds)


def cpu_baseline(w, st, n_seqs, min_seconds, workers=16):
    """The fp64 oracle, unchanged, on the first n_seqs sequences of the batch (their K/V copied to
    the host once, outside the timing), in two legs, each in fresh interpreters (spawned
    processes: no GPU or torch thread state; in this process, after torch has run, one-thread
    BLAS measured ~40% slower):
      * all cores: min(workers, os.cpu_count()) processes, each running its share of the
        sequences on one thread for at least min_seconds; the rate is the processes' summed
        context tokens per second of their own oracle time over the batch's mean context;
      * one thread: one process running every sequence for at least min_seconds.
    A decode step produces one token per sequence, so sequence-steps per second are tokens/s."""
    import multiprocessing as mp

    import torch

    from paged_kv_cache_378_amd import workloads as wl

    n_seqs = min(n_seqs, w.num_seqs)
    q = st.vals["q"]

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    seq_bits, tokens = [], 0
    for i in range(n_seqs):
        ks, vs = wl.logical_kv(w, w.step_ids[i], st.vals)
        seq_bits.append((bits(q[i]), bits(torch.cat(ks)), bits(torch.cat(vs))))
        tokens += seq_bits[-1][1].shape[0]
    ncpu = os.cpu_count() or 1
    what = (f"the first {n_seqs} of {w.num_seqs} sequences of one decode step ({tokens} context "
            f"tokens, all {w.hq} heads), numpy fp64")
    ctx = mp.get_context("spawn")  # fresh interpreters, no GPU state
    with ctx.Pool(1) as pool:
        d1, _, b1 = pool.apply(_oracle_worker, ((seq_bits, w.scale, min_seconds),))
    one = {"value": round(d1 / b1, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
           "os_cpu_count": ncpu,
           "sample": f"{what}, 1 process of 1 thread, run {d1 // n_seqs}x ({d1} sequence-steps "
                     f"in {b1:.1f} s of oracle time; the host copy of K/V is not timed)",
           "oracle_s": round(b1, 2)}
    nproc = min(workers, ncpu, n_seqs)
    if nproc <= 1:
        return one
    jobs = [(seq_bits[k::nproc], w.scale, min_seconds) for k in range(nproc)]
    t0 = time.perf_counter()
    with ctx.Pool(nproc) as pool:
        res = pool.map(_oracle_worker, jobs)
    wall = time.perf_counter() - t0
    done = sum(d for d, _, _ in res)
    # The processes' shares differ in length mix, so their rates are summed in context tokens
    # per second and converted back at the batch's mean context (a sum of sequence rates would
    # favour shares of short sequences).
    rate = sum(c / b for _, c, b in res) / (tokens / n_seqs)
    return {"value": round(rate, 1), "unit": "tokens/s", "cores": nproc, "os_cpu_count": ncpu,
            "kind": "oracle",
            "sample": f"{what}, {nproc} processes of 1 thread each, each on every {nproc}-th "
                      f"sequence for >= {min_seconds:.0f} s ({done} sequence-steps in all; rate = the "
                      f"processes' summed context tokens per second / the batch's mean context; "
                      f"the host copy of K/V is not timed)",
            "wall_s_with_startup": round(wall, 1), "one_thread": one}


if __name__ == "__main__":
    sys.exit(main())
