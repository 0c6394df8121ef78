"""GPU: many-token cache writes (the path that takes 32 consecutive tokens of one kv-head per
workgroup and stores the values transposed from LDS) against the oracle's scatter, bit for bit,
through the C ABI."""

import numpy as np
import pytest
import torch

from oracle import cache as ocache
from oracle.block_manager import BlockManagerModel

pytestmark = pytest.mark.gpu

# (raw bits on the host, signed view torch can hold, element dtype on the device)
DT = {"bf16": (np.uint16, np.int16, torch.int16, torch.bfloat16),
      "f32": (np.uint32, np.int32, torch.int32, torch.float32)}


def to_dev(a, dtype):
    _, signed, _, tdt = DT[dtype]
    return torch.from_numpy(np.ascontiguousarray(a).view(signed)).cuda().view(tdt)


def to_bits(t, dtype):
    raw, _, tview, _ = DT[dtype]
    return t.view(tview).cpu().numpy().view(raw)


def _slots(rng, NB, B, T):
    """Distinct slots: a run across block ends from an unaligned start, scattered slots,
    skipped tokens (negative and past the pool), and a second run at an aligned start."""
    n_slots = NB * B
    perm = rng.permutation(n_slots)
    run_a = np.arange(5 * B + 3, 5 * B + 3 + 600)
    used = set(run_a.tolist())
    start_b = ((5 * B + 3 + 600) // B + 2) * B  # block-aligned, past the first run
    run_b = np.arange(start_b, start_b + 200)
    used |= set(run_b.tolist())
    scattered = [s for s in perm if s not in used][:T - 600 - 200 - 40]
    skipped = [-1] * 20 + [n_slots + 7] * 10 + [-5] * 10
    slots = np.concatenate([run_a, np.asarray(scattered), np.asarray(skipped), run_b])
    assert len(slots) == T and len(set(s for s in slots if 0 <= s < n_slots)) == T - 40
    return slots.astype(np.int32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B", [16, 64])
def test_many_token_write_is_bit_exact(gpu, dtype, D, B):
    """1,515 tokens (a partial last tile of 11): pools bit-identical to the oracle's scatter,
    every byte the slots do not name keeps its sentinel, skipped tokens write nothing."""
    from paged_kv_cache_378_amd import _lib
    print(f"[gpu] many-token cache write {dtype} D={D} B={B}", flush=True)
    raw = DT[dtype][0]
    rng = np.random.default_rng(100 + D + B)
    Hkv, T = 4, 1515
    NB = (T + 64 * B) // B + 64
    slots = _slots(rng, NB, B, T)
    bits = int(np.iinfo(raw).max)
    key = rng.integers(0, bits, size=(T, Hkv, D), dtype=raw)
    value = rng.integers(0, bits, size=(T, Hkv, D), dtype=raw)
    k_or = np.full((NB, Hkv, B, D), 0x5A5A5A5A & bits, dtype=raw)
    v_or = np.full((NB, Hkv, D, B), 0x3C3C3C3C & bits, dtype=raw)
    kc, vc = to_dev(k_or, dtype), to_dev(v_or, dtype)
    kt, vt = to_dev(key, dtype), to_dev(value, dtype)
    _lib.pa_cache_write(kt, vt, kc, vc, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    ocache.write_kv(k_or, v_or, key, value, [s if s < NB * B else -1 for s in slots], B)
    assert np.array_equal(to_bits(kc, dtype), k_or)
    assert np.array_equal(to_bits(vc, dtype), v_or)


def test_many_token_append_patches_tables(gpu):
    """pa_cache_append of 4 sequences x 300 tokens (1,200 tokens: the many-token path) leaves
    the pools and the device-resident tables equal to the oracle model's, bit for bit."""
    from paged_kv_cache_378_amd import _lib
    print("[gpu] many-token append with table patch", flush=True)
    rng = np.random.default_rng(5)
    Hkv, D, B, S, C = 8, 128, 16, 4, 300
    NB = 200
    order = rng.permutation(NB).astype(np.int32)
    model = BlockManagerModel(NB, B, order.tolist())
    bm = _lib.BlockManager(NB, B, order)
    lens0 = [17, 1, 160, 95]
    for sid, n in enumerate(lens0):
        model.add_seq(sid, n)
        bm.add_seq(sid, n)
    ids = list(range(S))
    max_blocks = (max(lens0) + C + B - 1) // B
    tables, lens = bm.block_tables(ids, max_blocks)
    td, ld = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    slots, pairs = bm.append_slots(ids, C)
    mslots, mpairs = model.append_slots(ids, C)
    assert np.array_equal(slots, np.asarray(mslots)) and len(pairs) == 0
    ld.copy_(torch.from_numpy(bm.seq_lens(ids)))
    key = rng.integers(0, 65535, size=(S * C, Hkv, D), dtype=np.uint16)
    value = rng.integers(0, 65535, size=(S * C, Hkv, D), dtype=np.uint16)
    k_or = np.full((NB, Hkv, B, D), 0x7FC1, dtype=np.uint16)
    v_or = np.full((NB, Hkv, D, B), 0x7FC1, dtype=np.uint16)
    kc, vc = to_dev(k_or, "bf16"), to_dev(v_or, "bf16")
    kt, vt = to_dev(key, "bf16"), to_dev(value, "bf16")
    _lib.pa_cache_append(kt, vt, kc, vc, torch.from_numpy(slots).cuda(), td, ld, C)
    torch.cuda.synchronize()
    ocache.write_kv(k_or, v_or, key, value, slots, B)
    mt, ml = model.block_tables(ids, max_blocks)
    assert np.array_equal(td.cpu().numpy(), np.asarray(mt))
    assert np.array_equal(to_bits(kc, "bf16"), k_or)
    assert np.array_equal(to_bits(vc, "bf16"), v_or)
