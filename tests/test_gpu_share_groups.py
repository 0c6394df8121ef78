"""GPU parity of decoding with share groups (pa_decode_shared, pa_decode_step_shared).

"Taming the Tail", "Complex Memory Sharing": sequences forked from one system prompt read its
blocks from one physical copy.  With share groups a work item reads a group's common range once
for up to 16 / (Hq/Hkv) members, and each member merges that partial result with its own tokens.
Every output must match the fp64 oracle on the sequence's logical K/V, whether the groups were
computed before the step's copy-on-write or after it, at any partition length, at 4 and 8 query
heads per kv-head, and whatever malformed groups the caller passes (the plan drops or clamps
them).  Results do not depend on the physical layout, bit for bit."""

import numpy as np
import pytest
import torch

from paged_kv_cache_378_amd import workloads as wl

from parity import check, f64, oracle_decode

pytestmark = pytest.mark.gpu


def prepared(w, free_order=None):
    """State after the workload's step has been applied on the device (copy-on-write, cache
    write); returns the state, the step's tables/lengths (device) and the groups the host
    helper finds before and after the step."""
    from paged_kv_cache_378_amd import _lib
    from paged_kv_cache_378_amd.runner import PagedState
    st = PagedState(w, "cuda", poison=True, free_order=free_order)
    gm = min(4, 16 // (w.hq // w.hkv))
    before = st.bm.share_groups(w.step_ids, 4, 32)
    slots, pairs, tables, lens = st.host_step()
    slots_d, pairs_d, tables_d, lens_d = st.upload(slots, pairs, tables, lens)
    if pairs_d.numel():
        _lib.pa_copy_blocks(st.k_cache, st.v_cache, pairs_d)
    _lib.pa_cache_write(st.vals["k_step"], st.vals["v_step"], st.k_cache, st.v_cache, slots_d)
    after = st.bm.share_groups(w.step_ids, max(2, gm), 32)
    return st, tables_d, lens_d, before, after


def decode(st, tables_d, lens_d, groups, pt=0):
    from paged_kv_cache_378_amd import _lib
    w = st.w
    max_ctx = int(lens_d.max())
    ws = torch.empty(_lib.pa_decode_workspace_size(w.num_seqs, w.hq, w.head_dim, max_ctx, pt),
                     dtype=torch.uint8, device="cuda")
    out = st.new_out()
    g = None if groups is None else torch.from_numpy(np.ascontiguousarray(groups, np.int32)).cuda()
    _lib.pa_decode_shared(out, st.vals["q"], st.k_cache, st.v_cache, tables_d, lens_d, max_ctx,
                          w.scale, g, pt, ws)
    torch.cuda.synchronize()
    return out


CASES = {
    "g4_b16": lambda: wl.shared_prefix(B=16, n_seqs=24, prefix=200, n_families=6,
                                       suffix_range=(1, 300)),
    "g4_b32": lambda: wl.shared_prefix(B=32, n_seqs=24, prefix=330, n_families=6,
                                       suffix_range=(1, 300)),
    "g8_b16": lambda: wl.shared_prefix(B=16, n_seqs=20, prefix=260, n_families=5,
                                       suffix_range=(1, 200), hq=64, hkv=8),
    "g4_b64": lambda: wl.shared_prefix(B=64, n_seqs=12, prefix=700, n_families=3,
                                       suffix_range=(1, 300)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_groups_match_oracle(gpu, name):
    w = CASES[name]()
    print(f"[gpu] share groups {name}: S={w.num_seqs} Hq/Hkv={w.hq}/{w.hkv} B={w.block_size}",
          flush=True)
    st, tables_d, lens_d, before, after = prepared(w)
    assert len(before) and len(after)
    want = oracle_decode(w, st.vals)
    want = np.stack([want[i] for i in range(w.num_seqs)])
    for label, groups in (("groups before the step", before), ("groups after the step", after)):
        for pt in (0, 64, 128):
            got = decode(st, tables_d, lens_d, groups, pt)
            check(f64(got), want, "bf16", f"{name}, {label}, partition {pt or 'auto'}")
        again = decode(st, tables_d, lens_d, groups)
        assert torch.equal(again.view(torch.int16), decode(st, tables_d, lens_d, groups).view(torch.int16))
    # no groups through the same entry point: the plain decode
    check(f64(decode(st, tables_d, lens_d, None)), want, "bf16", f"{name}, no groups")


def test_groups_layout_invariance_bitwise(gpu):
    """The same groups over another physical layout of the same logical sequences give the
    same bits.  (The helper orders tables by physical block ids, so over another layout it may
    pick other, equally valid groups; the promise is about logical positions, so the first
    layout's groups hold for the second.)"""
    w = CASES["g4_b16"]()
    st, t, l, _, groups = prepared(w)
    a = decode(st, t, l, groups)
    st2, t2, l2, _, _ = prepared(w, free_order=np.arange(w.num_blocks, dtype=np.int32))
    b = decode(st2, t2, l2, groups)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_malformed_groups_are_dropped_or_clamped(gpu):
    """Sequences 0-3: a 100-token prompt and three forks of it (no appends since); 4-5
    independent sequences.  Every group list below either keeps the promise on what it
    accepts or has it dropped by the plan; the outputs must match the oracle each time."""
    from test_gpu_rollback_prefix import Mirror, decode_and_check
    print("[gpu] malformed share groups", flush=True)
    m = Mirror(NB=64, B=16, Hkv=8, D=128, dtype="bf16", seed=61)
    m.add(0, 100)
    for c in (1, 2, 3):
        m.fork(0, c)
    m.add(4, 70)
    m.add(5, 33)
    ids = [0, 1, 2, 3, 4, 5]
    bad_lists = {
        "L past every length (clamped to 100, then 96)": [[1000, 0, 1, 2, 3]],
        "a repeated member (the repeat dropped)": [[96, 0, 0, 1, -1]],
        "members out of range (dropped)": [[96, 7, 1, -5, 2]],
        "a member two groups name (the second loses it)": [[96, 0, 1, -1, -1], [96, 1, 2, 3, -1]],
        "L below 32 (group ignored)": [[20, 0, 1, 2, 3]],
        "one member left (group ignored)": [[96, 0, 9, -1, -1]],
        "L = 0 and negative L": [[0, 0, 1, -1, -1], [-64, 2, 3, -1, -1]],
        "as many groups as sequences": [[64, 0, 1, -1, -1], [64, 2, 3, -1, -1]] + [[64, -1, -1, -1, -1]] * 4,
    }
    for what, rows in bad_lists.items():
        decode_and_check(m, ids, 32, what, groups=np.array(rows, np.int32))


def test_groups_on_the_valu_kernel_are_ignored(gpu):
    """fp32 (the VALU kernel) has no group items: the groups are ignored."""
    from test_gpu_rollback_prefix import Mirror, decode_and_check
    m = Mirror(NB=64, B=16, Hkv=4, D=64, dtype="f32", seed=62)
    m.add(0, 150)
    for c in (1, 2, 3):
        m.fork(0, c)
    decode_and_check(m, [0, 1, 2, 3], 4, "fp32 with groups", groups=np.array([[144, 0, 1, 2, 3]], np.int32))


@pytest.mark.parametrize("B", [16, 32])
def test_full_size_shared_prefix_step_with_groups(gpu, B):
    """The shared-prefix batch (224 sequences) through pa_decode_step_shared with pinned slots
    and lengths and the groups found before the steps, two steps (the first one copies the
    families' shared last blocks); every sequence of the last step against the oracle."""
    from oracle import attention as att
    from paged_kv_cache_378_amd import _lib
    from paged_kv_cache_378_amd.runner import PagedState
    w = wl.shared_prefix(B=B)
    print(f"[gpu] full-size shared prefix with groups B={B}", flush=True)
    st = PagedState(w, "cuda", poison=True)
    S = w.num_seqs
    ids = np.asarray(w.step_ids, np.int64)
    groups = st.bm.share_groups(ids, 4, 32)
    groups_d = torch.from_numpy(groups).cuda()
    max_ctx = st.max_ctx + 1
    max_blocks = (max_ctx + B - 1) // B
    t0, l0 = st.bm.block_tables(ids, max_blocks)
    tables_d, lens_d = torch.from_numpy(t0).cuda(), torch.from_numpy(l0).cuda()
    ws = torch.empty(_lib.pa_decode_workspace_size(S, w.hq, w.head_dim, max_ctx, 0),
                     dtype=torch.uint8, device="cuda")
    base = {}
    for i, sid in enumerate(w.step_ids):
        ks, vs = wl.logical_kv(w, sid, st.vals)
        base[i] = (np.concatenate([f64(k) for k in ks[:-1]]), np.concatenate([f64(v) for v in vs[:-1]]))
    g = torch.Generator().manual_seed(99)
    new_k, new_v = [], []
    for step in range(2):
        if step == 0:
            kn, vn, q = st.vals["k_step"], st.vals["v_step"], st.vals["q"]
        else:
            kn = torch.randn((S, w.hkv, w.head_dim), generator=g).to(torch.bfloat16).cuda()
            vn = torch.randn((S, w.hkv, w.head_dim), generator=g).to(torch.bfloat16).cuda()
            q = torch.randn((S, w.hq, w.head_dim), generator=g).to(torch.bfloat16).cuda()
        slots, pairs = st.bm.append_slots(ids, 1)
        assert (len(pairs) > 0) == (step == 0)
        ps = torch.from_numpy(slots).pin_memory()
        pl = torch.from_numpy(st.bm.seq_lens(ids)).pin_memory()
        if len(pairs):
            _lib.pa_copy_blocks(st.k_cache, st.v_cache, torch.from_numpy(pairs).cuda())
        out = torch.empty_like(q)
        _lib.pa_decode_step_shared(out, q, kn, vn, st.k_cache, st.v_cache, ps, tables_d, lens_d,
                                   max_ctx, w.scale, groups_d, 0, ws, new_ctx_lens=pl)
        torch.cuda.synchronize()
        new_k.append(f64(kn))
        new_v.append(f64(vn))
    tables, lens = st.bm.block_tables(ids, max_blocks)
    assert np.array_equal(tables_d.cpu().numpy(), tables) and np.array_equal(lens_d.cpu().numpy(), lens)
    got, qf = f64(out), f64(q)
    for i in range(S):
        K = np.concatenate([base[i][0]] + [nk[i][None] for nk in new_k])
        V = np.concatenate([base[i][1]] + [nv[i][None] for nv in new_v])
        check(got[i], att.dense_decode(qf[i], K, V, w.scale), "bf16", f"seq {i} (n={K.shape[0]})")
