"""Decode-time append on the GPU against the oracle.

Histories start partly written; every step each (request, layer) appends one
record (the GPU writes the pinned pool with 16-byte stores, the oracle writes
its own copy of the pool) and the selection names the just-appended and
recently appended positions.  Checked bit-exactly: published slots, plans,
state, cached bytes, the host pool rows the GPU wrote, the lengths, and the
rejection of positions not yet written and of appends to a full history.
"""
import numpy as np
import pytest

import tracegen as tg
from gpu_helpers import make_pool, make_resolver

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def hs():
    import hierarchical_kv_cache_resolve_amd as m
    return m


@pytest.mark.parametrize("wgs", [0, -1], ids=["fetch_launch", "split_units"])
def test_append_then_select(hs, wgs):
    from oracle import Oracle
    L0 = 5000
    w = tg.Workload("append", 4, 2, 6000, 64, 2, 300, 600, 40, tg.LOCALITY, 0.8, seed_index=51)
    sel_base = tg.trace(w.replace(L_ctx=L0))     # every base position is below the initial length
    pool = make_pool(hs, w)
    pinned = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    pool_copy = pinned.copy()                     # the oracle's own host pool
    rr = w.region_rows()
    res = make_resolver(hs, w, pool)
    res.set_option(hs.HS_OPT_META_WGS, wgs)
    o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes)
    lengths = np.full((w.num_req, w.num_layers), L0, np.int64)
    res.set_lengths(lengths)
    o.set_lengths(lengths)
    assert np.array_equal(res.lengths(), lengths)
    rng = np.random.default_rng(5)
    dev = torch.device("cuda:0")
    out = torch.empty((w.num_req, w.k), dtype=torch.int32, device=dev)
    for t in range(w.steps):
        for l in range(w.num_layers):
            rows = rng.integers(0, 256, size=(w.num_req, w.row_bytes), dtype=np.uint8)
            res.append(l, torch.from_numpy(rows).to(dev))
            assert o.append(l, rows, pool_copy, rr).tolist() == [0] * w.num_req
            S = sel_base[t, l].copy()
            S[:, 0] = L0 + t                       # the record appended just now
            if t >= 3:
                S[:, 1] = L0 + t - 3               # one appended three steps ago
            res.resolve(l, torch.from_numpy(S).to(dev), out)
            ref = o.resolve(l, S, pool_copy, rr)
            assert np.all(ref["err"] == 0)
            got = out.cpu().numpy()
            assert np.array_equal(got, ref["slot_idx"]), f"step {t} layer {l}"
            st = res.state(l)
            assert np.array_equal(st["slot_pos"], o.slot_pos[l]) and np.array_equal(st["ts"], o.ts[l])
            assert np.array_equal(st["page_table"], o.page_table[l])
            for r in range(w.num_req):
                m = int(ref["miss_count"][r])
                assert np.array_equal(st["plan"][r, :m], ref["plan"][r, :m])
            occ = o.slot_pos[l] >= 0
            assert np.array_equal(res.cache_layer(l)[occ], o.cache[l][occ]), f"bytes step {t} layer {l}"
        # a position equal to the length (not yet written) is rejected on both sides
        if t == w.steps // 2:
            bad = sel_base[t, 0].copy()
            bad[2, 5] = L0 + t + 1
            res.resolve(0, torch.from_numpy(bad).to(dev), out)
            ref = o.resolve(0, bad, pool_copy, rr)
            assert np.array_equal(out.cpu().numpy(), ref["slot_idx"]) and np.all(ref["slot_idx"][2] == -1)
            assert res.error()[0] == hs.HS_DEV_RANGE
            res.clear_error()
    torch.cuda.synchronize()
    assert np.array_equal(res.lengths(), lengths + w.steps)
    assert np.array_equal(o.length.T, lengths + w.steps)
    for i in range(w.num_req * w.num_layers):
        a, b = rr[i] + L0, rr[i] + L0 + w.steps
        assert np.array_equal(pinned[a:b], pool_copy[a:b]), f"appended host rows of history {i}"
    # appending to a full history changes nothing and reports it
    full = np.full((w.num_req, w.num_layers), w.L_ctx, np.int64)
    res.set_lengths(full)
    before = pinned.copy()
    res.append(0, torch.zeros((w.num_req, w.row_bytes), dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    assert res.error()[0] == hs.HS_DEV_FULL
    assert np.array_equal(pinned, before) and np.array_equal(res.lengths(), full)
    with pytest.raises(hs.HisparseError):
        res.set_lengths(full + 1)
    res.close()
    pool.free()


@pytest.mark.parametrize("wgs", [0, -1], ids=["fetch_launch", "split_units"])
def test_shrink_drops_cached_tail_then_refetches(hs, wgs):
    """Lowering the lengths after records are cached: the positions cut off
    leave the cache on the GPU exactly as in the oracle (slot empty, stamp 0,
    page-table entry -1); records appended again at those positions are
    misses whose bytes are the new rows, not the old ones."""
    from oracle import Oracle
    L0, L1 = 5000, 4000
    w = tg.Workload("shrink", 3, 2, 6000, 64, 2, 300, 600, 12, tg.LOCALITY, 0.8, seed_index=53)
    base = tg.trace(w.replace(L_ctx=L0))
    pool = make_pool(hs, w)
    pinned = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    pool_copy = pinned.copy()
    rr = w.region_rows()
    res = make_resolver(hs, w, pool)
    res.set_option(hs.HS_OPT_META_WGS, wgs)
    o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes)
    lengths = np.full((w.num_req, w.num_layers), L0, np.int64)
    res.set_lengths(lengths)
    o.set_lengths(lengths)
    dev = torch.device("cuda:0")
    out = torch.empty((w.num_req, w.k), dtype=torch.int32, device=dev)
    rng = np.random.default_rng(9)

    def forced(S, first, limit):
        """S with its first entries set to `first`, every row kept distinct
        (repeats replaced by unused positions below `limit`)."""
        S = np.where(S >= limit, S % limit, S).astype(np.int32)
        S[:, :len(first)] = first
        for r in range(S.shape[0]):
            _, keep = np.unique(S[r], return_index=True)
            dup = np.setdiff1d(np.arange(S.shape[1]), keep)
            S[r, dup] = np.setdiff1d(np.arange(limit), S[r])[: dup.size]
        return S

    def step(l, S):
        res.resolve(l, torch.from_numpy(S).to(dev), out)
        ref = o.resolve(l, S, pool_copy, rr)
        assert np.all(ref["err"] == 0)
        assert np.array_equal(out.cpu().numpy(), ref["slot_idx"])
        st = res.state(l)
        for key in ("slot_pos", "ts", "clock", "page_table"):
            assert np.array_equal(st[key], getattr(o, key)[l]), key
        occ = o.slot_pos[l] >= 0
        assert np.array_equal(res.cache_layer(l)[occ], o.cache[l][occ])
        return ref

    # fill the caches; make sure positions in [L1, L0) are resident
    for t in range(4):
        for l in range(w.num_layers):
            step(l, forced(base[t, l], L1 + 100 * t + np.arange(8), L0))
    cut = {l: o.slot_pos[l] >= L1 for l in range(w.num_layers)}
    assert all(c.any() for c in cut.values())
    lengths[:] = L1
    res.set_lengths(lengths)
    o.set_lengths(lengths)
    for l in range(w.num_layers):
        st = res.state(l)
        for key in ("slot_pos", "ts", "page_table"):
            assert np.array_equal(st[key], getattr(o, key)[l]), f"after shrink: {key}"
        assert not np.any(st["slot_pos"] >= L1)
    # append new records at the cut-off positions, then select them
    for i in range(8):
        for l in range(w.num_layers):
            rows = rng.integers(0, 256, size=(w.num_req, w.row_bytes), dtype=np.uint8)
            res.append(l, torch.from_numpy(rows).to(dev))
            assert o.append(l, rows, pool_copy, rr).tolist() == [0] * w.num_req
    for l in range(w.num_layers):
        # the rewritten positions first; everything else below the old cut
        ref = step(l, forced(base[5, l], L1 + np.arange(8), L1 + 8))
        assert np.all(ref["hit_mask"][:, :8] == 0)
        for r in range(w.num_req):
            for j in range(8):
                slot = ref["slot_idx"][r, j]
                assert np.array_equal(res.cache_rows(l, r)[slot], pinned[rr[r * w.num_layers + l] + L1 + j])
    assert res.error()[0] == 0
    res.close()
    pool.free()
