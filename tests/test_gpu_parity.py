"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element.

Shapes span several workgroup tiles (B up to 16384 slots, i.e. 16 slots per
lane) and ragged tails (B and k not multiples of the lane count, B not a
multiple of 4, records of 16 B to 4 KB).  Everything integer is compared
bit-exactly: slot_idx, hit mask, miss count, the plan (victim slot, evicted
and new position), slot map, stamps, page table, clocks, and the cached bytes.
"""
import numpy as np
import pytest

import tracegen as tg
from gpu_helpers import checksum_ref, compare_step, executor, make_pool, make_resolver, oracle_step

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def hs():
    import hierarchical_kv_cache_resolve_amd as m
    return m


def run_parity(hs, w, steps=None, full_state_every=1, bytes_every=1, options=None):
    from oracle import Oracle
    steps = w.steps if steps is None else steps
    print(f"[parity] {w.name} R={w.num_req} L={w.num_layers} B={w.B} k={w.k} L_ctx={w.L_ctx} "
          f"row={w.row_bytes} steps={steps}", flush=True)
    tr = tg.trace(w, steps=steps)
    pool = make_pool(hs, w)
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = make_resolver(hs, w, pool)
    for key, val in (options or {}).items():
        res.set_option(key, val)
    o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes, model_bytes=True)
    dev = torch.device("cuda:0")
    sel_d = torch.from_numpy(tr).to(dev)
    out = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
    with executor() as ex:
        for t in range(steps):
            for l in range(w.num_layers):
                res.resolve(l, sel_d[t, l], out[l])
            refs = oracle_step(o, w, tr[t], pool_np, pool_exec=ex)
            got = out.cpu().numpy()
            for l in range(w.num_layers):
                st = res.state(l, page_table=(t % full_state_every == 0))
                compare_step(got[l], refs[l], st, w, l, t)
                if t % full_state_every == 0:
                    assert np.array_equal(st["slot_pos"], o.slot_pos[l]), f"slot_pos step {t} layer {l}"
                    assert np.array_equal(st["ts"], o.ts[l]), f"ts step {t} layer {l}"
                    assert np.array_equal(st["clock"], o.clock[l]), f"clock step {t} layer {l}"
                    assert np.array_equal(st["page_table"], o.page_table[l]), f"page_table step {t} layer {l}"
                if t % bytes_every == 0:
                    # bytes of occupied slots only: an empty slot holds nothing
                    occ = o.slot_pos[l] >= 0
                    assert np.array_equal(res.cache_layer(l)[occ], o.cache[l][occ]), f"cache bytes step {t} layer {l}"
    code, _, _ = res.error()
    assert code == 0
    s = res.stats()
    assert s.hits + s.misses == steps * w.num_layers * w.num_req * w.k
    res.close()
    pool.free()
    o.close()


def test_tiny_workload_full(hs):
    run_parity(hs, tg.TINY)


@pytest.mark.parametrize("wgs", [0, 1, 3, 32, -1], ids=["fetch_launch", "g1", "g3", "g32", "auto"])
def test_units_split_over_workgroups(hs, wgs):
    """Several workgroups per (request, layer) that plan the unit alike and
    copy its misses between them (no fetch launch; the last one to finish
    writes the metadata), one workgroup with a separate fetch launch (0), and
    the choice by launch size (-1): all equal the oracle bit for bit, cached
    bytes, page tables and stamps included, over steps with and without
    misses."""
    w = wl("split_wgs", num_req=4, k=512, B=1024, L_ctx=9000, W_KV=136, steps=10, p_keep=0.9)
    run_parity(hs, w, options={hs.HS_OPT_META_WGS: wgs})
    run_parity(hs, tg.hit_only(w).replace(name="split_wgs_hits"), steps=4, options={hs.HS_OPT_META_WGS: wgs})


def test_split_option_range(hs):
    w = wl("split_opt", steps=1)
    pool = make_pool(hs, w)
    res = make_resolver(hs, w, pool)
    for bad in (-2, hs.HS_MAX_META_WGS + 1):
        with pytest.raises(hs.HisparseError):
            res.set_option(hs.HS_OPT_META_WGS, bad)
    res.set_option(hs.HS_OPT_META_WGS, hs.HS_MAX_META_WGS)
    # the prefetch copy grid: 0 (the fetch grid) .. 65536 workgroups
    for bad in (-1, 65537):
        with pytest.raises(hs.HisparseError):
            res.set_option(hs.HS_OPT_PREFETCH_BLOCKS, bad)
    for ok in (0, 1, 65536):
        res.set_option(hs.HS_OPT_PREFETCH_BLOCKS, ok)
    res.close()
    pool.free()


def wl(name, **kw):
    base = dict(name=name, num_req=3, num_layers=2, L_ctx=6000, W_KV=72, elem_bytes=2, k=700, B=1500, steps=12,
                p_keep=0.8, seed_index=31)
    base.update(kw)
    return tg.Workload(**base)


RAGGED = [
    wl("ragged_b_not_mult4", B=1499, k=701),
    wl("per1_small", B=300, k=257, W_KV=8),
    wl("per2", B=2047, k=1023),
    wl("per4_mla", B=4096, k=2048, L_ctx=40000, W_KV=576, num_req=2, num_layers=2, steps=10),
    wl("per8", B=8000, k=3000, L_ctx=60000, W_KV=24, num_req=2, steps=8),
    # the smallest k that needs more than two selections per lane, and the largest that does not
    wl("k2049_three_per_lane", B=2100, k=2049, L_ctx=30000, W_KV=8, num_req=2, steps=8),
    wl("k2048_b2049", B=2049, k=2048, L_ctx=30000, W_KV=8, num_req=2, steps=8),
    wl("per16_maxb", B=16384, k=4096, L_ctx=90000, W_KV=8, num_req=1, num_layers=1, steps=6),
    wl("b_equals_k", B=900, k=900, p_keep=0.6),
    wl("uniform_small_ctx", mode=tg.UNIFORM, L_ctx=2000, B=1200, k=500),
    wl("k1_b1", k=1, B=1, L_ctx=5, steps=20, W_KV=8),
    wl("k1_b3", k=1, B=3, L_ctx=7, steps=30, W_KV=8),
    wl("gqa_row", W_KV=2048, B=600, k=300, L_ctx=3000, steps=8),
    wl("many_requests", num_req=64, num_layers=1, B=256, k=128, L_ctx=4000, W_KV=8, steps=10),
    wl("hit_only", mode=tg.HITONLY, p_keep=1.0, steps=6),
    # a history too long for the position bitmap in LDS: the slot scan falls back to the hash
    wl("long_ctx_hash_fallback", L_ctx=1_000_000, B=300, k=150, W_KV=8, num_req=2, num_layers=1, steps=8),
    # a history length that is not a multiple of the bitmap's 128-position groups
    wl("ctx_not_mult128", L_ctx=4101, B=700, k=300, W_KV=8, steps=10),
]


@pytest.mark.parametrize("w", RAGGED, ids=[w.name for w in RAGGED])
def test_ragged_shapes(hs, w):
    run_parity(hs, w)


SCAN_SUBSET = [w for w in RAGGED if w.name in ("ragged_b_not_mult4", "per1_small", "per4_mla", "per16_maxb",
                                              "b_equals_k", "uniform_small_ctx", "k1_b3", "hit_only")]


@pytest.mark.parametrize("probe", ["page_table", "hash"])
@pytest.mark.parametrize("w", SCAN_SUBSET, ids=[w.name for w in SCAN_SUBSET])
def test_other_probes(hs, w, probe):
    """The other two ways of finding hits give the same results as the default
    (the pages' slot scan with the position bitmap, which the default takes at
    these history lengths): one page-table load per selection, and the slot
    scan with the LDS hash."""
    opt = hs.HS_PROBE_PAGE_TABLE if probe == "page_table" else hs.HS_PROBE_SLOT_SCAN_HASH
    run_parity(hs, w, options={hs.HS_OPT_PROBE: opt})


@pytest.mark.parametrize("unroll,blocks,nt", [(1, 7, 0), (2, 64, 1), (8, 4096, 0)])
def test_fetch_launch_shapes(hs, unroll, blocks, nt):
    w = wl("fetch_shape", B=1000, k=600, W_KV=200, steps=6)
    run_parity(hs, w, options={hs.HS_OPT_FETCH_UNROLL: unroll, hs.HS_OPT_FETCH_BLOCKS: blocks,
                               hs.HS_OPT_NT_LOADS: nt})


def test_gather_checksum_matches_pool_rows(hs):
    w = wl("checksum", W_KV=576, B=800, k=512, L_ctx=5000, steps=5)
    tr = tg.trace(w)
    pool = make_pool(hs, w)
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = make_resolver(hs, w, pool)
    dev = torch.device("cuda:0")
    out = torch.empty((w.num_req, w.k), dtype=torch.int32, device=dev)
    cs = torch.empty(w.num_req, dtype=torch.int64, device=dev)
    rr = w.region_rows()
    for t in range(w.steps):
        for l in range(w.num_layers):
            res.resolve(l, torch.from_numpy(tr[t, l]).to(dev), out)
            res.gather_checksum(l, out, cs)
            got = cs.cpu().numpy().view(np.uint64)
            for r in range(w.num_req):
                rows = pool_np[rr[r * w.num_layers + l] + tr[t, l, r]]
                assert int(got[r]) == checksum_ref(rows)
    res.close()
    pool.free()


@pytest.mark.parametrize("wgs", [0, -1], ids=["fetch_launch", "split_units"])
def test_rejected_requests_and_sticky_error(hs, wgs):
    from oracle import Oracle
    w = wl("errors", num_req=4, num_layers=1, B=64, k=16, L_ctx=200, W_KV=8, steps=3)
    tr = tg.trace(w)
    pool = make_pool(hs, w)
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = make_resolver(hs, w, pool)
    res.set_option(hs.HS_OPT_META_WGS, wgs)
    o = Oracle(w.num_req, 1, w.B, w.L_ctx, w.row_bytes)
    dev = torch.device("cuda:0")
    out = torch.empty((w.num_req, w.k), dtype=torch.int32, device=dev)
    for t in range(2):
        res.resolve(0, torch.from_numpy(tr[t, 0]).to(dev), out)
        o.resolve(0, tr[t, 0], pool_np, w.region_rows())
    before = res.state(0)
    bad = tr[2, 0].copy()
    bad[1, 5] = bad[1, 9]          # repeated position in request 1
    bad[3, 0] = w.L_ctx            # out of range in request 3
    res.resolve(0, torch.from_numpy(bad).to(dev), out)
    ref = o.resolve(0, bad, pool_np, w.region_rows())
    got = out.cpu().numpy()
    assert np.array_equal(got, ref["slot_idx"])
    assert np.all(got[1] == -1) and np.all(got[3] == -1)
    assert ref["err"].tolist()[1] != 0 and ref["err"].tolist()[3] != 0
    after = res.state(0)
    for r in (1, 3):
        assert np.array_equal(after["slot_pos"][r], before["slot_pos"][r])
        assert np.array_equal(after["ts"][r], before["ts"][r])
        assert np.array_equal(after["page_table"][r], before["page_table"][r])
        assert after["clock"][r] == before["clock"][r]
    assert np.array_equal(after["slot_pos"], o.slot_pos[0])
    code, layer, req = res.error()
    assert code in (hs.HS_DEV_DUP, hs.HS_DEV_RANGE) and layer == 0 and req in (1, 3)
    res.clear_error()
    assert res.error()[0] == 0
    res.close()
    pool.free()


def test_synchronous_argument_errors(hs):
    w = wl("args", num_req=2, num_layers=2, B=32, k=8, L_ctx=100, W_KV=8)
    pool = make_pool(hs, w)
    res = make_resolver(hs, w, pool)
    dev = torch.device("cuda:0")
    sel = torch.zeros((2, 40), dtype=torch.int32, device=dev)
    out = torch.empty((2, 40), dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    assert hs.hisparse_resolve(res.h, 0, sel.data_ptr(), 33, out.data_ptr(), s) == hs.HS_E_K   # k > B
    assert hs.hisparse_resolve(res.h, 0, sel.data_ptr(), 0, out.data_ptr(), s) == hs.HS_E_K    # empty
    assert hs.hisparse_resolve(res.h, 2, sel.data_ptr(), 8, out.data_ptr(), s) == hs.HS_E_LAYER
    assert hs.hisparse_resolve(res.h, -1, sel.data_ptr(), 8, out.data_ptr(), s) == hs.HS_E_LAYER
    assert hs.hisparse_resolve(res.h, 0, 0, 8, out.data_ptr(), s) == hs.HS_E_INVAL
    assert hs.hisparse_prefetch(res.h, 0, [1], s) == hs.HS_E_ORDER   # anchor not resolved yet
    # record bytes not a multiple of 16
    desc = hs.hs_host_pool(pool.ptr, w.pool_rows, w.L_ctx, None)
    with pytest.raises(hs.HisparseError) as e:
        hs.hisparse_create(2, 2, 32, 7, hs.BF16, desc)
    assert e.value.rc == hs.HS_E_ALIGN
    # a history region outside the pool
    bad_rr = np.array([0, 0, 0, w.pool_rows], dtype=np.int64)
    desc = hs.hs_host_pool(pool.ptr, w.pool_rows, w.L_ctx, bad_rr.ctypes.data)
    with pytest.raises(hs.HisparseError) as e:
        hs.hisparse_create(2, 2, 32, 8, hs.BF16, desc)
    assert e.value.rc == hs.HS_E_POOL
    # pageable memory is not a pool
    pageable = np.zeros(w.pool_rows * w.row_bytes, np.uint8)
    desc = hs.hs_host_pool(pageable.ctypes.data, w.pool_rows, w.L_ctx, None)
    with pytest.raises(hs.HisparseError) as e:
        hs.hisparse_create(2, 2, 32, 8, hs.BF16, desc)
    assert e.value.rc == hs.HS_E_POOL
    with pytest.raises(hs.HisparseError):
        hs.hisparse_create(2, 2, 0, 8, hs.BF16, hs.hs_host_pool(pool.ptr, w.pool_rows, w.L_ctx, None))
    # batched resolve: a null selection pointer, a repeated layer, lists of different lengths
    sel8, out8 = sel[:, :8].contiguous(), out[:, :8].contiguous()
    assert hs.hisparse_resolve_layers(res.h, [0, 1], [sel8.data_ptr(), 0], 8,
                                      [out8.data_ptr(), out8.data_ptr()], s) == hs.HS_E_INVAL
    assert hs.hisparse_resolve_layers(res.h, [1, 1], [sel8.data_ptr()] * 2, 8, [out8.data_ptr()] * 2,
                                      s) == hs.HS_E_INVAL
    with pytest.raises(ValueError):
        res.resolve_layers([0, 1], [sel8], [out8, out8])
    # a destroyed handle is refused, not read
    h2 = hs.hisparse_create(2, 2, 32, 8, hs.BF16, hs.hs_host_pool(pool.ptr, w.pool_rows, w.L_ctx, None))
    assert hs.hisparse_destroy(h2) == hs.HS_OK
    assert hs.hisparse_destroy(h2) == hs.HS_E_HANDLE
    assert hs.hisparse_resolve(h2, 0, sel8.data_ptr(), 8, out8.data_ptr(), s) == hs.HS_E_HANDLE
    assert hs.hisparse_hbm_bytes(h2) == 0
    assert res.hbm_bytes() == hs.hisparse_kv_bytes(2, 2, 32, 8, hs.BF16) == 2 * 2 * 32 * 16
    # metadata: per slot a position, a stamp, a plan entry and a hit-mask byte; per history a
    # page table of L_ctx entries, four 32-bit words, the 64-bit region row and four 64-bit
    # counters; the error word
    nrl = 2 * 2
    assert hs.hisparse_meta_bytes(res.h) == (nrl * 32 * (4 + 4 + 16 + 1) + nrl * w.L_ctx * 4 + nrl * (5 * 4 + 8)
                                             + nrl * 4 * 8 + 16)
    res.close()
    pool.free()


def test_reset_refills_exactly(hs):
    from oracle import Oracle
    w = wl("reset", steps=6)
    tr = tg.trace(w)
    pool = make_pool(hs, w)
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = make_resolver(hs, w, pool)
    dev = torch.device("cuda:0")
    out = torch.empty((w.num_req, w.k), dtype=torch.int32, device=dev)
    for t in range(3):
        for l in range(w.num_layers):
            res.resolve(l, torch.from_numpy(tr[t, l]).to(dev), out)
    res.reset()
    assert res.stats().resolves == 0
    o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes)
    for t in range(3, 6):
        for l in range(w.num_layers):
            res.resolve(l, torch.from_numpy(tr[t, l]).to(dev), out)
            ref = o.resolve(l, tr[t, l], pool_np, w.region_rows())
            assert np.array_equal(out.cpu().numpy(), ref["slot_idx"])
            if t == 3:
                assert np.all(ref["miss_count"] == w.k)
            occ = o.slot_pos[l] >= 0
            assert np.array_equal(res.cache_layer(l)[occ], o.cache[l][occ])
    res.close()
    pool.free()


@pytest.mark.parametrize("wgs", [0, -1], ids=["fetch_launch", "split_units"])
def test_victims_older_than_histogram_range(hs, wgs):
    """Victims whose stamps are more than 1023 apart from 2t (slots filled early
    and never touched again) take the kernel's general radix-select path; a
    hand-built trace forces it, the oracle decides."""
    from oracle import Oracle
    rng = np.random.default_rng(7)
    R, L_ctx, k, B, W_KV = 2, 1000, 8, 32, 8
    perm = [rng.permutation(L_ctx).astype(np.int32) for _ in range(R)]
    steps = []
    for t in range(4):                        # fill 32 slots at 4 different stamps
        steps.append(np.stack([p[8 * t:8 * t + 8] for p in perm]))
    for _ in range(4, 700):                   # then only step 3's positions, all hits
        steps.append(steps[3].copy())
    for t in range(700, 712):                 # bursts of new positions
        steps.append(np.stack([p[32 + 8 * (t - 700):40 + 8 * (t - 700)] for p in perm]))
    w = tg.Workload("old_victims", R, 1, L_ctx, W_KV, 2, k, B, len(steps), seed_index=41)
    pool = make_pool(hs, w)
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = make_resolver(hs, w, pool)
    res.set_option(hs.HS_OPT_META_WGS, wgs)
    scan = make_resolver(hs, w, pool)
    scan.set_option(hs.HS_OPT_PROBE, hs.HS_PROBE_PAGE_TABLE)
    hscan = make_resolver(hs, w, pool)
    hscan.set_option(hs.HS_OPT_PROBE, hs.HS_PROBE_SLOT_SCAN_HASH)
    o = Oracle(R, 1, B, L_ctx, w.row_bytes)
    dev = torch.device("cuda:0")
    out = torch.empty((R, k), dtype=torch.int32, device=dev)
    out2 = torch.empty_like(out)
    out3 = torch.empty_like(out)
    for t, S in enumerate(steps):
        Sd = torch.from_numpy(S).to(dev)
        res.resolve(0, Sd, out)
        scan.resolve(0, Sd, out2)
        hscan.resolve(0, Sd, out3)
        ref = o.resolve(0, S, pool_np, w.region_rows())
        if t >= 690 or t < 6:
            got = out.cpu().numpy()
            assert np.array_equal(got, ref["slot_idx"]), f"step {t}"
            assert np.array_equal(out2.cpu().numpy(), ref["slot_idx"]), f"page-table probe step {t}"
            assert np.array_equal(out3.cpu().numpy(), ref["slot_idx"]), f"hash slot-scan step {t}"
            st = res.state(0)
            assert np.array_equal(st["slot_pos"], o.slot_pos[0]) and np.array_equal(st["ts"], o.ts[0]), f"step {t}"
            m = int(ref["miss_count"][0])
            assert np.array_equal(st["plan"][0, :m], ref["plan"][0, :m]), f"plan step {t}"
    assert res.error()[0] == 0 and scan.error()[0] == 0 and hscan.error()[0] == 0
    res.close()
    scan.close()
    hscan.close()
    pool.free()


BATCHED_SHAPES = [
    # 512 units: one per workgroup of the two-per-CU build
    tg.Workload("batched_wide", 64, 8, 8192, 8, 2, 256, 512, 6, tg.LOCALITY, 0.85, seed_index=95),
    # more units than the chip keeps resident at once (two rounds of workgroups)
    tg.Workload("batched_2x", 64, 16, 8192, 8, 2, 256, 512, 5, tg.LOCALITY, 0.85, seed_index=98),
    # 600 units at B = 4096, k = 2048 (a ragged second round)
    tg.Workload("batched_ragged_b4096", 40, 15, 16384, 8, 2, 2048, 4096, 4, tg.LOCALITY, 0.87, seed_index=99),
]


@pytest.mark.parametrize("w", BATCHED_SHAPES, ids=[w.name for w in BATCHED_SHAPES])
@pytest.mark.parametrize("probe", ["page_table", "bitmap", "hash"])
def test_batched_launch_over_many_units(hs, probe, w):
    """One launch over 512 or more (request, layer) units (the build held to
    two workgroups per CU, which copies its own misses) against the oracle,
    with misses and all-hit steps, with each probe."""
    from oracle import Oracle
    print(f"[parity] {w.name} R={w.num_req} L={w.num_layers} B={w.B} k={w.k} probe={probe}", flush=True)
    tr = tg.trace(w)
    tr[3] = tr[2]                         # an all-hit step
    pool = make_pool(hs, w)
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = make_resolver(hs, w, pool)
    res.set_option(hs.HS_OPT_PROBE, {"page_table": hs.HS_PROBE_PAGE_TABLE, "bitmap": hs.HS_PROBE_SLOT_SCAN,
                                     "hash": hs.HS_PROBE_SLOT_SCAN_HASH}[probe])
    o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes)
    dev = torch.device("cuda:0")
    layers = list(range(w.num_layers))
    sel = torch.from_numpy(tr).to(dev)
    out = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
    for t in range(w.steps):
        res.resolve_layers(layers, [sel[t, l] for l in layers], [out[l] for l in layers])
        torch.cuda.synchronize()
        for l in layers:
            ref = o.resolve(l, tr[t, l], pool_np, w.region_rows())
            assert np.array_equal(out[l].cpu().numpy(), ref["slot_idx"]), f"step {t} layer {l}"
        st = res.state(w.num_layers - 1)
        assert np.array_equal(st["ts"], o.ts[w.num_layers - 1])
        assert np.array_equal(st["slot_pos"], o.slot_pos[w.num_layers - 1])
        for l in layers:
            # the wide launch copies its own misses: bytes of occupied slots
            occ = o.slot_pos[l] >= 0
            assert np.array_equal(res.cache_layer(l)[occ], o.cache[l][occ]), f"cache bytes step {t} layer {l}"
    assert res.error()[0] == 0
    res.close()
    pool.free()


WIDE_SHAPES = [
    tg.Workload("wide_rows", 40, 8, 2048, 576, 2, 256, 512, 5, tg.LOCALITY, 0.8, seed_index=96),
    # B not a multiple of 4 (scalar slot runs), one slot a lane, ragged history length
    tg.Workload("wide_ragged", 40, 8, 2001, 72, 2, 150, 301, 5, tg.LOCALITY, 0.8, seed_index=97),
]


@pytest.mark.parametrize("w", WIDE_SHAPES, ids=[w.name for w in WIDE_SHAPES])
def test_wide_launch_copies_multi_piece_rows(hs, w):
    """Wide launches (40 requests x 8 layers): the metadata kernel's own copy
    moves every piece of each missed record, bytes checked against the
    oracle's cache model on every step.  On step 2 two request-layers are
    rejected (a repeated position, a position past the history); they copy
    nothing and keep their state, the others resolve as usual."""
    from oracle import Oracle
    print(f"[parity] {w.name} R={w.num_req} L={w.num_layers} B={w.B} k={w.k} row={w.row_bytes}", flush=True)
    tr = tg.trace(w)
    pool = make_pool(hs, w)
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = make_resolver(hs, w, pool)
    o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes)
    dev = torch.device("cuda:0")
    layers = list(range(w.num_layers))
    out = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
    tr = tr.copy()
    tr[2, 3, 7, 5] = tr[2, 3, 7, 9]        # layer 3, request 7: repeated position
    tr[2, 6, 30, 0] = w.L_ctx              # layer 6, request 30: outside the history
    sel = torch.from_numpy(tr).to(dev)
    for t in range(w.steps):
        res.resolve_layers(layers, [sel[t, l] for l in layers], [out[l] for l in layers])
        torch.cuda.synchronize()
        for l in layers:
            ref = o.resolve(l, tr[t, l], pool_np, w.region_rows())
            assert np.array_equal(out[l].cpu().numpy(), ref["slot_idx"]), f"step {t} layer {l}"
            occ = o.slot_pos[l] >= 0
            assert np.array_equal(res.cache_layer(l)[occ], o.cache[l][occ]), f"cache bytes step {t} layer {l}"
            st = res.state(l)
            assert np.array_equal(st["slot_pos"], o.slot_pos[l]) and np.array_equal(st["ts"], o.ts[l])
        if t == 2:
            assert res.error()[0] in (hs.HS_DEV_DUP, hs.HS_DEV_RANGE)
            res.clear_error()
    assert res.error()[0] == 0
    res.close()
    pool.free()


@pytest.mark.parametrize("wgs", [0, -1], ids=["fetch_launch", "split_units"])
def test_instrumentation_changes_nothing(hs, wgs):
    """Per-launch timing, phase stamps and roctx ranges on: results still
    equal the oracle bit for bit, every launch is counted (no fetch launch
    when units copy their own misses), and each request-layer's stamps (taken
    by the first wave of its lead workgroup, in program order) never go
    backwards."""
    from oracle import Oracle
    w = wl("instrumented", num_req=4, num_layers=2, B=1024, k=512, L_ctx=20000, W_KV=8, steps=6)
    tr = tg.trace(w)
    pool = make_pool(hs, w)
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = make_resolver(hs, w, pool)
    res.set_option(hs.HS_OPT_TIMING, 1)
    res.set_option(hs.HS_OPT_PHASE_TRACE, 1)
    res.set_option(hs.HS_OPT_MARKERS, 1)   # the image ships the profiler's marker library
    res.set_option(hs.HS_OPT_META_WGS, wgs)
    o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes)
    dev = torch.device("cuda:0")
    sel = torch.from_numpy(tr).to(dev)
    out = torch.empty((w.num_req, w.k), dtype=torch.int32, device=dev)
    # the bitmap kernel's stamp slots in program order: a split unit looks its
    # selections up (7, 8) before it finds the victim threshold (4, 5)
    order = [0, 1, 2, 3, 4, 5, 7, 8, 6, 9, 10] if wgs == 0 else [0, 1, 2, 3, 7, 8, 4, 5, 6, 9, 10]
    for t in range(w.steps):
        for l in range(w.num_layers):
            res.resolve(l, sel[t, l], out)
            ref = o.resolve(l, tr[t, l], pool_np, w.region_rows())
            assert np.array_equal(out.cpu().numpy(), ref["slot_idx"]), f"step {t} layer {l}"
            stamps, ns = hs.hisparse_phase_trace(res.h, l, w.num_req)
            assert ns > 0
            for r in range(w.num_req):
                seq = [int(stamps[r, i]) for i in order if stamps[r, i] != 0]
                assert stamps[r, 0] != 0 and stamps[r, 10] != 0
                assert seq == sorted(seq), f"stamps out of order, step {t} layer {l} request {r}"
    tim = res.timing(clear=True)
    assert tim.plan_launches == w.steps * w.num_layers
    assert tim.fetch_launches == (w.steps * w.num_layers if wgs == 0 else 0)
    assert tim.dropped == 0 and tim.plan_ms > 0 and (tim.fetch_ms > 0) == (wgs == 0)
    st = res.state(w.num_layers - 1)
    assert np.array_equal(st["slot_pos"], o.slot_pos[w.num_layers - 1])
    assert res.error()[0] == 0
    res.set_option(hs.HS_OPT_PHASE_TRACE, 0)
    res.set_option(hs.HS_OPT_TIMING, 0)
    res.set_option(hs.HS_OPT_MARKERS, 0)
    res.close()
    pool.free()


def test_fine_grained_pool(hs):
    """A pool in fine-grained (coherent) pinned memory gives the same slots and
    the same cached bytes as the oracle (the default pool is coarse-grained)."""
    from oracle import Oracle
    w = wl("coherent_pool", num_req=3, num_layers=2, B=600, k=300, L_ctx=5000, W_KV=72, steps=6)
    tr = tg.trace(w)
    pool = make_pool(hs, w, coherent=True)
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = make_resolver(hs, w, pool)
    o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes)
    dev = torch.device("cuda:0")
    sel = torch.from_numpy(tr).to(dev)
    out = torch.empty((w.num_req, w.k), dtype=torch.int32, device=dev)
    for t in range(w.steps):
        for l in range(w.num_layers):
            res.resolve(l, sel[t, l], out)
            ref = o.resolve(l, tr[t, l], pool_np, w.region_rows())
            assert np.array_equal(out.cpu().numpy(), ref["slot_idx"]), f"step {t} layer {l}"
            occ = o.slot_pos[l] >= 0
            assert np.array_equal(res.cache_layer(l)[occ], o.cache[l][occ]), f"cache step {t} layer {l}"
    assert res.error()[0] == 0
    res.close()
    pool.free()


@pytest.mark.parametrize("dtype,elem", [("FP8", 1), ("FP16", 2), ("FP32", 4)])
def test_other_element_types(hs, dtype, elem):
    """The element type only sets the record size (bytes are copied verbatim):
    64-byte records of fp8, fp16 and fp32 elements resolve like bf16 ones,
    slots and cached bytes equal to the oracle's, footprint identity exact."""
    from oracle import Oracle
    W_KV = 64 // elem
    w = tg.Workload(f"elem_{dtype}", 3, 2, 4000, W_KV, elem, 200, 400, 5, tg.LOCALITY, 0.8, seed_index=130 + elem)
    assert w.row_bytes == 64
    tr = tg.trace(w)
    pool = hs.HostPool.allocate(w.pool_rows * w.row_bytes)
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    pool_np[:] = np.random.default_rng(elem).integers(0, 256, pool_np.shape, dtype=np.uint8)
    res = hs.Resolver(w.num_req, w.num_layers, w.B, W_KV, getattr(hs, dtype), pool, w.L_ctx, w.pool_rows,
                      region_row=w.region_rows())
    assert res.hbm_bytes() == hs.hisparse_kv_bytes(w.num_req, w.num_layers, w.B, W_KV, getattr(hs, dtype)) \
        == w.num_req * w.num_layers * w.B * 64
    o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes)
    dev = torch.device("cuda:0")
    sel = torch.from_numpy(tr).to(dev)
    out = torch.empty((w.num_req, w.k), dtype=torch.int32, device=dev)
    for t in range(w.steps):
        for l in range(w.num_layers):
            res.resolve(l, sel[t, l], out)
            ref = o.resolve(l, tr[t, l], pool_np, w.region_rows())
            assert np.array_equal(out.cpu().numpy(), ref["slot_idx"]), f"step {t} layer {l}"
            occ = o.slot_pos[l] >= 0
            assert np.array_equal(res.cache_layer(l)[occ], o.cache[l][occ]), f"cache step {t} layer {l}"
    assert res.error()[0] == 0
    res.close()
    pool.free()
