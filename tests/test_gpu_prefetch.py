"""Exact layer-wise prefetch on the GPU (the shared-indexer workload's shape, reduced).

Layers of one group receive their anchor's selection every step.  With
prefetch on, the anchor's plan is replayed into the shared layers on a side
stream and their resolve only publishes.  The test checks, step by step and
bit-exactly, that prefetch-on equals prefetch-off equals the oracle (which
has no notion of prefetch and runs every layer on its own state): published
slots, hit masks, miss counts, plans, slot maps, stamps, page tables, clocks
and cached bytes.
"""
import numpy as np
import pytest

import tracegen as tg
from gpu_helpers import compare_step, executor, make_pool, make_resolver, oracle_step

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def hs():
    import hierarchical_kv_cache_resolve_amd as m
    return m


def run_step_prefetch(res, w, sel_t, out, main, side):
    """One decode step in model order: each anchor resolves, then its group's
    replay starts on the side stream, then the shared layers publish."""
    for g0 in range(0, w.num_layers, w.group):
        res.resolve(g0, sel_t[g0], out[g0], main)
        shared = list(range(g0 + 1, min(g0 + w.group, w.num_layers)))
        if shared:
            res.prefetch(g0, shared, side)
        for l in shared:
            res.resolve(l, sel_t[l], out[l], main)


SMALL = tg.PREFETCH.replace(name="prefetch_small", num_req=3, L_ctx=20000, k=512, B=1024, steps=12)
MID = tg.PREFETCH.replace(name="prefetch_mid", num_req=8, L_ctx=120000, k=2048, B=4096, steps=8, W_KV=64)


@pytest.mark.parametrize("w,copy_wgs", [(SMALL, 0), (MID, 0), (SMALL, 3)],
                         ids=["prefetch_small", "prefetch_mid", "prefetch_small_3_copy_wgs"])
def test_prefetch_equals_no_prefetch_equals_oracle(hs, w, copy_wgs):
    """copy_wgs: workgroups of the replay's copy launch (0: the default grid;
    3 makes every copying workgroup loop over many rounds of misses)."""
    from oracle import Oracle
    print(f"[prefetch] {w.name} R={w.num_req} layers={w.num_layers} group={w.group} k={w.k} B={w.B} "
          f"copy_wgs={copy_wgs}", flush=True)
    tr = tg.trace(w)
    pool = make_pool(hs, w)
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    on = make_resolver(hs, w, pool)
    on.set_option(hs.HS_OPT_PREFETCH_BLOCKS, copy_wgs)
    off = make_resolver(hs, w, pool)
    o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes, model_bytes=True)
    dev = torch.device("cuda:0")
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    sel = torch.from_numpy(tr).to(dev)
    out_on = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
    out_off = torch.empty_like(out_on)
    with executor() as ex:
        for t in range(w.steps):
            run_step_prefetch(on, w, sel[t], out_on, main, side)
            for l in range(w.num_layers):
                off.resolve(l, sel[t, l], out_off[l], main)
            refs = oracle_step(o, w, tr[t], pool_np, pool_exec=ex)
            torch.cuda.synchronize()
            got_on, got_off = out_on.cpu().numpy(), out_off.cpu().numpy()
            for l in range(w.num_layers):
                st_on, st_off = on.state(l), off.state(l)
                compare_step(got_on[l], refs[l], st_on, w, l, t)
                compare_step(got_off[l], refs[l], st_off, w, l, t)
                for key in ("slot_pos", "ts", "clock", "page_table"):
                    ref = {"slot_pos": o.slot_pos, "ts": o.ts, "clock": o.clock, "page_table": o.page_table}[key][l]
                    assert np.array_equal(st_on[key], ref), f"{key} (prefetch on) step {t} layer {l}"
                    assert np.array_equal(st_off[key], ref), f"{key} (prefetch off) step {t} layer {l}"
                occ = o.slot_pos[l] >= 0
                assert np.array_equal(on.cache_layer(l)[occ], o.cache[l][occ]), f"bytes (on) step {t} layer {l}"
                assert np.array_equal(off.cache_layer(l)[occ], o.cache[l][occ]), f"bytes (off) step {t} layer {l}"
                # shared layers publish exactly what their anchor published
                a = (l // w.group) * w.group
                assert np.array_equal(got_on[l], got_on[a])
    for r in (on, off):
        assert r.error()[0] == 0
    t_on = on.stats()
    assert t_on.hits + t_on.misses == w.steps * w.num_layers * w.num_req * w.k
    on.close()
    off.close()
    pool.free()


def test_prefetch_ordering_and_divergence_errors(hs):
    w = tg.PREFETCH.replace(name="prefetch_err", num_req=2, num_layers=4, group=4, L_ctx=5000, k=64, B=128,
                            steps=4, W_KV=8)
    tr = tg.trace(w)
    pool = make_pool(hs, w)
    res = make_resolver(hs, w, pool)
    dev = torch.device("cuda:0")
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    sel = torch.from_numpy(tr).to(dev)
    out = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
    s_main, s_side = main.cuda_stream, side.cuda_stream
    # step 0 without prefetch
    for l in range(4):
        res.resolve(l, sel[0, l], out[l], main)
    # prefetch before the anchor's resolve of this step: out of order
    assert hs.hisparse_prefetch(res.h, 0, [1, 2, 3], s_side) == hs.HS_E_ORDER
    res.resolve(0, sel[1, 0], out[0], main)
    assert hs.hisparse_prefetch(res.h, 0, [0], s_side) == hs.HS_E_INVAL       # anchor in its own group
    assert hs.hisparse_prefetch(res.h, 0, [1, 1], s_side) == hs.HS_E_INVAL    # repeated shared layer
    assert hs.hisparse_prefetch(res.h, 0, [4], s_side) == hs.HS_E_LAYER
    res.prefetch(0, [1, 2, 3], side)
    assert hs.hisparse_prefetch(res.h, 0, [1], s_side) == hs.HS_E_ORDER       # replay already pending
    for l in (1, 2, 3):
        res.resolve(l, sel[1, l], out[l], main)
    torch.cuda.synchronize()
    assert res.error()[0] == 0
    assert np.array_equal(out[1].cpu().numpy(), out[0].cpu().numpy())
    # layer 3 resolves a different selection on its own: its state diverges
    res.resolve(0, sel[2, 0], out[0], main)
    for l in (1, 2):
        res.resolve(l, sel[2, l], out[l], main)
    # same positions in reverse order: the misses take the victims in the
    # opposite order, so layer 3's slot map no longer mirrors its anchor's
    other = torch.from_numpy(np.ascontiguousarray(tr[2, 3][:, ::-1])).to(dev)
    res.resolve(3, other, out[3], main)
    res.resolve(0, sel[3, 0], out[0], main)
    res.prefetch(0, [1, 2, 3], side)
    for l in (1, 2, 3):
        res.resolve(l, sel[3, l], out[l], main)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got[1], got[0]) and np.array_equal(got[2], got[0])
    code, layer, _ = res.error()
    assert code == hs.HS_DEV_DIVERGED and layer == 3
    # whatever layer 3 published is either rejected (-1) or exact for its own state
    st3 = res.state(3)
    for r in range(w.num_req):
        row = got[3][r]
        if row[0] == -1:
            assert np.all(row == -1)
        else:
            assert np.array_equal(st3["slot_pos"][r][row], tr[3, 3, r])
    res.close()
    pool.free()


def test_shared_layer_selection_must_be_the_anchors(hs):
    """A shared layer whose selection is not the anchor's -- the same
    positions in another order, all of them resident -- is refused with
    HS_DEV_DIVERGED and publishes -1: its hit mask and stamps would otherwise
    silently be the anchor's, not its own.  The other shared layers of the
    group publish normally."""
    w = tg.PREFETCH.replace(name="prefetch_perm", num_req=2, num_layers=4, group=4, L_ctx=5000, k=64, B=128,
                            steps=3, W_KV=8)
    tr = tg.trace(w)
    pool = make_pool(hs, w)
    res = make_resolver(hs, w, pool)
    dev = torch.device("cuda:0")
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    sel = torch.from_numpy(tr).to(dev)
    out = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
    for l in range(4):
        res.resolve(l, sel[0, l], out[l], main)
    res.resolve(0, sel[1, 0], out[0], main)
    res.prefetch(0, [1, 2, 3], side)
    permuted = torch.from_numpy(np.ascontiguousarray(tr[1, 1][:, ::-1])).to(dev)
    res.resolve(1, permuted, out[1], main)
    for l in (2, 3):
        res.resolve(l, sel[1, l], out[l], main)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    code, layer, _ = res.error()
    assert code == hs.HS_DEV_DIVERGED and layer == 1
    assert np.all(got[1] == -1)
    assert np.array_equal(got[2], got[0]) and np.array_equal(got[3], got[0])
    # the same selection, in the anchor's order, publishes again
    res.clear_error()
    res.resolve(0, sel[2, 0], out[0], main)
    res.prefetch(0, [1, 2, 3], side)
    for l in (1, 2, 3):
        res.resolve(l, sel[2, l], out[l], main)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert res.error()[0] == 0
    for l in (1, 2, 3):
        assert np.array_equal(got[l], got[0])
    res.close()
    pool.free()
