"""RESOLVE inside a HIP graph: a captured decode step replayed over many steps
equals the same steps run eagerly, bit-exactly (the step clock lives on the
device, the grid is fixed and no call allocates, synchronises or records a
memset).  Eager work and synchronisations run between the replays."""
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


@pytest.mark.parametrize("prefetch", [False, True], ids=["plain", "prefetch"])
def test_graph_replay_equals_eager(hs, prefetch):
    w = tg.PREFETCH.replace(name="graph", num_req=4, num_layers=8, group=4 if prefetch else 1, L_ctx=30000,
                            k=512, B=1024, steps=10, W_KV=64)
    tr = tg.trace(w)
    pool = make_pool(hs, w)
    eager = make_resolver(hs, w, pool)
    graphed = make_resolver(hs, w, pool)
    dev = torch.device("cuda:0")
    sel = torch.from_numpy(tr).to(dev)
    sel_buf = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
    out_buf = torch.empty_like(sel_buf)
    out_eager = torch.empty_like(sel_buf)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()

    def eager_step(res, t, out_t):
        for g0 in range(0, w.num_layers, w.group):
            res.resolve(g0, sel[t, g0], out_t[g0], main)
            shared = list(range(g0 + 1, g0 + w.group))
            if shared:
                res.prefetch(g0, shared, side)
            for l in shared:
                res.resolve(l, sel[t, l], out_t[l], main)

    # both handles first run two steps eagerly, so the capture starts with the
    # library's cross-stream events recorded outside it
    for t in range(2):
        eager_step(graphed, t, out_buf)
        eager_step(eager, t, out_eager)
    g = torch.cuda.CUDAGraph()

    def captured_step():
        cur = torch.cuda.current_stream()
        for g0 in range(0, w.num_layers, w.group):
            graphed.resolve(g0, sel_buf[g0], out_buf[g0], cur)
            shared = list(range(g0 + 1, g0 + w.group))
            if shared:
                side.wait_stream(cur)
                graphed.prefetch(g0, shared, side)
            for l in shared:
                graphed.resolve(l, sel_buf[l], out_buf[l], cur)

    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        captured_step()
    for t in range(2, w.steps):
        sel_buf.copy_(sel[t])
        g.replay()
        junk = torch.randn(1 << 20, device=dev).sum()  # unrelated eager work between replays
        eager_step(eager, t, out_eager)
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        assert np.array_equal(out_buf.cpu().numpy(), out_eager.cpu().numpy()), f"replay {t}"
        for l in range(w.num_layers):
            a, b = graphed.state(l), eager.state(l)
            for key in ("slot_pos", "ts", "clock", "page_table", "miss_count"):
                assert np.array_equal(a[key], b[key]), f"{key} replay {t} layer {l}"
            occ = b["slot_pos"] >= 0
            assert np.array_equal(graphed.cache_layer(l)[occ], eager.cache_layer(l)[occ])
    assert graphed.error()[0] == 0 and eager.error()[0] == 0
    del g
    graphed.close()
    eager.close()
    pool.free()


def test_graph_replay_of_wide_batched_launches(hs):
    """A batched launch over 40 requests x 8 layers (320 request-layers: the
    two-per-CU build, which copies its own misses, no fetch launch) captured
    once and replayed step after step equals the oracle on every replay."""
    from oracle import Oracle
    w = tg.Workload("graph_wide", 40, 8, 8192, 64, 2, 256, 512, 8, tg.LOCALITY, 0.85, seed_index=120)
    print(f"[graph] {w.name} R={w.num_req} L={w.num_layers} B={w.B} k={w.k}", flush=True)
    tr = tg.trace(w)
    pool = make_pool(hs, w)
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = make_resolver(hs, w, pool)
    o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes)
    dev = torch.device("cuda:0")
    layers = list(range(w.num_layers))
    sel = torch.from_numpy(tr).to(dev)
    sel_buf = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
    out_buf = torch.empty_like(sel_buf)

    def check(t):
        for l in layers:
            ref = o.resolve(l, tr[t, l], pool_np, w.region_rows())
            assert np.array_equal(out_buf[l].cpu().numpy(), ref["slot_idx"]), f"step {t} layer {l}"
            st = res.state(l)
            assert np.array_equal(st["slot_pos"], o.slot_pos[l]) and np.array_equal(st["ts"], o.ts[l])
            occ = o.slot_pos[l] >= 0
            assert np.array_equal(res.cache_layer(l)[occ], o.cache[l][occ]), f"cache step {t} layer {l}"

    # one eager step first, then the capture
    sel_buf.copy_(sel[0])
    res.resolve_layers(layers, [sel_buf[l] for l in layers], [out_buf[l] for l in layers])
    torch.cuda.synchronize()
    check(0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cur = torch.cuda.current_stream()
        res.resolve_layers(layers, [sel_buf[l] for l in layers], [out_buf[l] for l in layers], cur)
    for t in range(1, w.steps):
        sel_buf.copy_(sel[t])
        g.replay()
        junk = torch.randn(1 << 20, device=dev).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        check(t)
    assert res.error()[0] == 0
    del g
    res.close()
    pool.free()


def test_timing_skips_captured_launches(hs):
    """Per-launch timing left on while a step is captured: the captured
    launches are not timed (their events would never be recorded on the
    stream), the eager launches around the capture are, and reading the
    times after the replays succeeds."""
    w = tg.PREFETCH.replace(name="graph_timing", num_req=4, num_layers=4, group=1, L_ctx=30000,
                            k=512, B=1024, steps=6, W_KV=64)
    print(f"[graph] {w.name} R={w.num_req} L={w.num_layers} B={w.B} k={w.k}", flush=True)
    tr = tg.trace(w)
    pool = make_pool(hs, w)
    res = make_resolver(hs, w, pool)
    dev = torch.device("cuda:0")
    sel = torch.from_numpy(tr).to(dev)
    sel_buf = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
    out_buf = torch.empty_like(sel_buf)
    cur = torch.cuda.current_stream()
    res.set_option(hs.HS_OPT_META_WGS, 0)  # a metadata and a fetch launch per layer
    res.set_option(hs.HS_OPT_TIMING, 1)
    res.timing(clear=True)
    for l in range(w.num_layers):  # one eager step: timed
        res.resolve(l, sel[0, l], out_buf[l], cur)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c = torch.cuda.current_stream()
        for l in range(w.num_layers):
            res.resolve(l, sel_buf[l], out_buf[l], c)
    for t in (1, 2):
        sel_buf.copy_(sel[t])
        g.replay()
    torch.cuda.synchronize()
    for l in range(w.num_layers):  # one more eager step: timed
        res.resolve(l, sel[3, l], out_buf[l], cur)
    tim = res.timing(clear=True)
    assert tim.plan_launches == 2 * w.num_layers and tim.fetch_launches == 2 * w.num_layers
    assert tim.dropped == 0 and tim.plan_ms > 0 and tim.fetch_ms > 0
    assert res.error()[0] == 0
    st = res.state(0)
    assert int(st["clock"][0]) == 4  # every step, captured or not, advanced the clock
    del g
    res.close()
    pool.free()
