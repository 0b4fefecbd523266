"""Parity at the five workloads' full sizes, in the launch configuration the benchmark uses.

Every step of every layer: published slots, hit masks, miss counts, plans
(victim slot, evicted and new position), slot maps, stamps and clocks are
compared element by element with the oracle (run in parallel threads, one
per layer; each layer's state is independent).  Page tables are compared in
full on the first, a middle and the last step.  Record bytes are checked
without copying whole caches every step: the consumer stand-in's checksum of
the k published records is compared with the same reduction over the host
pool's rows for sampled (request, layer) pairs every step, and the whole
cache of sampled layers is compared with the pool rows its slot map names on
sampled steps (exactness: a cached slot holds exactly the host row of its
position).  The GQA-record workload's 512 GiB logical pool exceeds the host,
so its histories alias onto a 64 GiB physical pool (regions repeat modulo the
physical size); both sides use the same map.
"""
import numpy as np
import pytest

import tracegen as tg
from gpu_helpers import checksum_ref, executor, make_pool, make_resolver, oracle_step

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def hs():
    import hierarchical_kv_cache_resolve_amd as m
    return m


def full_parity(hs, w, prefetch=False, samples_per_step=2, seed=0):
    from oracle import Oracle
    print(f"[full] {w.name}: R={w.num_req} layers={w.num_layers} L_ctx={w.L_ctx} k={w.k} B={w.B} "
          f"row={w.row_bytes} steps={w.steps} pool={w.pool_rows * w.row_bytes / 2**30:.1f} GiB "
          f"prefetch={prefetch}", flush=True)
    rng = np.random.default_rng(seed)
    tr = tg.trace(w)
    pool = make_pool(hs, w)
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    rr = w.region_rows()
    res = make_resolver(hs, w, pool)
    o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes, model_bytes=False)
    dev = torch.device("cuda:0")
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    sel = torch.from_numpy(tr).to(dev)
    out = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
    cs = torch.empty((w.num_layers, w.num_req), dtype=torch.int64, device=dev)
    full_pt_steps = {0, w.steps // 2, w.steps - 1}
    bytes_steps = {0, w.steps // 3, w.steps - 1}
    jk = np.arange(w.k)[None, :]
    with executor() as ex:
        for t in range(w.steps):
            if prefetch:
                for g0 in range(0, w.num_layers, w.group):
                    res.resolve(g0, sel[t, g0], out[g0], main)
                    shared = list(range(g0 + 1, min(g0 + w.group, w.num_layers)))
                    res.prefetch(g0, shared, side)
                    for l in shared:
                        res.resolve(l, sel[t, l], out[l], main)
            else:
                for l in range(w.num_layers):
                    res.resolve(l, sel[t, l], out[l], main)
            for l in range(w.num_layers):
                res.gather_checksum(l, out[l], cs[l], main)
            refs = oracle_step(o, w, tr[t], None, pool_arg=False, pool_exec=ex)
            got = out.cpu().numpy()
            got_cs = cs.cpu().numpy().view(np.uint64)
            for l in range(w.num_layers):
                ref = refs[l]
                assert np.all(ref["err"] == 0)
                assert np.array_equal(got[l], ref["slot_idx"]), f"slot_idx step {t} layer {l}"
                st = res.state(l, page_table=(t in full_pt_steps))
                assert np.array_equal(st["hit_mask"][:, :w.k], ref["hit_mask"]), f"hit_mask step {t} layer {l}"
                assert np.array_equal(st["miss_count"], ref["miss_count"]), f"miss_count step {t} layer {l}"
                mk = jk < ref["miss_count"][:, None]
                assert np.array_equal(st["plan"][:, :w.k][mk], ref["plan"][mk]), f"plan step {t} layer {l}"
                assert np.array_equal(st["slot_pos"], o.slot_pos[l]), f"slot_pos step {t} layer {l}"
                assert np.array_equal(st["ts"], o.ts[l]), f"ts step {t} layer {l}"
                assert np.array_equal(st["clock"], o.clock[l]), f"clock step {t} layer {l}"
                if t in full_pt_steps:
                    assert np.array_equal(st["page_table"], o.page_table[l]), f"page_table step {t} layer {l}"
            # bytes: consumer checksum of sampled (request, layer) pairs
            for _ in range(samples_per_step):
                l = int(rng.integers(w.num_layers))
                r = int(rng.integers(w.num_req))
                rows = pool_np[rr[r * w.num_layers + l] + tr[t, l, r]]
                assert int(got_cs[l, r]) == checksum_ref(rows), f"checksum step {t} layer {l} request {r}"
            if t in bytes_steps:
                l = int(rng.integers(w.num_layers))
                cache = res.cache_layer(l)
                for r in range(w.num_req):
                    spos = o.slot_pos[l, r]
                    occ = np.nonzero(spos >= 0)[0]
                    assert np.array_equal(cache[r][occ], pool_np[rr[r * w.num_layers + l] + spos[occ]]), \
                        f"cache bytes step {t} layer {l} request {r}"
    assert res.error()[0] == 0
    st = res.stats()
    assert st.hits + st.misses == w.steps * w.num_layers * w.num_req * w.k
    miss_rate = st.misses / (st.hits + st.misses)
    print(f"[full] {w.name}: miss rate {miss_rate:.4f}", flush=True)
    res.close()
    o.close()
    pool.free()
    return miss_rate


@pytest.mark.timeout(900)
def test_full_tiny(hs):
    full_parity(hs, tg.TINY)


@pytest.mark.timeout(900)
def test_full_mla_latent(hs):
    full_parity(hs, tg.MLA)


@pytest.mark.timeout(900)
def test_full_no_locality(hs):
    w = tg.NOLOCALITY
    rate = full_parity(hs, w)
    # uniform selection with B = k: after the all-miss step 0 the hit count is
    # Hypergeometric(L_ctx, B, k), so the miss rate is 1 - B/L_ctx in expectation
    N, K, n = w.L_ctx, w.B, w.k
    samples = (w.steps - 1) * w.num_req * w.num_layers
    var = n * (K / N) * (1 - K / N) * (N - n) / (N - 1)
    expect = (1 + (w.steps - 1) * (1 - K / N)) / w.steps
    sigma = np.sqrt(var / samples) / n * (w.steps - 1) / w.steps
    assert abs(rate - expect) < 6 * sigma


@pytest.mark.timeout(900)
def test_full_gqa_record(hs):
    full_parity(hs, tg.GQA, samples_per_step=1)


@pytest.mark.timeout(900)
def test_full_shared_prefetch(hs):
    full_parity(hs, tg.PREFETCH, prefetch=True)


@pytest.mark.timeout(900)
def test_full_page_records(hs):
    """Block-granular records: 18 KB pages of 16 tokens selected by page index."""
    full_parity(hs, tg.PAGES)
