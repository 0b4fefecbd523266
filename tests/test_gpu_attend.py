"""The consumer on the GPU against the float64 oracle: sparse MLA decode
attention over the records RESOLVE published.

End to end: selections go through RESOLVE (which fetches misses from the
pinned pool), the attention kernel reads the published slots of the HBM
cache, and the oracle computes attention over the same positions read from
the pool itself.  Tolerance: the per-element bound of
``oracle.attention.error_bound`` on the output; on the log-sum-exp the fp32
score error bound ``scale * max_j sum_d |q_d rec_j[d]| * 576 * 2^-24`` plus
``k * 2^-24`` for the sum and 1e-6.
"""
import numpy as np
import pytest

import tracegen as tg
from gpu_helpers import make_pool, make_resolver

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

D_QK, D_V = 576, 512


@pytest.fixture(scope="module")
def hs():
    import hierarchical_kv_cache_resolve_amd as m
    return m


_live = []


def keep(obj):
    """Release at the end of the test (resolvers before the pools they use)."""
    _live.append(obj)
    return obj


@pytest.fixture(autouse=True)
def _release_after_test():
    yield
    while _live:
        obj = _live.pop()
        if hasattr(obj, "close"):
            obj.close()
        else:
            obj.free()


def rand_bits(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    u = x.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def records(w, pool_np, layer, sel):
    """Pool rows of the selected positions as bf16 bits [R][k][576]."""
    rr = w.region_rows()
    R, k = sel.shape
    rows = np.empty((R, k, w.row_bytes), np.uint8)
    for r in range(R):
        rows[r] = pool_np[rr[r * w.num_layers + layer] + sel[r]]
    return rows.view(np.uint16)


def check(hs, q, rec, scale, out, lse, valid=None):
    from oracle.attention import bf16_to_f64, error_bound, mla_decode
    R = q.shape[0]
    got_o = out.cpu().numpy().astype(np.float64)
    got_l = lse.cpu().numpy().astype(np.float64)
    for r in range(R):
        rr = rec[r:r + 1] if valid is None else rec[r:r + 1, valid[r]]
        if rr.shape[1] == 0:
            assert np.all(got_o[r] == 0.0) and np.all(np.isneginf(got_l[r])), f"request {r} has no records"
            continue
        ref_o, ref_l = mla_decode(q[r:r + 1], rr, scale)
        bound = error_bound(q[r:r + 1], rr, scale)
        err = np.abs(got_o[r:r + 1] - ref_o)
        assert np.all(err <= bound), f"request {r}: out error {err.max():.3g} over bound at {np.argmax(err - bound)}"
        qa, ra = np.abs(bf16_to_f64(q[r])), np.abs(bf16_to_f64(rr[0]))
        lb = scale * (qa @ ra.T).max() * D_QK * 2.0 ** -24 + rr.shape[1] * 2.0 ** -24 + 1e-6
        lerr = np.abs(got_l[r] - ref_l[0])
        assert np.all(lerr <= lb), f"request {r}: lse error {lerr.max():.3g} > {lb:.3g}"


def run_attend(hs, res, layer, q_np, slot_idx, scale, dev):
    R, H, _ = q_np.shape
    q = torch.from_numpy(q_np.view(np.int16)).to(dev)
    out = torch.full((R, H, D_V), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device=dev)
    res.attend_mla(layer, q, slot_idx, scale, out, lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("heads_per_wg", [0, 32, 64])
def test_attend_after_resolve_ragged(hs, heads_per_wg):
    """k from 1 to 1000 (ragged sub-chunks and chunks), 64 to 1024 heads (192
    and 320: three and five groups of 64, grids that do not divide into the
    eight XCDs), two scales, with the head grouping chosen by shape and forced
    to 32 and to 64 heads a workgroup."""
    w = tg.Workload("attend", 3, 2, 8192, 576, 2, 1000, 1024, 11, tg.LOCALITY, 0.8, seed_index=61)
    sel_all = tg.trace(w)
    pool = keep(make_pool(hs, w))
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = keep(make_resolver(hs, w, pool))
    res.set_option(hs.HS_OPT_ATTN_HEADS, heads_per_wg)
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(7)
    cases = [(1, 64, 0.0417), (37, 128, 0.25), (64, 64, 0.0417), (65, 128, 0.0417), (200, 64, 0.25),
             (513, 64, 0.25), (777, 128, 0.0417), (1000, 128, 0.0417), (150, 192, 0.0417), (333, 320, 0.25),
             (97, 1024, 0.0417)]
    for t, (k, H, scale) in enumerate(cases):
        for l in range(w.num_layers):
            sel = np.ascontiguousarray(sel_all[t, l, :, :k])
            slot_idx = torch.empty((w.num_req, k), dtype=torch.int32, device=dev)
            res.resolve(l, torch.from_numpy(sel).to(dev), slot_idx)
            res.check_error()
            q_np = rand_bits(rng, (w.num_req, H, D_QK))
            print(f"attend k={k} H={H} scale={scale} layer={l} heads/wg={heads_per_wg}", flush=True)
            out, lse = run_attend(hs, res, l, q_np, slot_idx, scale, dev)
            check(hs, q_np, records(w, pool_np, l, sel), scale, out, lse)


def test_attend_skips_unpublished_slots(hs):
    """Slots of -1 are left out; a request with none gives zeros and -inf."""
    w = tg.Workload("attend_holes", 4, 1, 4096, 576, 2, 300, 512, 1, tg.UNIFORM, 0.0, seed_index=62)
    sel = np.ascontiguousarray(tg.trace(w)[0, 0])
    pool = keep(make_pool(hs, w))
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = keep(make_resolver(hs, w, pool))
    dev = torch.device("cuda:0")
    slot_idx = torch.empty((w.num_req, w.k), dtype=torch.int32, device=dev)
    res.resolve(0, torch.from_numpy(sel).to(dev), slot_idx)
    res.check_error()
    rng = np.random.default_rng(8)
    valid = rng.random((w.num_req, w.k)) < 0.7
    valid[1, :] = False            # a request with nothing published
    valid[2, :] = False
    valid[2, 299] = True           # a single record, last of a ragged sub-chunk
    s = slot_idx.cpu().numpy()
    s[~valid] = -1
    slot_idx = torch.from_numpy(s).to(dev)
    q_np = rand_bits(rng, (w.num_req, 64, D_QK))
    out, lse = run_attend(hs, res, 0, q_np, slot_idx, 0.1, dev)
    check(hs, q_np, records(w, pool_np, 0, sel), 0.1, out, lse, valid=valid)


def test_attend_rejected_request(hs):
    """A request rejected by RESOLVE (duplicate position) publishes -1: its attention is empty."""
    w = tg.Workload("attend_rej", 2, 1, 4096, 576, 2, 128, 256, 1, tg.UNIFORM, 0.0, seed_index=63)
    sel = np.ascontiguousarray(tg.trace(w)[0, 0])
    sel[1, 5] = sel[1, 9]
    pool = keep(make_pool(hs, w))
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = keep(make_resolver(hs, w, pool))
    dev = torch.device("cuda:0")
    slot_idx = torch.empty((w.num_req, w.k), dtype=torch.int32, device=dev)
    res.resolve(0, torch.from_numpy(sel).to(dev), slot_idx)
    torch.cuda.synchronize()
    assert np.all(slot_idx.cpu().numpy()[1] == -1)
    res.clear_error()
    rng = np.random.default_rng(9)
    q_np = rand_bits(rng, (w.num_req, 64, D_QK))
    out, lse = run_attend(hs, res, 0, q_np, slot_idx, 0.05, dev)
    valid = np.ones((2, w.k), bool)
    valid[1] = False
    check(hs, q_np, records(w, pool_np, 0, sel), 0.05, out, lse, valid=valid)


def test_attend_rejects_bad_arguments(hs):
    w = tg.Workload("attend_args", 1, 1, 1024, 64, 2, 16, 32, 1, seed_index=64)
    pool = keep(make_pool(hs, w))
    res = keep(make_resolver(hs, w, pool))
    dev = torch.device("cuda:0")
    q = torch.zeros((1, 64, D_QK), dtype=torch.int16, device=dev)
    idx = torch.zeros((1, 16), dtype=torch.int32, device=dev)
    out = torch.zeros((1, 64, D_V), dtype=torch.float32, device=dev)
    with pytest.raises(hs.HisparseError):
        res.attend_mla(0, q, idx, 0.1, out)     # records of 64 elements are not MLA records
    w2 = tg.Workload("attend_args2", 1, 1, 1024, 576, 2, 16, 32, 1, seed_index=65)
    pool2 = keep(make_pool(hs, w2))
    res2 = keep(make_resolver(hs, w2, pool2))
    with pytest.raises(hs.HisparseError):
        res2.attend_mla(0, q[:, :32].contiguous(), idx, 0.1, out)   # heads not a multiple of 64
    with pytest.raises(hs.HisparseError):
        res2.attend_mla(1, q, idx, 0.1, out)           # no such layer
    q_many = torch.zeros((1, 1088, D_QK), dtype=torch.int16, device=dev)
    out_many = torch.zeros((1, 1088, D_V), dtype=torch.float32, device=dev)
    with pytest.raises(hs.HisparseError):
        res2.attend_mla(0, q_many, idx, 0.1, out_many)  # more heads than HS_MAX_HEADS
    with pytest.raises(hs.HisparseError):
        res2.set_option(hs.HS_OPT_ATTN_HEADS, 48)       # 32 or 64 heads a workgroup, or 0
    # queries and outputs move 16 bytes a lane: views 2 and 4 bytes off alignment are refused
    qbuf = torch.zeros(64 * D_QK + 8, dtype=torch.int16, device=dev)
    obuf = torch.zeros(64 * D_V + 4, dtype=torch.float32, device=dev)
    q_off = qbuf[1:1 + 64 * D_QK].view(1, 64, D_QK)
    out_off = obuf[1:1 + 64 * D_V].view(1, 64, D_V)
    assert q_off.data_ptr() % 16 == 2 and out_off.data_ptr() % 16 == 4
    with pytest.raises(hs.HisparseError):
        res2.attend_mla(0, q_off, idx, 0.1, out)
    with pytest.raises(hs.HisparseError):
        res2.attend_mla(0, q, idx, 0.1, out_off)
    assert hs.hisparse_attend_mla_noalloc(res2.h, 0, q_off.data_ptr(), 64, idx.data_ptr(), 16, 0.1, out.data_ptr(),
                                          0, 0) == hs.HS_E_INVAL


@pytest.mark.parametrize("heads_per_wg", [0, 32])
def test_attend_full_size(hs, heads_per_wg):
    """16 requests, k = 2048 of a 4096-slot cache, 128 heads: the decode shape
    of the MLA workload (64 heads a workgroup by shape; also forced to 32)."""
    w = tg.Workload("attend_full", 16, 1, 32768, 576, 2, 2048, 4096, 3, tg.LOCALITY, 0.87, seed_index=66)
    sel_all = tg.trace(w)
    pool = keep(make_pool(hs, w))
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = keep(make_resolver(hs, w, pool))
    res.set_option(hs.HS_OPT_ATTN_HEADS, heads_per_wg)
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(10)
    slot_idx = torch.empty((w.num_req, w.k), dtype=torch.int32, device=dev)
    for t in range(w.steps):
        sel = np.ascontiguousarray(sel_all[t, 0])
        res.resolve(0, torch.from_numpy(sel).to(dev), slot_idx)
        res.check_error()
    q_np = rand_bits(rng, (w.num_req, 128, D_QK))
    print("attend full size", flush=True)
    out, lse = run_attend(hs, res, 0, q_np, slot_idx, 1.0 / 24.0, dev)
    check(hs, q_np, records(w, pool_np, 0, sel), 1.0 / 24.0, out, lse)


@pytest.mark.parametrize("heads_per_wg", [0, 32])
def test_attend_large_batch_single_chunk(hs, heads_per_wg):
    """128 requests x 128 heads, k = 640: enough workgroups without splitting
    the records, so each workgroup's outputs are final and go out in fp32 from
    the partial kernel with no combine launch (also with 32 heads a
    workgroup); every request checked against the float64 oracle."""
    w = tg.Workload("attend_big", 128, 1, 8192, 576, 2, 640, 1024, 2, tg.LOCALITY, 0.87, seed_index=67)
    sel_all = tg.trace(w)
    pool = keep(make_pool(hs, w))
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = keep(make_resolver(hs, w, pool))
    res.set_option(hs.HS_OPT_ATTN_HEADS, heads_per_wg)
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(12)
    slot_idx = torch.empty((w.num_req, w.k), dtype=torch.int32, device=dev)
    for t in range(w.steps):
        sel = np.ascontiguousarray(sel_all[t, 0])
        res.resolve(0, torch.from_numpy(sel).to(dev), slot_idx)
        res.check_error()
    q_np = rand_bits(rng, (w.num_req, 128, D_QK))
    print(f"attend large batch heads/wg={heads_per_wg}", flush=True)
    out, lse = run_attend(hs, res, 0, q_np, slot_idx, 1.0 / 24.0, dev)
    check(hs, q_np, records(w, pool_np, 0, sel), 1.0 / 24.0, out, lse)


@pytest.mark.parametrize("heads_per_wg", [0, 32])
def test_attend_full_size_with_holes(hs, heads_per_wg):
    """The decode shape with slots left out: whole leading sub-chunks of every
    chunk empty (the running maximum stays -inf across them), a single record,
    no record, random holes; a large scale so that the lazily moved reference
    of the softmax moves often."""
    w = tg.Workload("attend_full_holes", 16, 1, 32768, 576, 2, 2048, 4096, 2, tg.LOCALITY, 0.87, seed_index=69)
    sel_all = tg.trace(w)
    pool = keep(make_pool(hs, w))
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = keep(make_resolver(hs, w, pool))
    res.set_option(hs.HS_OPT_ATTN_HEADS, heads_per_wg)
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(12)
    slot_idx = torch.empty((w.num_req, w.k), dtype=torch.int32, device=dev)
    for t in range(w.steps):
        sel = np.ascontiguousarray(sel_all[t, 0])
        res.resolve(0, torch.from_numpy(sel).to(dev), slot_idx)
        res.check_error()
    valid = rng.random((w.num_req, w.k)) < 0.9
    valid[0, :] = True
    valid[1, :] = (np.arange(w.k) % 256) >= 200     # the first 200 of every 256 left out
    valid[2, :] = False
    valid[2, w.k - 1] = True
    valid[3, :] = False
    s = slot_idx.cpu().numpy()
    s[~valid] = -1
    slot_idx = torch.from_numpy(s).to(dev)
    q_np = rand_bits(rng, (w.num_req, 128, D_QK))
    print(f"attend full size with holes, heads/wg={heads_per_wg}", flush=True)
    out, lse = run_attend(hs, res, 0, q_np, slot_idx, 0.5, dev)
    check(hs, q_np, records(w, pool_np, 0, sel), 0.5, out, lse, valid=valid)


def test_attend_in_a_captured_graph(hs):
    """RESOLVE + attention captured together and replayed over several steps,
    with eager work between replays: every replay equals the eager run."""
    w = tg.Workload("attend_graph", 2, 2, 8192, 576, 2, 256, 512, 6, tg.LOCALITY, 0.8, seed_index=67)
    sel_all = torch.from_numpy(tg.trace(w)).to(torch.device("cuda:0"))
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(11)
    q = torch.from_numpy(rand_bits(rng, (w.num_req, 64, D_QK)).view(np.int16)).to(dev)

    def run(res, graph_steps):
        outs = []
        slot = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
        o = torch.empty((w.num_layers, w.num_req, 64, D_V), dtype=torch.float32, device=dev)
        lse = torch.empty((w.num_layers, w.num_req, 64), dtype=torch.float32, device=dev)
        res.resolve(0, sel_all[0, 0], slot[0])
        res.attend_mla(0, q, slot[0], 0.1, o[0], lse[0])      # sizes the workspace before any capture
        torch.cuda.synchronize()
        res.reset()
        if graph_steps:
            g = torch.cuda.CUDAGraph()
            # the captured step reads its selection from a fixed buffer
            cur = torch.empty_like(sel_all[0])
            with torch.cuda.graph(g):
                for l in range(w.num_layers):
                    res.resolve(l, cur[l], slot[l])
                    res.attend_mla(l, q, slot[l], 0.1, o[l], lse[l])
            for t in range(w.steps):
                cur.copy_(sel_all[t])
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                _ = torch.ones(1024, device=dev).sum().item()       # eager work between replays
                outs.append((o.cpu().clone(), lse.cpu().clone()))
            del g
        else:
            for t in range(w.steps):
                for l in range(w.num_layers):
                    res.resolve(l, sel_all[t, l], slot[l])
                    res.attend_mla(l, q, slot[l], 0.1, o[l], lse[l])
                torch.cuda.synchronize()
                outs.append((o.cpu().clone(), lse.cpu().clone()))
        res.check_error()
        return outs

    pool = keep(make_pool(hs, w))
    eager = run(keep(make_resolver(hs, w, pool)), False)
    graph = run(keep(make_resolver(hs, w, pool)), True)
    for t, ((oe, le), (og, lg)) in enumerate(zip(eager, graph)):
        assert torch.equal(oe, og) and torch.equal(le, lg), f"step {t}"
