"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties the oracle to something other than itself:
  - a hand-derived walkthrough (tests/golden/resolve_walkthrough.txt);
  - the footprint identity and the pages' printed instance (golden/footprint.txt);
  - closed forms: step 0 is all-miss, B = k reduces to top-k-only staging,
    uniform selection gives a hypergeometric hit count;
  - invariants: set identity of hits and misses, B >= k safety, occupancy,
    byte exactness of every cached record, page-table consistency.
"""
import os

import numpy as np
import pytest

import tracegen as tg
from oracle import E_DUP, E_RANGE, Oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def parse_walkthrough():
    params, steps, final = {}, [], {}
    with open(os.path.join(GOLDEN, "resolve_walkthrough.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("step"):
                parts = [p.strip() for p in line.split("|")]
                head = parts[0].split()
                rec = {"sel": [int(x) for x in head[3:]]}
                for p in parts[1:]:
                    toks = p.split()
                    if toks[0] == "plan":
                        rec["plan"] = [tuple(int(v) for v in e.split(",")) for e in toks[1:]]
                    else:
                        rec[toks[0]] = [int(x) for x in toks[1:]]
                steps.append(rec)
            elif line.startswith("final"):
                toks = line.split()
                final[toks[1]] = [int(x) for x in toks[2:]]
            else:
                k, v = line.split()
                params[k] = int(v)
    return params, steps, final


def test_golden_walkthrough():
    p, steps, final = parse_walkthrough()
    o = Oracle(1, 1, p["B"], p["L_ctx"], 16, model_bytes=False)
    for st in steps:
        r = o.resolve(0, np.array([st["sel"]], np.int32))
        assert r["err"][0] == st["err"][0], st
        assert r["slot_idx"][0].tolist() == st["slot_idx"], st
        assert r["hit_mask"][0].tolist() == st["hit"], st
        m = int(r["miss_count"][0])
        assert m == len(st["plan"]), st
        assert [tuple(x) for x in r["plan"][0, :m].tolist()] == st["plan"], st
    assert o.slot_pos[0, 0].tolist() == final["slot_pos"]
    assert o.ts[0, 0].tolist() == final["ts"]
    assert o.page_table[0, 0].tolist() == final["page_table"]
    assert int(o.clock[0, 0]) == final["clock"][0]


def test_footprint_identity_printed_instance():
    vals = {}
    with open(os.path.join(GOLDEN, "footprint.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    # HBM = N_l * B * W_KV * s does not contain L_ctx: the full-context figure
    # scales by B / L_ctx.
    cached = vals["full_context_gb"] * vals["B"] / vals["L_ctx"]
    assert vals["L_ctx"] / vals["B"] == vals["ratio"]
    assert abs(cached - vals["cached_gb_printed"]) < 0.05
    # the oracle's device-side model holds exactly N_l*B*row bytes per request
    w = tg.TINY
    o = Oracle(2, 3, w.B, w.L_ctx, w.row_bytes)
    assert o.cache.nbytes == 2 * 3 * w.B * w.W_KV * w.elem_bytes
    assert o.cache.shape == (3, 2, w.B, w.row_bytes)


def run_workload(w, steps, model_bytes=True, layers=None):
    """Replay `steps` steps; yields (t, l, sel, result, oracle) after each call."""
    tr = tg.trace(w, steps=steps)
    pool = tg.small_pool(w) if model_bytes else None
    rr = w.region_rows()
    o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes, model_bytes=model_bytes)
    layers = range(w.num_layers) if layers is None else layers
    for t in range(steps):
        for l in layers:
            res = o.resolve(l, tr[t, l], pool, rr)
            yield t, l, tr[t, l], res, o, pool


def small_wl(**kw):
    base = dict(name="pin", num_req=3, num_layers=2, L_ctx=3000, W_KV=24, elem_bytes=2, k=200, B=320,
                steps=30, p_keep=0.8, seed_index=21)
    base.update(kw)
    return tg.Workload(**base)


@pytest.mark.parametrize("w", [
    small_wl(),
    small_wl(B=200, name="b_eq_k"),
    small_wl(mode=tg.UNIFORM, L_ctx=900, name="uniform"),
    small_wl(k=7, B=13, L_ctx=40, steps=60, p_keep=0.5, window=3, name="tiny_ragged"),
])
def test_invariants_small(w):
    """P1 step 0 all-miss; P2 miss count = |S_t minus R_{t-1}|; P3 B >= k safety;
    P4 occupancy; P8 exactness and page-table consistency."""
    resident_prev = {}
    fetched = {}
    for t, l, sel, res, o, pool in run_workload(w, w.steps):
        for r in range(w.num_req):
            S = sel[r].tolist()
            key = (l, r)
            prev = resident_prev.get(key, set())
            m = int(res["miss_count"][r])
            assert res["err"][r] == 0
            if t == 0:
                assert m == w.k and res["slot_idx"][r].tolist() == list(range(w.k))
            # P2: set identity, resident set tracked with plain Python sets
            assert m == len(set(S) - prev)
            assert int(res["hit_mask"][r].sum()) == len(set(S) & prev)
            plan = res["plan"][r, :m]
            evicted = {int(x) for x in plan[:, 2] if x >= 0}
            # P3: nothing selected is evicted; everything selected is resident after
            assert not (evicted & set(S))
            now = (prev - evicted) | set(S)
            spos = o.slot_pos[l, r]
            assert now == {int(x) for x in spos if x >= 0}
            assert set(S) <= now
            # P4: occupancy = min(B, total misses so far)
            fetched[key] = fetched.get(key, 0) + m
            assert len(now) == min(w.B, fetched[key])
            resident_prev[key] = now
            # P8: published slot holds exactly S[j]; state maps are mutually inverse
            si = res["slot_idx"][r]
            assert np.array_equal(spos[si], sel[r])
            pt = o.page_table[l, r]
            occ = np.nonzero(spos >= 0)[0]
            assert np.array_equal(pt[spos[occ]], occ)
            assert int((pt >= 0).sum()) == occ.size
            base = w.region_rows()[r * w.num_layers + l]
            assert np.array_equal(o.cache[l, r][occ], pool[base + spos[occ]])


def test_b_equals_k_is_topk_staging():
    """P5: with B = k the resident set after each step is exactly S_t (top-k-only
    staging, the pages' Swap-vanilla baseline), so m_t = |S_t minus S_{t-1}|."""
    w = small_wl(B=200, k=200, steps=25, p_keep=0.7)
    prev = {}
    for t, l, sel, res, o, _ in run_workload(w, w.steps, model_bytes=False):
        for r in range(w.num_req):
            S = set(sel[r].tolist())
            if (l, r) in prev:
                assert int(res["miss_count"][r]) == len(S - prev[(l, r)])
            assert {int(x) for x in o.slot_pos[l, r]} == S
            prev[(l, r)] = S


def test_uniform_selection_hypergeometric():
    """P6 (the review's falsifier): with k uniform positions per step and B = k,
    once full the hit count is Hypergeometric(L_ctx, B, k); mean B*k/L_ctx."""
    w = small_wl(mode=tg.UNIFORM, k=256, B=256, L_ctx=4096, num_req=8, num_layers=2, steps=60)
    hits = []
    for t, l, sel, res, o, _ in run_workload(w, w.steps, model_bytes=False):
        if t > 0:
            hits.extend((w.k - res["miss_count"]).tolist())
    hits = np.array(hits, np.float64)
    N, K, n = w.L_ctx, w.B, w.k
    mean = n * K / N
    var = n * (K / N) * (1 - K / N) * (N - n) / (N - 1)
    assert abs(hits.mean() - mean) < 5 * np.sqrt(var / hits.size)
    assert abs(hits.var() - var) < 0.15 * var
    # expected miss rate 1 - B/L_ctx
    assert abs(1 - hits.mean() / n - (1 - K / N)) < 0.01


def test_uniform_selection_no_locality_workload():
    """P6 at the no-locality workload's shape (B = k = 2048 of 262144): the mean
    hit count over every (request, layer, step > 0) is 16 +- 5 sigma."""
    w = tg.NOLOCALITY.replace(steps=24)
    hits = []
    for t, l, sel, res, o, _ in run_workload(w, w.steps, model_bytes=False):
        if t > 0:
            hits.extend((w.k - res["miss_count"]).tolist())
    hits = np.array(hits, np.float64)
    N, K, n = w.L_ctx, w.B, w.k
    var = n * (K / N) * (1 - K / N) * (N - n) / (N - 1)
    assert abs(hits.mean() - 16.0) < 5 * np.sqrt(var / hits.size)


def test_shared_layers_equal_anchor():
    """P10: layers that receive their anchor's selection every step produce the
    anchor's outputs (each layer keeps its own state)."""
    w = tg.PREFETCH.replace(num_req=2, L_ctx=20000, steps=12, k=256, B=512)
    out = {}
    for t, l, sel, res, o, _ in run_workload(w, w.steps, model_bytes=False):
        out[(t, l)] = res
    for t in range(w.steps):
        for l in range(w.num_layers):
            a = out[(t, (l // w.group) * w.group)]
            for key in ("slot_idx", "hit_mask", "miss_count"):
                assert np.array_equal(out[(t, l)][key], a[key])


def test_rejected_inputs_leave_state():
    o = Oracle(2, 1, 8, 50, 4, model_bytes=False)
    good = np.array([[1, 2, 3], [4, 5, 6]], np.int32)
    o.resolve(0, good)
    snap = (o.slot_pos.copy(), o.ts.copy(), o.page_table.copy(), o.clock.copy())
    bad = np.array([[7, 7, 8], [50, 1, 2]], np.int32)
    r = o.resolve(0, bad)
    assert r["err"].tolist() == [E_DUP, E_RANGE]
    assert np.all(r["slot_idx"] == -1) and np.all(r["miss_count"] == 0)
    for a, b in zip(snap, (o.slot_pos, o.ts, o.page_table, o.clock)):
        assert np.array_equal(a, b)
    # k > B is refused
    o2 = Oracle(1, 1, 2, 50, 4, model_bytes=False)
    r = o2.resolve(0, np.array([[1, 2, 3]], np.int32))
    assert r["err"][0] != 0


def test_append_grows_history_and_is_fetched_on_first_selection():
    """Decode-time append: the record goes to the history's next position in
    the pool; positions at or beyond the length are out of range; the first
    selection of the appended position is a miss that copies exactly the
    appended bytes; a full history refuses the append."""
    from oracle import E_FULL
    R, L_ctx, B, row = 2, 12, 4, 16
    pool = np.zeros((R * L_ctx, row), np.uint8)
    o = Oracle(R, 1, B, L_ctx, row)
    o.length[0, :] = 5
    r0 = o.resolve(0, np.array([[0, 5], [1, 2]], np.int32), pool)   # position 5 not written yet
    assert r0["err"].tolist() == [E_RANGE, 0]
    rows = np.arange(R * row, dtype=np.uint8).reshape(R, row) + 1
    assert o.append(0, rows, pool).tolist() == [0, 0]
    assert o.length[0].tolist() == [6, 6]
    assert np.array_equal(pool[5], rows[0]) and np.array_equal(pool[L_ctx + 5], rows[1])
    r1 = o.resolve(0, np.array([[5, 0], [5, 1]], np.int32), pool)
    assert r1["err"].tolist() == [0, 0]
    assert r1["hit_mask"][0, 0] == 0 and r1["hit_mask"][1, 0] == 0 and r1["hit_mask"][1, 1] == 1
    assert np.array_equal(o.cache[0, 0, r1["slot_idx"][0, 0]], rows[0])
    assert np.array_equal(o.cache[0, 1, r1["slot_idx"][1, 0]], rows[1])
    o.length[0, :] = L_ctx
    before = pool.copy()
    assert o.append(0, rows, pool).tolist() == [E_FULL, E_FULL]
    assert np.array_equal(pool, before) and o.length[0].tolist() == [L_ctx, L_ctx]


def test_shrinking_a_history_drops_its_cached_tail():
    """Lowering a history's length drops the cached copies of the positions
    it cuts off, so a record appended again at such a position is fetched
    from the pool rather than served from the old copy (the host pool is
    the authoritative copy, blog section 2, item 1).  Hand-derived: B = 3,
    step 0 selects [2, 7] (slots 0, 1, stamp 1); length 5 empties slot 1
    (position 7 > 4) and keeps slot 0; three appends write positions 5, 6, 7;
    step 1 selects [7, 2]: 2 hits slot 0 (stamp 4), 7 misses and takes the
    empty slot 1 (stamp 3) and its new bytes."""
    L_ctx, row = 10, 16
    pool = np.zeros((L_ctx, row), np.uint8)
    for p in range(L_ctx):
        pool[p] = p + 1
    o = Oracle(1, 1, 3, L_ctx, row)
    r0 = o.resolve(0, np.array([[2, 7]], np.int32), pool)
    assert r0["slot_idx"].tolist() == [[0, 1]] and o.ts[0, 0].tolist() == [1, 1, 0]
    o.set_lengths([[5]])
    assert o.slot_pos[0, 0].tolist() == [2, -1, -1]
    assert o.ts[0, 0].tolist() == [1, 0, 0]
    assert o.page_table[0, 0, 7] == -1 and o.page_table[0, 0, 2] == 0
    assert o.length[0, 0] == 5
    for v in (0x51, 0x61, 0xAB):
        assert o.append(0, np.full((1, row), v, np.uint8), pool).tolist() == [0]
    assert o.length[0, 0] == 8 and np.all(pool[7] == 0xAB)
    r1 = o.resolve(0, np.array([[7, 2]], np.int32), pool)
    assert r1["slot_idx"].tolist() == [[1, 0]] and r1["hit_mask"].tolist() == [[0, 1]]
    assert r1["plan"][0, 0].tolist() == [0, 1, -1, 7]
    assert o.ts[0, 0].tolist() == [4, 3, 0]
    assert np.all(o.cache[0, 0, 1] == 0xAB)
    # a length outside [0, L_ctx] is refused
    with pytest.raises(ValueError):
        o.set_lengths([[L_ctx + 1]])
