"""Seeded input generators: published test vectors, determinism and trace shape."""
import numpy as np
import pytest

import tracegen as tg


def test_splitmix64_published_vectors():
    # splitmix64 (Steele, Lea & Flood 2014): first outputs for seeds 0 and 1234567
    # as printed alongside the generator's reference implementation.
    assert tg.splitmix64_at(0, 0) == 0xE220A8397B1DCDAF
    assert tg.splitmix64_at(1234567, 0) == 6457827717110365317
    assert tg.splitmix64_at(1234567, 1) == 3203168211198807973


def test_xoshiro256starstar_hand_values():
    # From state {1,2,3,4}: out0 = rotl(2*5,7)*9 = 11520; after one update s1 = 0
    # so out1 = 0; after the second s1 = 262149, out2 = rotl(262149*5,7)*9.
    out = tg.xoshiro_outputs([1, 2, 3, 4], 3)
    assert out == [11520, 0, (262149 * 5 << 7) * 9]


def small(mode=tg.LOCALITY, **kw):
    base = dict(name="t", num_req=3, num_layers=4, L_ctx=5000, W_KV=8, elem_bytes=2, k=300, B=600,
                steps=40, mode=mode, p_keep=0.8, seed_index=11)
    base.update(kw)
    return tg.Workload(**base)


@pytest.mark.parametrize("mode", [tg.LOCALITY, tg.UNIFORM, tg.HITONLY])
def test_trace_distinct_in_range_deterministic(mode):
    w = small(mode)
    a = tg.trace(w, threads=3)
    b = tg.trace(w, threads=1)
    assert np.array_equal(a, b)
    assert a.shape == (w.steps, w.num_layers, w.num_req, w.k)
    assert a.min() >= 0 and a.max() < w.L_ctx
    s = np.sort(a, axis=-1)
    assert not np.any(s[..., 1:] == s[..., :-1])


def test_trace_retention_and_locality():
    w = small(tg.LOCALITY, p_keep=0.87, k=2048, L_ctx=131072, B=4096, num_req=2, num_layers=2, steps=30)
    tr = tg.trace(w)
    same = (tr[1:] == tr[:-1])
    n = same.size
    # retention is Bernoulli(p) per (step, j): 6 sigma binomial band
    sig = np.sqrt(0.87 * 0.13 / n)
    assert abs(same.mean() - 0.87) < 6 * sig


def test_trace_redraws_half_local():
    # Sparse setting so that a uniform redraw rarely lands near a kept position:
    # then about half of the redraws (the local branch) sit within +-64 of one.
    w = small(tg.LOCALITY, p_keep=0.5, k=256, L_ctx=1 << 22, num_req=16, num_layers=1, steps=4)
    tr = tg.trace(w)
    near_all = []
    for t in range(1, w.steps):
        for r in range(w.num_req):
            prev, cur = tr[t - 1, 0, r], tr[t, 0, r]
            kept = np.sort(cur[prev == cur])
            red = cur[prev != cur]
            pos = np.searchsorted(kept, red)
            lo = np.abs(red - kept[np.clip(pos - 1, 0, kept.size - 1)])
            hi = np.abs(kept[np.clip(pos, 0, kept.size - 1)] - red)
            near_all.append(np.minimum(lo, hi) <= 64)
    near = np.concatenate(near_all)
    assert abs(near.mean() - 0.5) < 6 * np.sqrt(0.25 / near.size) + 0.01


def test_trace_groups_share_selection():
    w = small(tg.LOCALITY, num_layers=8, group=4)
    tr = tg.trace(w)
    for g in range(2):
        for l in range(1, 4):
            assert np.array_equal(tr[:, 4 * g], tr[:, 4 * g + l])
    assert not np.array_equal(tr[:, 0], tr[:, 4])


def test_hitonly_repeats_step0():
    tr = tg.trace(small(tg.HITONLY))
    assert np.all(tr == tr[:1])


def test_pool_counter_based_and_normal():
    seed = 99
    n = 1 << 20
    full = np.empty(n, np.uint16)
    tg.pool_fill(full.ctypes.data, 0, n, seed, 4)
    part = np.empty(1001, np.uint16)
    tg.pool_fill(part.ctypes.data, 12345, 1001, seed, 1)
    assert np.array_equal(part, full[12345:13346])
    f = (full.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(f.mean()) < 5 / np.sqrt(n)
    assert abs(f.std() - 1.0) < 0.01
    assert abs((np.abs(f) < 1).mean() - 0.6827) < 0.005


def test_workload_shapes():
    assert tg.MLA.row_bytes == 1152 and tg.GQA.row_bytes == 4096
    assert tg.GQA.logical_rows * tg.GQA.row_bytes == 512 << 30
    assert tg.GQA.pool_rows * tg.GQA.row_bytes == 64 << 30
    rr = tg.GQA.region_rows()
    assert rr.max() + tg.GQA.L_ctx <= tg.GQA.pool_rows
    assert np.array_equal(tg.MLA.region_rows(), np.arange(128) * 131072)
