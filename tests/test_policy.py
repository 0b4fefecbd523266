"""The cache-policy trace study's replay library, pinned on the CPU.

Pins: every policy reduces to top-k-only staging at B = k (closed form
|S_t minus S_{t-1}|); the RESOLVE contract's policy reproduces the oracle's
miss counts step by step (two independent implementations); Belady's
farthest-next-use rule equals the exhaustive optimum over all eviction
choices on tiny traces and never exceeds any other policy; optimal misses
do not grow with B; invalid traces are refused.
"""
import functools
import itertools

import numpy as np
import pytest

import tracegen as tg

pol = pytest.importorskip("hierarchical_kv_cache_resolve_amd.policy")
ALL = (pol.LRU_PROMOTE, pol.LRU, pol.FIFO, pol.BELADY)


def random_trace(rng, steps, k, L, keep):
    out = np.empty((steps, k), np.int32)
    prev = None
    for t in range(steps):
        chosen = []
        if prev is not None:
            chosen = [int(p) for p in prev if rng.random() < keep]
        pool = [p for p in range(L) if p not in set(chosen)]
        extra = rng.choice(pool, size=k - len(chosen), replace=False) if k > len(chosen) else []
        row = np.array(chosen + [int(x) for x in extra], np.int32)
        rng.shuffle(row)
        out[t] = row
        prev = row
    return out


def optimum(sel, B):
    """Fewest total misses over every eviction choice (exhaustive search)."""
    steps = [frozenset(int(x) for x in row) for row in sel]

    @functools.lru_cache(maxsize=None)
    def f(t, cache):
        if t == len(steps):
            return 0
        S = steps[t]
        miss = len(S - cache)
        rest = sorted(cache - S)
        room = B - len(S)
        best = None
        for r in range(0, min(room, len(rest)) + 1):
            for keep in itertools.combinations(rest, r):
                v = f(t + 1, S | frozenset(keep))
                best = v if best is None else min(best, v)
        return miss + best

    return f(0, frozenset())


def test_b_equals_k_is_topk_only_for_every_policy():
    rng = np.random.default_rng(1)
    for _ in range(20):
        k = int(rng.integers(1, 9))
        L = int(rng.integers(k, 40))
        sel = random_trace(rng, 12, k, L, 0.6)
        expect = [k] + [len(set(sel[t].tolist()) - set(sel[t - 1].tolist())) for t in range(1, len(sel))]
        for p in ALL:
            assert pol.replay(p, sel, k, L).tolist() == expect, pol.NAMES[p]


def test_contract_policy_matches_the_oracle_step_by_step():
    from oracle import Oracle
    rng = np.random.default_rng(2)
    for case in range(12):
        k = int(rng.integers(1, 33))
        B = k + int(rng.integers(0, 3 * k + 1))
        L = B + int(rng.integers(1, 200))
        sel = random_trace(rng, 15, k, L, float(rng.choice([0.3, 0.7, 0.95])))
        o = Oracle(1, 1, B, L, 8, model_bytes=False)
        ref = [int(o.resolve(0, sel[t][None, :])["miss_count"][0]) for t in range(len(sel))]
        assert pol.replay(pol.LRU_PROMOTE, sel, B, L).tolist() == ref, case
    w = tg.TINY
    tr = tg.trace(w)
    o = Oracle(1, 1, w.B, w.L_ctx, 8, model_bytes=False)
    ref = [int(o.resolve(0, tr[t, 0])["miss_count"][0]) for t in range(w.steps)]
    assert pol.replay(pol.LRU_PROMOTE, tr[:, 0, 0], w.B, w.L_ctx).tolist() == ref


def test_belady_is_the_exhaustive_optimum_on_tiny_traces():
    rng = np.random.default_rng(3)
    checked = 0
    for _ in range(150):
        k = int(rng.integers(1, 3))
        L = int(rng.integers(k + 1, 7))
        B = int(rng.integers(k, min(L, 4) + 1))
        sel = random_trace(rng, int(rng.integers(2, 6)), k, L, 0.5)
        best = optimum(sel, B)
        got = {p: int(pol.replay(p, sel, B, L).sum()) for p in ALL}
        assert got[pol.BELADY] == best, (sel.tolist(), B, got, best)
        assert all(v >= best for v in got.values())
        checked += 1
    assert checked == 150


def test_belady_never_worse_and_monotone_in_b():
    rng = np.random.default_rng(4)
    for _ in range(10):
        k = int(rng.integers(2, 17))
        L = int(rng.integers(4 * k + 1, 20 * k))
        sel = random_trace(rng, 30, k, L, 0.7)
        prev = None
        for B in range(k, 4 * k + 1, max(1, k // 2)):
            tot = {p: int(pol.replay(p, sel, B, L).sum()) for p in ALL}
            assert tot[pol.BELADY] <= min(tot.values())
            if prev is not None:
                assert tot[pol.BELADY] <= prev
            prev = tot[pol.BELADY]


def test_replay_many_equals_single_replays():
    w = tg.TINY.replace(num_req=3, num_layers=2, steps=20, k=64, B=128, seed_index=77)
    tr = tg.trace(w)                                  # [steps][layers][req][k]
    for p in ALL:
        many = pol.replay_many(p, tr, 96, w.L_ctx, threads=3)
        single = [int(pol.replay(p, tr[:, l, r], 96, w.L_ctx).sum())
                  for l in range(w.num_layers) for r in range(w.num_req)]
        assert many.tolist() == single


def test_study_rates_and_step_zero():
    w = tg.TINY.replace(steps=16)
    tr = tg.trace(w)
    rates = pol.study(tr, w.L_ctx, [w.k, 2 * w.k])
    misses = pol.replay(pol.BELADY, tr[:, 0, 0], 2 * w.k, w.L_ctx)
    assert misses[0] == w.k
    assert rates[("belady", 2 * w.k)] == pytest.approx(misses[1:].sum() / (15 * w.k))
    assert rates[("belady", w.k)] == rates[("lru_promote", w.k)]


def test_invalid_traces_are_refused():
    good = np.array([[0, 1], [2, 3]], np.int32)
    with pytest.raises(ValueError):
        pol.replay(pol.LRU, np.array([[0, 0]], np.int32), 2, 4)       # repeated position
    with pytest.raises(ValueError):
        pol.replay(pol.LRU, np.array([[0, 9]], np.int32), 2, 4)       # outside [0, L_ctx)
    with pytest.raises(ValueError):
        pol.replay(pol.LRU, good, 1, 4)                              # B < k
    with pytest.raises(ValueError):
        pol.replay(7, good, 2, 4)                                    # unknown policy
