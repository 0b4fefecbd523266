"""Brute force on tiny caches: the stamp-based oracle against the recency-list model.

Every ordered selection sequence with L_ctx <= 5, k <= 2, T <= 3 steps and
every B in [k, L_ctx] is replayed through both models (plus a random sample
of longer sequences with L_ctx = 6, k = 3); slot assignment, hit mask and
plan must agree exactly.  The victim set is also checked against an
enumeration over all m-subsets of the candidate slots: it must be the
subset whose sorted (stamp, slot) keys are lexicographically smallest.
"""
import itertools
import os
import random
import shutil
import subprocess
import sys

import numpy as np
import pytest

from spec_model import RecencyListModel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sequences(L, k, T):
    tuples = list(itertools.permutations(range(L), k))
    return itertools.product(tuples, repeat=T)


def compare(oracle_cls, B, L, seq):
    o = oracle_cls(1, 1, B, L, 4, model_bytes=False)
    spec = RecencyListModel(B)
    for S in seq:
        ts_before = o.ts[0, 0].copy()
        res = o.resolve(0, np.array([S], np.int32))
        sidx, hit, plan = spec.resolve(list(S))
        m = int(res["miss_count"][0])
        if res["slot_idx"][0].tolist() != sidx or res["hit_mask"][0].tolist() != hit:
            return False
        if [tuple(x) for x in res["plan"][0, :m].tolist()] != plan:
            return False
        # victims are the lexicographically smallest m-subset of candidates
        hit_slots = {sidx[j] for j in range(len(S)) if hit[j]}
        cand = [s for s in range(B) if s not in hit_slots]
        best = min(itertools.combinations(cand, m),
                   key=lambda c: sorted((int(ts_before[s]), s) for s in c))
        if sorted(best) != sorted(p[1] for p in plan):
            return False
    o.close()
    return True


def exhaustive(oracle_cls):
    n = 0
    for L in range(1, 6):
        for k in range(1, min(2, L) + 1):
            for T in range(1, 4):
                for B in range(k, L + 1):
                    for seq in _sequences(L, k, T):
                        if not compare(oracle_cls, B, L, seq):
                            return False, (L, k, T, B, seq)
                        n += 1
    return True, n


def sampled(oracle_cls, n_seq=400, seed=5):
    rng = random.Random(seed)
    for _ in range(n_seq):
        L = rng.randint(3, 6)
        k = rng.randint(1, min(3, L))
        B = rng.randint(k, L)
        T = rng.randint(2, 8)
        seq = [tuple(rng.sample(range(L), k)) for _ in range(T)]
        if not compare(oracle_cls, B, L, seq):
            return False, (L, k, B, seq)
    return True, n_seq


def test_bruteforce_exhaustive():
    from oracle import Oracle
    ok, info = exhaustive(Oracle)
    assert ok, info
    assert info > 40000


def test_bruteforce_sampled():
    from oracle import Oracle
    ok, info = sampled(Oracle)
    assert ok, info


# ---- planted mistakes: a copy of the oracle with one deliberate error must be
# caught by the brute force or the golden walkthrough. -----------------------

MUTATIONS = [
    ("hit stamp equals miss stamp", "ts[out_idx[j]] = 2u * t + 2u", "ts[out_idx[j]] = 2u * t + 1u"),
    ("miss stamp above hits", "ts[v] = 2u * t + 1u", "ts[v] = 2u * t + 3u"),
    ("newest evicted first", "if (x->ts != y->ts) return x->ts < y->ts ? -1 : 1;",
     "if (x->ts != y->ts) return x->ts > y->ts ? -1 : 1;"),
    ("highest slot wins ties", "return (x->slot > y->slot) - (x->slot < y->slot);",
     "return (x->slot < y->slot) - (x->slot > y->slot);"),
    ("victims not re-sorted", "qsort(victims, (size_t)m, sizeof(int32_t), cmp_int);", ""),
    ("hits not promoted", "if (out_hit[j]) ts[out_idx[j]] = 2u * t + 2u;", ""),
    ("evicted page not cleared", "if (old >= 0) pt[old] = -1;", ""),
    ("clock not advanced", "o->clock[rl] = t + 1u;", ""),
]


def _build_mutant(tmp_path, src, name):
    so = tmp_path / f"liboracle_{name}.so"
    c = tmp_path / f"oracle_{name}.c"
    c.write_text(src)
    subprocess.run(["gcc", "-O1", "-std=c11", "-shared", "-fPIC", "-o", str(so), str(c)], check=True)
    return str(so)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("label,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, label, old, new):
    import oracle as oracle_pkg
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(old) == 1, label
    path = _build_mutant(tmp_path, src.replace(old, new), abs(hash(label)) % 10**8)
    import ctypes
    saved = oracle_pkg._lib
    try:
        oracle_pkg._lib = None
        oracle_pkg._LIB_PATH, orig = path, oracle_pkg._LIB_PATH
        caught = False
        try:
            from test_oracle_pins import test_golden_walkthrough
            test_golden_walkthrough()
        except AssertionError:
            caught = True
        if not caught:
            ok, _ = sampled(oracle_pkg.Oracle, n_seq=300, seed=7)
            caught = not ok
        if not caught:
            ok, _ = exhaustive(oracle_pkg.Oracle)
            caught = not ok
        if not caught and "page" in label:
            # consistency of page table vs slot map is an invariant test
            o = oracle_pkg.Oracle(1, 1, 2, 6, 4, model_bytes=False)
            for S in ([0, 1], [2, 3], [4, 5]):
                o.resolve(0, np.array([S], np.int32))
            caught = int((o.page_table[0, 0] >= 0).sum()) != 2
        assert caught, f"planted mistake not caught: {label}"
    finally:
        oracle_pkg._LIB_PATH = orig
        oracle_pkg._lib = saved
