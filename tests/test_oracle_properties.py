"""Property tests of the oracle on shapes and selection sequences drawn by
Hypothesis (derandomized, so every run checks the same cases).

For every (request, layer) and step, against an independent model and
against the set identities that the pages fix:
  - slot assignment, hit mask and plan equal the stamp-free recency-list
    model (tests/spec_model.py) -- LRU with hits promoted above the step's
    misses, empty slots first, lowest slot first among equals;
  - misses = |S_t minus R_{t-1}|, the resident set before the step;
  - nothing selected is evicted (B >= k): S_t is resident afterwards;
  - occupancy |R_t| = min(B, |R_{t-1}| + m_t);
  - the page table and the slot map are inverse maps;
  - every occupied slot holds its position's host row byte for byte
    (exactness: the host copy is authoritative);
  - the step clock advances by one.
"""
import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

from spec_model import RecencyListModel  # noqa: E402


@st.composite
def scenario(draw):
    B = draw(st.integers(1, 10))
    k = draw(st.integers(1, B))
    L = draw(st.integers(k, 24))
    R = draw(st.integers(1, 2))
    NL = draw(st.integers(1, 2))
    T = draw(st.integers(1, 6))
    steps = [[[draw(st.lists(st.integers(0, L - 1), min_size=k, max_size=k, unique=True)) for _ in range(R)]
              for _ in range(NL)] for _ in range(T)]
    seed = draw(st.integers(0, 2**31 - 1))
    return B, k, L, R, NL, steps, seed


@settings(max_examples=150, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(scenario())
def test_oracle_properties(sc):
    from oracle import Oracle
    B, k, L, R, NL, steps, seed = sc
    row = 16
    pool = np.random.default_rng(seed).integers(0, 256, size=(R * NL * L, row), dtype=np.uint8)
    o = Oracle(R, NL, B, L, row)
    models = {(l, r): RecencyListModel(B) for l in range(NL) for r in range(R)}
    try:
        for t, step in enumerate(steps):
            for l in range(NL):
                before = {r: models[(l, r)].resident() for r in range(R)}
                res = o.resolve(l, np.array(step[l], np.int32), pool)
                for r in range(R):
                    S = step[l][r]
                    sidx, hit, plan = models[(l, r)].resolve(list(S))
                    m = int(res["miss_count"][r])
                    assert res["err"][r] == 0
                    assert res["slot_idx"][r].tolist() == sidx
                    assert res["hit_mask"][r].tolist() == hit
                    assert [tuple(x) for x in res["plan"][r, :m].tolist()] == plan
                    assert m == len(set(S) - before[r])
                    after = models[(l, r)].resident()
                    assert set(S) <= after
                    assert len(after) == min(B, len(before[r]) + m)
                    spos = o.slot_pos[l, r]
                    assert {int(p) for p in spos if p >= 0} == after
                    pt = o.page_table[l, r]
                    occ = np.nonzero(spos >= 0)[0]
                    assert np.array_equal(pt[spos[occ]], occ)
                    assert int((pt >= 0).sum()) == len(occ)
                    base = (r * NL + l) * L
                    assert np.array_equal(o.cache[l, r][occ], pool[base + spos[occ]])
                    assert int(o.clock[l, r]) == t + 1
    finally:
        o.close()


# The same properties must fail on every planted mistake of the brute-force
# test (a copy of the oracle with one deliberate error each).
import os  # noqa: E402
import shutil  # noqa: E402

from test_bruteforce import MUTATIONS, _build_mutant  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("label,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_properties_catch_planted_mistakes(tmp_path, label, old, new):
    import oracle as oracle_pkg
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(old) == 1, label
    path = _build_mutant(tmp_path, src.replace(old, new), abs(hash(label)) % 10**8)
    saved, orig = oracle_pkg._lib, oracle_pkg._LIB_PATH
    try:
        oracle_pkg._lib = None
        oracle_pkg._LIB_PATH = path
        with pytest.raises(AssertionError):
            test_oracle_properties()
    finally:
        oracle_pkg._LIB_PATH = orig
        oracle_pkg._lib = saved
