"""Randomized parity: seeded random shapes and selections, k changing from call
to call, several handles alive at once, bit-exact against the oracle."""
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


def random_case(rng, i):
    B = int(rng.choice([1, 2, 3, 5, 17, 64, 255, 256, 511, 1000, 1023, 1024, 1025, 2048, 3001, 4096, 5000, 8192,
                        12000, 16384]))
    R = int(rng.integers(1, 9))
    NL = int(rng.integers(1, 4))
    L_ctx = int(max(B * rng.choice([1, 2, 4, 16]), B + int(rng.integers(0, 50))))
    W_KV = int(rng.choice([8, 24, 72, 576, 2048]))
    steps = int(rng.integers(3, 12))
    return tg.Workload(f"rand{i}", R, NL, L_ctx, W_KV, 2, min(B, 4096), B, steps, seed_index=100 + i)


def selection(rng, L_ctx, k, prev, keep):
    """k distinct positions, reusing a share of `prev` (which may be longer or shorter)."""
    out = []
    seen = set()
    if prev is not None:
        for p in prev:
            if len(out) >= k:
                break
            if rng.random() < keep and p not in seen:
                out.append(int(p))
                seen.add(int(p))
    while len(out) < k:
        x = int(rng.integers(0, L_ctx))
        if x not in seen:
            out.append(x)
            seen.add(x)
    rng.shuffle(out)
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_and_varying_k(hs, seed):
    from oracle import Oracle
    rng = np.random.default_rng(1000 + seed)
    w = random_case(rng, seed)
    print(f"[random] seed={seed} R={w.num_req} L={w.num_layers} B={w.B} L_ctx={w.L_ctx} row={w.row_bytes} "
          f"steps={w.steps}", flush=True)
    pool = make_pool(hs, w)
    pool_np = pool.numpy_view().reshape(w.pool_rows, w.row_bytes)
    res = make_resolver(hs, w, pool)
    other = make_resolver(hs, w, pool)   # a second live handle on the same pool, other probe
    other.set_option(hs.HS_OPT_PROBE, hs.HS_PROBE_PAGE_TABLE if seed % 2 == 0 else hs.HS_PROBE_SLOT_SCAN_HASH)
    o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes)
    dev = torch.device("cuda:0")
    prev = {}
    keep = float(rng.choice([0.0, 0.5, 0.9, 1.0]))
    for t in range(w.steps):
        k = int(rng.integers(1, min(w.B, 4096) + 1))
        for l in range(w.num_layers):
            sel = np.stack([selection(rng, w.L_ctx, k, prev.get((l, r)), keep) for r in range(w.num_req)])
            for r in range(w.num_req):
                prev[(l, r)] = sel[r]
            out = torch.empty((w.num_req, k), dtype=torch.int32, device=dev)
            out2 = torch.empty_like(out)
            sd = torch.from_numpy(sel).to(dev)
            res.resolve(l, sd, out)
            other.resolve(l, sd, out2)
            ref = o.resolve(l, sel, pool_np, w.region_rows())
            got = out.cpu().numpy()
            assert np.array_equal(got, ref["slot_idx"]), f"seed {seed} step {t} layer {l} k {k}"
            assert np.array_equal(out2.cpu().numpy(), got)
            st = res.state(l)
            assert np.array_equal(st["hit_mask"][:, :k], ref["hit_mask"])
            assert np.array_equal(st["slot_pos"], o.slot_pos[l])
            assert np.array_equal(st["ts"], o.ts[l])
            assert np.array_equal(st["page_table"], o.page_table[l])
            for r in range(w.num_req):
                m = int(ref["miss_count"][r])
                assert np.array_equal(st["plan"][r, :m], ref["plan"][r, :m])
            occ = o.slot_pos[l] >= 0
            assert np.array_equal(res.cache_layer(l)[occ], o.cache[l][occ])
    assert res.error()[0] == 0 and other.error()[0] == 0
    res.close()
    other.close()
    pool.free()
