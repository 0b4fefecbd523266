"""Shared helpers of the GPU parity tests: run the HIP path and the oracle side by side."""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import tracegen as tg


def threads() -> int:
    return max(1, min(16, int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)))


def make_pool(hs, w, coherent=False):
    """Pinned host pool holding the workload's seeded rows."""
    pool = hs.HostPool.allocate(w.pool_rows * w.row_bytes, coherent=coherent)
    tg.pool_fill(pool.ptr, 0, w.pool_rows * w.W_KV, w.pool_seed, threads())
    return pool


def make_resolver(hs, w, pool):
    return hs.Resolver(w.num_req, w.num_layers, w.B, w.W_KV, hs.BF16, pool, w.L_ctx, w.pool_rows,
                       region_row=w.region_rows())


def oracle_step(o, w, sel_t, pool_np, pool_arg=True, pool_exec=None):
    """Run the oracle on all layers of one step (layers in parallel threads:
    each call touches only its own layer's state)."""
    rr = w.region_rows()
    pool = pool_np if pool_arg else None
    if pool_exec is None:
        return [o.resolve(l, sel_t[l], pool, rr) for l in range(w.num_layers)]
    futs = [pool_exec.submit(o.resolve, l, sel_t[l], pool, rr) for l in range(w.num_layers)]
    return [f.result() for f in futs]


def executor():
    return cf.ThreadPoolExecutor(max_workers=threads())


def compare_step(res_gpu_slot_idx, ref, state, w, l, t, check_plan=True):
    """Element-wise comparison of one layer's published output and plan."""
    assert np.array_equal(res_gpu_slot_idx, ref["slot_idx"]), f"slot_idx differs at step {t} layer {l}"
    k = ref["slot_idx"].shape[1]
    assert np.array_equal(state["hit_mask"][:, :k], ref["hit_mask"]), f"hit_mask differs at step {t} layer {l}"
    assert np.array_equal(state["miss_count"], ref["miss_count"]), f"miss_count differs at step {t} layer {l}"
    if check_plan:
        for r in range(w.num_req):
            m = int(ref["miss_count"][r])
            assert np.array_equal(state["plan"][r, :m], ref["plan"][r, :m]), f"plan differs step {t} l {l} r {r}"


def checksum_ref(rows: np.ndarray) -> int:
    """The consumer stand-in's reduction over gathered rows [k][row_bytes], in uint64 arithmetic."""
    words = rows.reshape(-1).view(np.uint64)
    idx = np.arange(words.size, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return int(np.sum(words * (2 * idx + 1), dtype=np.uint64))
