"""Cache-policy trace study: replay selection traces under replacement policies.

The study replays a sparse-selection trace under several cache
configurations and reports miss rates (pith.science review of HiSparse,
Figure 6 caption and "What carries the argument": top-k-only staging at
B = k against LRU caches of B slots; Belady's offline-optimal replacement as
the bound, the review's supporting citation [3]).  The replay itself is the
C++ library libhspolicy.so (include/hspolicy.h); this module marshals numpy
arrays and runs the sweep.

    python -m hierarchical_kv_cache_resolve_amd.policy --workload mla_latent

prints the miss rate of every policy at B = k, 1.5k, 2k, 3k, 4k on the
workload's seeded synthetic trace.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libhspolicy.so")

LRU_PROMOTE, LRU, FIFO, BELADY = 0, 1, 2, 3
NAMES = {LRU_PROMOTE: "lru_promote", LRU: "lru", FIFO: "fifo", BELADY: "belady"}
ERRORS = {-1: "invalid argument", -2: "position out of range", -3: "repeated position", -4: "out of memory"}

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built (run hierarchical_kv_cache_resolve_amd/_build.py)")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.hs_policy_replay.restype = i32
        lib.hs_policy_replay.argtypes = [i32, i32, i32, i32, i64, vp, vp]
        lib.hs_policy_replay_many.restype = i32
        lib.hs_policy_replay_many.argtypes = [i32, i32, i32, i32, i64, i32, vp, vp, i32]
        _lib = lib
    return _lib


def _check(rc):
    if rc != 0:
        raise ValueError(f"policy replay failed: {ERRORS.get(rc, rc)}")


def replay(policy: int, sel: np.ndarray, B: int, L_ctx: int) -> np.ndarray:
    """Misses per step of one history; sel int32 [steps][k]."""
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    steps, k = sel.shape
    out = np.zeros(steps, np.int32)
    _check(_load().hs_policy_replay(policy, B, k, steps, L_ctx, sel.ctypes.data, out.ctypes.data))
    return out


def replay_many(policy: int, trace: np.ndarray, B: int, L_ctx: int, threads: int = 0) -> np.ndarray:
    """Total misses of every history of a [steps][...][k] trace, flattened over the middle axes."""
    trace = np.ascontiguousarray(trace, dtype=np.int32)
    steps, k = trace.shape[0], trace.shape[-1]
    n_hist = int(np.prod(trace.shape[1:-1])) if trace.ndim > 2 else 1
    out = np.zeros(n_hist, np.int64)
    threads = threads or min(16, os.cpu_count() or 1)
    _check(_load().hs_policy_replay_many(policy, B, k, steps, L_ctx, n_hist, trace.ctypes.data, out.ctypes.data,
                                         threads))
    return out


def study(trace: np.ndarray, L_ctx: int, Bs, policies=(LRU_PROMOTE, LRU, FIFO, BELADY), threads: int = 0) -> dict:
    """Miss rate of each (policy, B) over steps 1.. of the trace.  Step 0 is
    all-miss for every policy (k misses per history into an empty cache) and
    is left out."""
    trace = np.ascontiguousarray(trace, dtype=np.int32)
    steps, k = trace.shape[0], trace.shape[-1]
    n_hist = int(np.prod(trace.shape[1:-1])) if trace.ndim > 2 else 1
    rates = {}
    for B in Bs:
        for p in policies:
            total = int(replay_many(p, trace, B, L_ctx, threads).sum())
            rates[(NAMES[p], B)] = (total - n_hist * k) / ((steps - 1) * n_hist * k)
    return rates


def main(argv=None):
    import tracegen as tg

    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="mla_latent")
    ap.add_argument("--steps", type=int, default=0, help="trace steps (default: the workload's)")
    ap.add_argument("--b-factors", default="1,1.5,2,3,4", help="B as multiples of k")
    ap.add_argument("--threads", type=int, default=0)
    args = ap.parse_args(argv)
    w = tg.WORKLOADS[args.workload]
    steps = args.steps or w.steps
    tr = tg.trace(w, steps=steps)
    Bs = [int(round(float(f) * w.k)) for f in args.b_factors.split(",")]
    t0 = time.time()
    rates = study(tr, w.L_ctx, Bs, threads=args.threads)
    dt = time.time() - t0
    names = [NAMES[p] for p in (LRU_PROMOTE, LRU, FIFO, BELADY)]
    print(f"workload {w.name}: {w.num_req} requests x {w.num_layers} layers, k={w.k}, L_ctx={w.L_ctx}, "
          f"{steps} steps (miss rate over steps 1..{steps - 1}); replay took {dt:.1f} s")
    print("| B | " + " | ".join(names) + " |")
    print("|---|" + "---|" * len(names))
    for B in Bs:
        print(f"| {B} ({B / w.k:g}k) | " + " | ".join(f"{rates[(n, B)]:.4f}" for n in names) + " |")


if __name__ == "__main__":
    main()
