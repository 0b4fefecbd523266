"""Seeded synthetic inputs: selection traces and the host KV pool.

Holds none of the cache method's arithmetic.  Both the CPU oracle's tests
and the GPU path draw their inputs from here, so the two always see the
same positions and the same pool bytes.

The five workloads below restate the shapes of the HiSparse study (k = 2048
selections per step, B = 2k cache slots, 576-element MLA-style latent
records or 4 KB GQA-style records, contexts of 128K-512K tokens, layer
groups sharing one indexer output); the per-step retention probability
stands in for the temporal locality that the trace study measured on one
real selection trace ("Per-step top-k miss rate", Figure 6), which is not
reproduced.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtracegen.so")

BASE_SEED = 260807009

LOCALITY, UNIFORM, HITONLY = 0, 1, 2


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.tg_trace.restype = ctypes.c_int
    lib.tg_trace.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                             ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_int, ctypes.c_int,
                             ctypes.c_uint64, ctypes.c_int]
    lib.tg_pool_fill.restype = None
    lib.tg_pool_fill.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                 ctypes.c_int]
    lib.tg_splitmix64_at.restype = ctypes.c_uint64
    lib.tg_splitmix64_at.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    lib.tg_xoshiro_outputs.restype = None
    lib.tg_xoshiro_outputs.argtypes = [ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64),
                                       ctypes.c_int]
    lib.tg_stream_key.restype = ctypes.c_uint64
    lib.tg_stream_key.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64]
    return lib


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def default_threads() -> int:
    n = os.environ.get("OMP_NUM_THREADS")
    if n and n.isdigit() and int(n) > 0:
        return int(n)
    return max(1, min(16, os.cpu_count() or 1))


def splitmix64_at(seed: int, i: int) -> int:
    return int(lib().tg_splitmix64_at(seed & (2**64 - 1), i))


def xoshiro_outputs(state, n: int):
    st = (ctypes.c_uint64 * 4)(*[s & (2**64 - 1) for s in state])
    out = (ctypes.c_uint64 * n)()
    lib().tg_xoshiro_outputs(st, out, n)
    return [int(x) for x in out]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic decode workload: cache shape plus trace recipe."""
    name: str
    num_req: int
    num_layers: int
    L_ctx: int
    W_KV: int          # elements per record
    elem_bytes: int    # s
    k: int
    B: int
    steps: int
    mode: int = LOCALITY
    p_keep: float = 0.87
    window: int = 64
    group: int = 1     # layers per shared-selection group (anchor = first layer)
    seed_index: int = 0
    pool_rows_cap: int = 0   # 0: dense pool; else physical rows, regions alias modulo

    @property
    def row_bytes(self) -> int:
        return self.W_KV * self.elem_bytes

    @property
    def trace_seed(self) -> int:
        return splitmix64_at(BASE_SEED, 2 * self.seed_index)

    @property
    def pool_seed(self) -> int:
        return splitmix64_at(BASE_SEED, 2 * self.seed_index + 1)

    @property
    def logical_rows(self) -> int:
        return self.num_req * self.num_layers * self.L_ctx

    @property
    def pool_rows(self) -> int:
        if self.pool_rows_cap and self.pool_rows_cap < self.logical_rows:
            return self.pool_rows_cap
        return self.logical_rows

    def region_rows(self) -> np.ndarray:
        """First pool row of each (request, layer) history, [num_req*num_layers]."""
        i = np.arange(self.num_req * self.num_layers, dtype=np.int64)
        if self.pool_rows == self.logical_rows:
            return i * self.L_ctx
        n_regions = self.pool_rows // self.L_ctx
        return (i % n_regions) * self.L_ctx

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the study shape (W_KV in bf16 elements).
TINY = Workload("tiny", 1, 1, 8192, 576, 2, 256, 512, 64, LOCALITY, 0.85, seed_index=1)
MLA = Workload("mla_latent", 16, 8, 131072, 576, 2, 2048, 4096, 256, LOCALITY, 0.87, seed_index=2)
NOLOCALITY = Workload("no_locality", 32, 4, 262144, 576, 2, 2048, 2048, 128, UNIFORM, 0.0, seed_index=3)
# 512 GiB of logical pool; physical rows capped at 64 GiB, regions alias.
GQA = Workload("gqa_record", 64, 16, 131072, 2048, 2, 2048, 4096, 128, LOCALITY, 0.87, seed_index=4,
               pool_rows_cap=(64 << 30) // 4096)
PREFETCH = Workload("shared_prefetch", 8, 8, 524288, 576, 2, 2048, 4096, 64, LOCALITY, 0.87, group=4,
                    seed_index=5)

# Block-granular records (a selector that picks pages of 16 tokens, Quest-style):
# a record is 16 tokens x 576 bf16 elements = 18 KB, positions are page
# indices, and k = 128 pages covers the same 2048 tokens as the token-level
# workloads.
PAGES = Workload("page_records", 16, 8, 8192, 16 * 576, 2, 128, 256, 128, LOCALITY, 0.87, window=4,
                 seed_index=6)

WORKLOADS = {w.name: w for w in (TINY, MLA, NOLOCALITY, GQA, PREFETCH, PAGES)}


def hit_only(w: Workload) -> Workload:
    """Same shapes, but every step after the first repeats it (all hits)."""
    return w.replace(name=w.name + "_hitonly", mode=HITONLY, p_keep=1.0)


def trace(w: Workload, steps: int | None = None, threads: int | None = None) -> np.ndarray:
    """int32 [steps][num_layers][num_req][k]."""
    steps = w.steps if steps is None else steps
    out = np.empty((steps, w.num_layers, w.num_req, w.k), dtype=np.int32)
    rc = lib().tg_trace(out.ctypes.data, steps, w.num_req, w.num_layers, w.group, w.k, w.L_ctx,
                        float(w.p_keep), w.mode, w.window, w.trace_seed,
                        threads or default_threads())
    if rc != 0:
        raise ValueError(f"tg_trace rejected workload {w}")
    return out


def pool_fill(dst_ptr: int, first_elem: int, n_elems: int, seed: int, threads: int | None = None) -> None:
    """Write bf16 pool elements [first_elem, first_elem+n_elems) to dst_ptr."""
    lib().tg_pool_fill(ctypes.c_void_p(dst_ptr), first_elem, n_elems, seed, threads or default_threads())


def pool_rows_np(w: Workload, rows: np.ndarray) -> np.ndarray:
    """Pool bytes of the given physical rows, regenerated: uint8 [len(rows)][row_bytes]."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    out = np.empty((rows.size, w.row_bytes), dtype=np.uint8)
    for i, r in enumerate(rows):
        pool_fill(out[i].ctypes.data, int(r) * w.W_KV, w.W_KV, w.pool_seed, 1)
    return out


def small_pool(w: Workload) -> np.ndarray:
    """Whole pool in ordinary memory (small workloads only): uint8 [pool_rows][row_bytes]."""
    out = np.empty((w.pool_rows, w.row_bytes), dtype=np.uint8)
    pool_fill(out.ctypes.data, 0, w.pool_rows * w.W_KV, w.pool_seed)
    return out
