"""CPU oracle of the HiSparse RESOLVE step -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding)
never does.  The arithmetic lives in ``oracle.c`` (plain single-threaded C,
built with gcc); this module only marshals numpy arrays through ctypes.

Parity pins (what ties the oracle to something other than itself) are in
``tests/test_oracle_pins.py``, ``tests/test_bruteforce.py`` and the hand
derived fixtures under ``tests/golden/``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

E_OK, E_RANGE, E_DUP, E_K, E_FULL = 0, 1, 2, 3, 4

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    vp = ctypes.c_void_p
    lib.oracle_create.restype = vp
    lib.oracle_create.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int]
    lib.oracle_destroy.restype = None
    lib.oracle_destroy.argtypes = [vp]
    lib.oracle_reset.restype = None
    lib.oracle_reset.argtypes = [vp]
    for name in ("oracle_slot_pos", "oracle_ts", "oracle_page_table", "oracle_clock", "oracle_cache"):
        getattr(lib, name).restype = vp
        getattr(lib, name).argtypes = [vp]
    lib.oracle_length.restype = vp
    lib.oracle_length.argtypes = [vp]
    lib.oracle_set_length.restype = ctypes.c_int
    lib.oracle_set_length.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int64]
    lib.oracle_append.restype = ctypes.c_int
    lib.oracle_append.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp]
    lib.oracle_resolve.restype = ctypes.c_int
    lib.oracle_resolve.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]
    _lib = lib
    return lib


def _view(ptr, dtype, shape):
    n = int(np.prod(shape))
    if n == 0:
        return np.zeros(shape, dtype=dtype)
    buf = (ctypes.c_byte * (n * np.dtype(dtype).itemsize)).from_address(ptr)
    return np.frombuffer(buf, dtype=dtype).reshape(shape)


class Oracle:
    """State for num_req x num_layers (request, layer) caches of B slots."""

    def __init__(self, num_req, num_layers, B, L_ctx, row_bytes, model_bytes=True):
        self.lib = _load()
        self.num_req, self.num_layers, self.B, self.L_ctx = num_req, num_layers, B, L_ctx
        self.row_bytes = row_bytes
        self.h = self.lib.oracle_create(num_req, num_layers, B, L_ctx, row_bytes, 1 if model_bytes else 0)
        if not self.h:
            raise MemoryError("oracle_create failed")
        nl, nr = num_layers, num_req
        self.slot_pos = _view(self.lib.oracle_slot_pos(self.h), np.int32, (nl, nr, B))
        self.ts = _view(self.lib.oracle_ts(self.h), np.uint32, (nl, nr, B))
        self.page_table = _view(self.lib.oracle_page_table(self.h), np.int32, (nl, nr, L_ctx))
        self.clock = _view(self.lib.oracle_clock(self.h), np.uint32, (nl, nr))
        self.length = _view(self.lib.oracle_length(self.h), np.int64, (nl, nr))
        self.cache = (_view(self.lib.oracle_cache(self.h), np.uint8, (nl, nr, B, row_bytes))
                      if model_bytes else None)

    def close(self):
        if self.h:
            self.lib.oracle_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self):
        self.lib.oracle_reset(self.h)

    def set_lengths(self, lengths):
        """lengths [num_req][num_layers]: set every history's length (cached
        positions at or past a lowered length leave the cache)."""
        lengths = np.asarray(lengths, dtype=np.int64).reshape(self.num_req, self.num_layers)
        for r in range(self.num_req):
            for l in range(self.num_layers):
                if self.lib.oracle_set_length(self.h, l, r, int(lengths[r, l])) != E_OK:
                    raise ValueError(f"length {lengths[r, l]} outside [0, {self.L_ctx}]")

    def append(self, layer, rows, pool, region_row=None):
        """rows: uint8 [num_req][row_bytes]; pool: writable uint8 array holding the host pool."""
        rows = np.ascontiguousarray(rows, dtype=np.uint8)
        assert rows.shape == (self.num_req, self.row_bytes)
        err = np.empty(self.num_req, np.int32)
        rr = None
        if region_row is not None:
            region_row = np.ascontiguousarray(region_row, dtype=np.int64)
            rr = region_row.ctypes.data
        self.lib.oracle_append(self.h, layer, rows.ctypes.data, pool.ctypes.data, rr, err.ctypes.data)
        return err

    def resolve(self, layer, sel, pool=None, region_row=None):
        """sel: int32 [num_req][k].  Returns dict of slot_idx, hit_mask, miss_count, plan, err."""
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        nr, k = sel.shape
        assert nr == self.num_req
        slot_idx = np.empty((nr, k), np.int32)
        hit_mask = np.empty((nr, k), np.uint8)
        miss_count = np.empty(nr, np.int32)
        plan = np.full((nr, k, 4), -2, np.int32)
        err = np.empty(nr, np.int32)
        pool_ptr = None
        if pool is not None:
            pool_ptr = pool.ctypes.data if isinstance(pool, np.ndarray) else int(pool)
        rr = None
        if region_row is not None:
            region_row = np.ascontiguousarray(region_row, dtype=np.int64)
            rr = region_row.ctypes.data
        self.lib.oracle_resolve(self.h, layer, sel.ctypes.data, k, pool_ptr, rr, slot_idx.ctypes.data,
                                hit_mask.ctypes.data, miss_count.ctypes.data, plan.ctypes.data, err.ctypes.data)
        return dict(slot_idx=slot_idx, hit_mask=hit_mask, miss_count=miss_count, plan=plan, err=err)
