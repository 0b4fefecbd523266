"""Python binding of libhisparse.so (the MI355X RESOLVE library).

Argument marshalling only: every step of RESOLVE runs in the library's HIP
kernels.  The module-level functions carry the C names of include/hisparse.h;
``Resolver`` and ``HostPool`` are thin conveniences over them.  PyTorch is
used only for device tensors and streams.  If the library is not built this
module fails to import -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhisparse.so")

HS_OK = 0
HS_E_INVAL, HS_E_HANDLE, HS_E_LAYER, HS_E_K, HS_E_ALIGN = -1, -2, -3, -4, -5
HS_E_POOL, HS_E_NOMEM, HS_E_HIP, HS_E_DEVICE, HS_E_ORDER = -6, -7, -8, -9, -10
HS_E_SCRATCH = -11
HS_SCRATCH_BYTES = 64 << 20
HS_DEV_RANGE, HS_DEV_DUP, HS_DEV_NOT_RESIDENT, HS_DEV_DIVERGED, HS_DEV_FULL = 1, 2, 3, 4, 5
HS_MAX_B, HS_MAX_K, HS_MAX_REQ = 16384, 4096, 1024
BF16, FP16, FP8, FP32 = 0, 1, 2, 3
ELEM_BYTES = {BF16: 2, FP16: 2, FP8: 1, FP32: 4}
HS_OPT_FETCH_BLOCKS, HS_OPT_FETCH_UNROLL, HS_OPT_TIMING, HS_OPT_NT_LOADS, HS_OPT_PHASE_TRACE, HS_OPT_PROBE = 1, 2, 3, 4, 5, 6
HS_OPT_ATTN_HEADS = 7
HS_OPT_META_LANES = 8
HS_OPT_META_WGS, HS_MAX_META_WGS = 9, 64
HS_OPT_MARKERS = 10
HS_OPT_PREFETCH_BLOCKS = 11
HS_PROBE_PAGE_TABLE, HS_PROBE_SLOT_SCAN, HS_PROBE_SLOT_SCAN_HASH = 0, 1, 2

_ERR_NAMES = {v: k for k, v in dict(HS_E_INVAL=-1, HS_E_HANDLE=-2, HS_E_LAYER=-3, HS_E_K=-4, HS_E_ALIGN=-5,
                                     HS_E_POOL=-6, HS_E_NOMEM=-7, HS_E_HIP=-8, HS_E_DEVICE=-9,
                                     HS_E_ORDER=-10, HS_E_SCRATCH=-11).items()}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (no fallback path exists)")

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t


class hs_host_pool(ctypes.Structure):
    _fields_ = [("base", _vp), ("pool_rows", _i64), ("L_ctx", _i64), ("region_row", _vp)]


class hs_layer_state(ctypes.Structure):
    _fields_ = [("d_cache", _vp), ("d_slot_pos", _vp), ("d_ts", _vp), ("d_page_table", _vp), ("d_clock", _vp),
                ("d_plan", _vp), ("d_miss_count", _vp), ("d_hit_mask", _vp), ("row_bytes", _i64), ("B", _i32),
                ("num_req", _i32), ("L_ctx", _i64)]


class hs_stats(ctypes.Structure):
    _fields_ = [("hits", ctypes.c_uint64), ("misses", ctypes.c_uint64), ("miss_bytes", ctypes.c_uint64),
                ("resolves", ctypes.c_uint64)]


class hs_timing(ctypes.Structure):
    _fields_ = [("plan_ms", ctypes.c_double), ("fetch_ms", ctypes.c_double), ("replay_ms", ctypes.c_double),
                ("publish_ms", ctypes.c_double), ("plan_launches", _i64), ("fetch_launches", _i64),
                ("replay_launches", _i64), ("publish_launches", _i64), ("dropped", _i64)]


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_sig("hisparse_create", _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(hs_host_pool), ctypes.POINTER(_vp))
_sig("hisparse_resolve", _i32, _vp, _i32, _vp, _i32, _vp, _vp)
_sig("hisparse_resolve_layers", _i32, _vp, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_vp), _i32,
     ctypes.POINTER(_vp), _vp)
_sig("hisparse_prefetch", _i32, _vp, _i32, ctypes.POINTER(_i32), _i32, _vp)
_sig("hisparse_destroy", _i32, _vp)
_sig("hisparse_append", _i32, _vp, _i32, _vp, _vp)
_sig("hisparse_set_lengths", _i32, _vp, _vp)
_sig("hisparse_get_lengths", _i32, _vp, _vp)
_sig("hisparse_kv_bytes", _sz, _i32, _i32, _i32, _i32, _i32)
_sig("hisparse_hbm_bytes", _sz, _vp)
_sig("hisparse_meta_bytes", _sz, _vp)
_sig("hisparse_layer_state", _i32, _vp, _i32, ctypes.POINTER(hs_layer_state))
_sig("hisparse_get_error", _i32, _vp, ctypes.POINTER(_i32), ctypes.POINTER(_i32), ctypes.POINTER(_i32))
_sig("hisparse_clear_error", _i32, _vp)
_sig("hisparse_stats", _i32, _vp, _i32, ctypes.POINTER(hs_stats))
_sig("hisparse_reset", _i32, _vp)
_sig("hisparse_set_option", _i32, _vp, _i32, _i64)
_sig("hisparse_timing", _i32, _vp, ctypes.POINTER(hs_timing), _i32)
_sig("hisparse_memcpy_d2h", _i32, _vp, _vp, _sz)
_sig("hisparse_phase_trace", _i32, _vp, _i32, _vp, ctypes.POINTER(ctypes.c_double))
_sig("hisparse_host_alloc", _i32, _sz, _i32, ctypes.POINTER(_vp))
_sig("hisparse_host_free", _i32, _vp)
_sig("hisparse_gather_checksum", _i32, _vp, _i32, _vp, _i32, _vp, _vp)
_sig("hisparse_attend_mla", _i32, _vp, _i32, _vp, _i32, _vp, _i32, ctypes.c_float, _vp, _vp, _vp)
_sig("hisparse_attend_mla_noalloc", _i32, _vp, _i32, _vp, _i32, _vp, _i32, ctypes.c_float, _vp, _vp, _vp)
for _n in ("hisparse_probe_link_sdma", "hisparse_probe_link_kernel", "hisparse_probe_hbm"):
    _sig(_n, _i32, _vp, _vp, _sz, _i32, _vp, ctypes.POINTER(ctypes.c_double))


class HisparseError(RuntimeError):
    def __init__(self, fn, rc):
        super().__init__(f"{fn} returned {rc} ({_ERR_NAMES.get(rc, 'unknown')})")
        self.rc = rc


def _check(fn, rc):
    if rc != HS_OK:
        raise HisparseError(fn, rc)
    return rc


def _ptr(x) -> int:
    """Device or host address of a torch tensor, numpy array or int."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _stream(s) -> int:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


# ---- functions with the C names (raw pointers / handles) -------------------

def hisparse_create(num_req, num_layers, B, W_KV, dtype, pool: hs_host_pool) -> int:
    h = _vp()
    _check("hisparse_create", _lib.hisparse_create(num_req, num_layers, B, W_KV, dtype, ctypes.byref(pool),
                                                   ctypes.byref(h)))
    return h.value


def hisparse_resolve(h, layer, d_sel, k, d_slot_idx, stream) -> int:
    return _lib.hisparse_resolve(h, layer, d_sel, k, d_slot_idx, stream)


def hisparse_resolve_layers(h, layers, d_sels, k, d_outs, stream) -> int:
    n = len(layers)
    return _lib.hisparse_resolve_layers(h, n, (_i32 * n)(*layers), (_vp * n)(*d_sels), k, (_vp * n)(*d_outs),
                                        stream)


def hisparse_prefetch(h, anchor, shared, side_stream) -> int:
    n = len(shared)
    return _lib.hisparse_prefetch(h, anchor, (_i32 * n)(*shared), n, side_stream)


def hisparse_destroy(h) -> int:
    return _lib.hisparse_destroy(h)


def hisparse_append(h, layer, d_rows, stream) -> int:
    return _lib.hisparse_append(h, layer, d_rows, stream)


def hisparse_set_lengths(h, lengths) -> int:
    a = np.ascontiguousarray(lengths, dtype=np.int64)
    return _check("hisparse_set_lengths", _lib.hisparse_set_lengths(h, a.ctypes.data))


def hisparse_get_lengths(h, n) -> np.ndarray:
    a = np.empty(n, dtype=np.int64)
    _check("hisparse_get_lengths", _lib.hisparse_get_lengths(h, a.ctypes.data))
    return a


def hisparse_kv_bytes(num_req, num_layers, B, W_KV, dtype) -> int:
    return int(_lib.hisparse_kv_bytes(num_req, num_layers, B, W_KV, dtype))


def hisparse_hbm_bytes(h) -> int:
    return int(_lib.hisparse_hbm_bytes(h))


def hisparse_meta_bytes(h) -> int:
    return int(_lib.hisparse_meta_bytes(h))


def hisparse_layer_state(h, layer) -> hs_layer_state:
    st = hs_layer_state()
    _check("hisparse_layer_state", _lib.hisparse_layer_state(h, layer, ctypes.byref(st)))
    return st


def hisparse_get_error(h):
    c, l, r = _i32(), _i32(), _i32()
    _check("hisparse_get_error", _lib.hisparse_get_error(h, ctypes.byref(c), ctypes.byref(l), ctypes.byref(r)))
    return c.value, l.value, r.value


def hisparse_clear_error(h) -> int:
    return _check("hisparse_clear_error", _lib.hisparse_clear_error(h))


def hisparse_stats(h, layer=-1) -> hs_stats:
    st = hs_stats()
    _check("hisparse_stats", _lib.hisparse_stats(h, layer, ctypes.byref(st)))
    return st


def hisparse_reset(h) -> int:
    return _check("hisparse_reset", _lib.hisparse_reset(h))


def hisparse_set_option(h, key, value) -> int:
    return _check("hisparse_set_option", _lib.hisparse_set_option(h, key, value))


def hisparse_timing(h, clear=False) -> hs_timing:
    t = hs_timing()
    _check("hisparse_timing", _lib.hisparse_timing(h, ctypes.byref(t), 1 if clear else 0))
    return t


def hisparse_phase_trace(h, layer, num_req):
    """Raw phase stamps [num_req][16] of the last metadata launch and the tick period in ns."""
    out = np.zeros((num_req, 16), dtype=np.uint64)
    ns = ctypes.c_double()
    _check("hisparse_phase_trace", _lib.hisparse_phase_trace(h, layer, out.ctypes.data, ctypes.byref(ns)))
    return out, ns.value


def hisparse_memcpy_d2h(dst, d_src, nbytes) -> int:
    return _check("hisparse_memcpy_d2h", _lib.hisparse_memcpy_d2h(dst, d_src, nbytes))


def hisparse_host_alloc(nbytes, coherent=False) -> int:
    p = _vp()
    _check("hisparse_host_alloc", _lib.hisparse_host_alloc(nbytes, 1 if coherent else 0, ctypes.byref(p)))
    return p.value


def hisparse_host_free(p) -> int:
    return _check("hisparse_host_free", _lib.hisparse_host_free(p))


def hisparse_gather_checksum(h, layer, d_slot_idx, k, d_out, stream) -> int:
    return _lib.hisparse_gather_checksum(h, layer, d_slot_idx, k, d_out, stream)


def hisparse_attend_mla(h, layer, d_q, num_heads, d_slot_idx, k, scale, d_out, d_lse, stream) -> int:
    return _lib.hisparse_attend_mla(h, layer, d_q, num_heads, d_slot_idx, k, scale, d_out, d_lse, stream)


def hisparse_attend_mla_noalloc(h, layer, d_q, num_heads, d_slot_idx, k, scale, d_out, d_lse, stream) -> int:
    return _lib.hisparse_attend_mla_noalloc(h, layer, d_q, num_heads, d_slot_idx, k, scale, d_out, d_lse, stream)


def _probe(name, src, dst, nbytes, iters, stream):
    g = ctypes.c_double()
    _check(name, getattr(_lib, name)(src, dst, nbytes, iters, stream, ctypes.byref(g)))
    return g.value


def hisparse_probe_link_sdma(host_src, d_dst, nbytes, iters, stream) -> float:
    return _probe("hisparse_probe_link_sdma", host_src, d_dst, nbytes, iters, stream)


def hisparse_probe_link_kernel(host_src, d_dst, nbytes, iters, stream) -> float:
    return _probe("hisparse_probe_link_kernel", host_src, d_dst, nbytes, iters, stream)


def hisparse_probe_hbm(d_src, d_dst, nbytes, iters, stream) -> float:
    return _probe("hisparse_probe_hbm", d_src, d_dst, nbytes, iters, stream)


# ---- conveniences -----------------------------------------------------------

class HostPool:
    """Pinned, device-readable host memory holding the authoritative KV pool."""

    def __init__(self, ptr: int, nbytes: int):
        self.ptr, self.nbytes = ptr, nbytes

    @classmethod
    def allocate(cls, nbytes: int, coherent: bool = False) -> "HostPool":
        return cls(hisparse_host_alloc(nbytes, coherent), nbytes)

    def numpy_view(self) -> np.ndarray:
        buf = (ctypes.c_uint8 * self.nbytes).from_address(self.ptr)
        return np.frombuffer(buf, dtype=np.uint8)

    def free(self):
        if self.ptr:
            hisparse_host_free(self.ptr)
            self.ptr = 0


def _dev_arg(t, nbytes, itemsize, name):
    """Refuse a device tensor that the kernels would index out of bounds: it
    must be a contiguous GPU tensor of the element size the call expects and
    hold at least nbytes."""
    if t is None or isinstance(t, int):
        return                                           # raw pointers are the caller's responsibility
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name}: expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if itemsize and t.element_size() != itemsize:
        raise ValueError(f"{name}: expected {itemsize}-byte elements, got {t.element_size()}")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, need {nbytes}")


class Resolver:
    """One handle: num_req x num_layers GPU caches of B slots over a host pool."""

    def __init__(self, num_req, num_layers, B, W_KV, dtype, pool: HostPool, L_ctx, pool_rows, region_row=None):
        self._region = None if region_row is None else np.ascontiguousarray(region_row, dtype=np.int64)
        desc = hs_host_pool(pool.ptr, int(pool_rows), int(L_ctx),
                            self._region.ctypes.data if self._region is not None else None)
        self.h = hisparse_create(num_req, num_layers, B, W_KV, dtype, desc)
        self.num_req, self.num_layers, self.B, self.L_ctx = num_req, num_layers, B, L_ctx
        self.row_bytes = W_KV * ELEM_BYTES[dtype]

    def close(self):
        if self.h:
            _check("hisparse_destroy", hisparse_destroy(self.h))
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def resolve(self, layer, sel, out, stream=None):
        k = int(sel.shape[-1])
        _dev_arg(sel, 4 * self.num_req * k, 4, "sel")
        _dev_arg(out, 4 * self.num_req * k, 4, "out")
        _check("hisparse_resolve", hisparse_resolve(self.h, layer, _ptr(sel), k, _ptr(out), _stream(stream)))

    def resolve_layers(self, layers, sels, outs, stream=None):
        if not (len(layers) == len(sels) == len(outs)) or len(layers) == 0:
            raise ValueError(f"resolve_layers: {len(layers)} layers, {len(sels)} selections, {len(outs)} outputs")
        k = int(sels[0].shape[-1])
        for s_, o_ in zip(sels, outs):
            _dev_arg(s_, 4 * self.num_req * k, 4, "sel")
            _dev_arg(o_, 4 * self.num_req * k, 4, "out")
        _check("hisparse_resolve_layers", hisparse_resolve_layers(
            self.h, list(layers), [_ptr(s) for s in sels], k, [_ptr(o) for o in outs], _stream(stream)))

    def prefetch(self, anchor, shared, side_stream):
        _check("hisparse_prefetch", hisparse_prefetch(self.h, anchor, list(shared), _stream(side_stream)))

    def set_option(self, key, value):
        hisparse_set_option(self.h, key, value)

    def append(self, layer, rows, stream=None):
        """rows: device tensor [num_req][row_bytes] (any dtype of that byte size)."""
        _dev_arg(rows, self.num_req * self.row_bytes, 0, "rows")
        _check("hisparse_append", hisparse_append(self.h, layer, _ptr(rows), _stream(stream)))

    def set_lengths(self, lengths):
        """lengths [num_req][num_layers] (or flat, index r*num_layers + l)."""
        hisparse_set_lengths(self.h, np.asarray(lengths).reshape(-1))

    def lengths(self):
        return hisparse_get_lengths(self.h, self.num_req * self.num_layers).reshape(self.num_req, self.num_layers)

    def timing(self, clear=False):
        return hisparse_timing(self.h, clear)

    def stats(self, layer=-1):
        return hisparse_stats(self.h, layer)

    def reset(self):
        hisparse_reset(self.h)

    def hbm_bytes(self):
        return hisparse_hbm_bytes(self.h)

    def error(self):
        return hisparse_get_error(self.h)

    def clear_error(self):
        hisparse_clear_error(self.h)

    def check_error(self):
        code, layer, req = self.error()
        if code:
            raise HisparseError(f"device error code {code} at layer {layer} request {req}", HS_E_DEVICE)

    def gather_checksum(self, layer, slot_idx, out, stream=None):
        _dev_arg(slot_idx, 4 * self.num_req * int(slot_idx.shape[-1]), 4, "slot_idx")
        _dev_arg(out, 8 * self.num_req, 8, "out")
        _check("hisparse_gather_checksum", hisparse_gather_checksum(
            self.h, layer, _ptr(slot_idx), int(slot_idx.shape[-1]), _ptr(out), _stream(stream)))

    def attend_mla(self, layer, q, slot_idx, scale, out, lse=None, stream=None):
        """q: bf16 device tensor [num_req][H][576]; out fp32 [num_req][H][512]; lse fp32 [num_req][H] or None."""
        R, H, k = self.num_req, int(q.shape[1]), int(slot_idx.shape[-1])
        _dev_arg(q, 2 * R * H * 576, 2, "q")
        _dev_arg(slot_idx, 4 * R * k, 4, "slot_idx")
        _dev_arg(out, 4 * R * H * 512, 4, "out")
        _dev_arg(lse, 4 * R * H, 4, "lse")
        _check("hisparse_attend_mla", hisparse_attend_mla(
            self.h, layer, _ptr(q), int(q.shape[1]), _ptr(slot_idx), int(slot_idx.shape[-1]), float(scale),
            _ptr(out), _ptr(lse), _stream(stream)))

    def _d2h(self, dptr, dtype, shape):
        a = np.empty(shape, dtype=dtype)
        hisparse_memcpy_d2h(a.ctypes.data, dptr, a.nbytes)
        return a

    def state(self, layer, page_table=True):
        """Host copies of one layer's state (synchronises the device)."""
        st = hisparse_layer_state(self.h, layer)
        R, B = self.num_req, self.B
        out = dict(
            slot_pos=self._d2h(st.d_slot_pos, np.int32, (R, B)),
            ts=self._d2h(st.d_ts, np.uint32, (R, B)),
            clock=self._d2h(st.d_clock, np.uint32, (R,)),
            plan=self._d2h(st.d_plan, np.int32, (R, B, 4)),
            miss_count=self._d2h(st.d_miss_count, np.int32, (R,)),
            hit_mask=self._d2h(st.d_hit_mask, np.uint8, (R, B)),
        )
        if page_table:
            out["page_table"] = self._d2h(st.d_page_table, np.int32, (R, self.L_ctx))
        return out

    def cache_rows(self, layer, req):
        """Host copy of one (request, layer) cache: uint8 [B][row_bytes]."""
        st = hisparse_layer_state(self.h, layer)
        base = st.d_cache + req * self.B * self.row_bytes
        return self._d2h(base, np.uint8, (self.B, self.row_bytes))

    def cache_layer(self, layer):
        st = hisparse_layer_state(self.h, layer)
        return self._d2h(st.d_cache, np.uint8, (self.num_req, self.B, self.row_bytes))
