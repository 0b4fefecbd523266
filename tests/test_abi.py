"""The C-ABI library loads on a machine without a GPU and exports every declared symbol."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "hisparse.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hisparse_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(os.path.join(ROOT, "hierarchical_kv_cache_resolve_amd", "libhisparse.so"))
    names = declared_functions()
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_footprint_identity_pure_function():
    import hierarchical_kv_cache_resolve_amd as hs
    # HBM = N_l * B * W_KV * s per request, no L_ctx term
    assert hs.hisparse_kv_bytes(16, 8, 4096, 576, hs.BF16) == 16 * 8 * 4096 * 576 * 2
    assert hs.hisparse_kv_bytes(64, 16, 4096, 2048, hs.BF16) == 64 * 16 * 4096 * 4096
    assert hs.hisparse_kv_bytes(1, 1, 512, 576, hs.FP8) == 512 * 576
    assert hs.hisparse_kv_bytes(1, 1, 512, 576, hs.FP32) == 512 * 576 * 4
    assert hs.hisparse_kv_bytes(0, 1, 512, 576, hs.BF16) == 0
    assert hs.hisparse_kv_bytes(1, 1, 512, 576, 9) == 0


def test_no_oracle_on_product_path():
    pkg = os.path.join(ROOT, "hierarchical_kv_cache_resolve_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp", ".c")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


def test_policy_library_exports_every_declared_symbol():
    src = open(os.path.join(ROOT, "include", "hspolicy.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = sorted(set(re.findall(r"\b(hs_policy_[a-z0-9_]+)\s*\(", src)))
    assert names == ["hs_policy_replay", "hs_policy_replay_many"]
    lib = ctypes.CDLL(os.path.join(ROOT, "hierarchical_kv_cache_resolve_amd", "libhspolicy.so"))
    assert all(hasattr(lib, n) for n in names)


def test_binding_refuses_tensors_the_kernels_would_overrun():
    import hierarchical_kv_cache_resolve_amd as hs
    import pytest
    import torch

    class FakeDev:
        is_cuda = True

        def __init__(self, n, size, contiguous=True):
            self.n, self.size, self.c = n, size, contiguous

        def is_contiguous(self):
            return self.c

        def element_size(self):
            return self.size

        def numel(self):
            return self.n

    hs._dev_arg(None, 100, 4, "x")                     # optional argument
    hs._dev_arg(12345, 100, 4, "x")                    # raw pointer: the caller's responsibility
    hs._dev_arg(FakeDev(25, 4), 100, 4, "x")
    with pytest.raises(ValueError):
        hs._dev_arg(torch.zeros(25, dtype=torch.int32), 100, 4, "x")     # host tensor
    with pytest.raises(ValueError):
        hs._dev_arg(FakeDev(24, 4), 100, 4, "x")        # too small
    with pytest.raises(ValueError):
        hs._dev_arg(FakeDev(50, 2), 100, 4, "x")        # wrong element size
    with pytest.raises(ValueError):
        hs._dev_arg(FakeDev(25, 4, contiguous=False), 100, 4, "x")


def test_binding_constants_match_the_header():
    """Every numeric HS_* constant of include/hisparse.h that the binding
    names has the header's value, and every option and probe constant is named."""
    import re
    hs = pytest.importorskip("hierarchical_kv_cache_resolve_amd")
    text = open(os.path.join(ROOT, "include", "hisparse.h")).read()
    defs = dict(re.findall(r"#define\s+(HS_[A-Z0-9_]+)\s+\(?(-?\d+)\)?", text))
    assert defs, "no constants parsed"
    for name, val in defs.items():
        if name.startswith(("HS_OPT_", "HS_PROBE_")):
            assert hasattr(hs, name), f"binding lacks {name}"
        if hasattr(hs, name):
            assert getattr(hs, name) == int(val), f"{name}: binding {getattr(hs, name)} != header {val}"
