"""The CPU-side C code (the oracle and the seeded input generators) run under
AddressSanitizer and UndefinedBehaviorSanitizer: both are rebuilt with
-fsanitize=address,undefined in a temporary directory and exercised in a
child process that preloads the sanitizer runtimes (the interpreter itself is
not instrumented).  Any report aborts the child, which fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import numpy as np
import oracle, tracegen
oracle._LIB_PATH = {oracle_so!r}; oracle._lib = None
tracegen._LIB_PATH = {tracegen_so!r}; tracegen._lib = None
import tracegen as tg
from oracle import Oracle
# generators: a short locality trace, a uniform trace and a pool fill
w = tg.TINY.replace(steps=12)
tr = tg.trace(w)
tu = tg.trace(tg.NOLOCALITY.replace(num_req=2, num_layers=1, steps=3))
pool = np.zeros(w.pool_rows * w.row_bytes, np.uint8)
tg.pool_fill(pool.ctypes.data, 0, w.pool_rows * w.W_KV, w.pool_seed)
# oracle: the tiny workload with bytes, then the pins that drive it hardest
o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes)
for t in range(w.steps):
    o.resolve(0, tr[t, 0], pool)
o.close()
from test_oracle_pins import test_golden_walkthrough
test_golden_walkthrough()
from test_bruteforce import sampled
ok, info = sampled(Oracle, n_seq=200, seed=11)
assert ok, info
from test_oracle_properties import test_oracle_properties
test_oracle_properties()
print("sanitized run ok")
"""


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_and_generators_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("sanitizer runtimes not installed")
    flags = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
             "-shared", "-fPIC"]
    oracle_so, tracegen_so = str(tmp_path / "liboracle_san.so"), str(tmp_path / "libtracegen_san.so")
    subprocess.run(["gcc", *flags, "-std=c11", "-o", oracle_so, os.path.join(ROOT, "oracle", "oracle.c")], check=True)
    subprocess.run(["gcc", *flags, "-std=gnu11", "-o", tracegen_so, os.path.join(ROOT, "tracegen", "tracegen.c"),
                    "-lm", "-lpthread"], check=True)
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}", ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), oracle_so=oracle_so, tracegen_so=tracegen_so)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "sanitized run ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
