"""The peak probes that every reported fraction is taken against: each
reports a positive, finite rate, the two copy kernels deliver exactly the
bytes they claim to move (host pool -> HBM, HBM -> HBM), and sizes that are
not whole 16-byte pieces are refused."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def hs():
    import hierarchical_kv_cache_resolve_amd as m
    return m


def test_peak_probes_move_the_bytes_they_time(hs):
    nbytes = 64 << 20
    host = hs.HostPool.allocate(nbytes)
    hv = host.numpy_view()
    hv[:] = np.random.default_rng(5).integers(0, 256, nbytes, dtype=np.uint8)
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    try:
        print("[probes] link kernel, link sdma, hbm over 64 MiB", flush=True)
        a.zero_()
        torch.cuda.synchronize()
        g = hs.hisparse_probe_link_kernel(host.ptr, a.data_ptr(), nbytes, 2, s)
        assert math.isfinite(g) and g > 0
        assert np.array_equal(a.cpu().numpy(), hv)
        a.zero_()
        torch.cuda.synchronize()
        g = hs.hisparse_probe_link_sdma(host.ptr, a.data_ptr(), nbytes, 2, s)
        assert math.isfinite(g) and g > 0
        assert np.array_equal(a.cpu().numpy(), hv)
        b.zero_()
        torch.cuda.synchronize()
        g = hs.hisparse_probe_hbm(a.data_ptr(), b.data_ptr(), nbytes, 2, s)
        assert math.isfinite(g) and g > 0
        assert torch.equal(a, b)
        for bad in (15, 0):
            with pytest.raises(hs.HisparseError):
                hs.hisparse_probe_hbm(a.data_ptr(), b.data_ptr(), bad, 1, s)
    finally:
        host.free()
