"""The no-allocation attention entry point, through the C ABI, against the
allocating one: hisparse_attend_mla_noalloc must give exactly the outputs and
log-sum-exps of hisparse_attend_mla (the same kernels; only where the split-k
partials live differs), on two calls in a row with the second smaller, and
must refuse a call whose partials exceed its fixed area."""
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


def bf16_bits(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    u = x.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_noalloc_equals_allocating_entry_point(hs):
    w = tg.MLA.replace(name="noalloc", num_req=8, num_layers=2, L_ctx=40000, steps=2)
    print(f"[noalloc] R={w.num_req} k={w.k} B={w.B}", flush=True)
    tr = tg.trace(w)
    pool = make_pool(hs, w)
    res = make_resolver(hs, w, pool)
    dev = torch.device("cuda:0")
    sel = torch.from_numpy(tr).to(dev)
    slots = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
    for t in range(w.steps):
        for l in range(w.num_layers):
            res.resolve(l, sel[t, l], slots[l])
    torch.cuda.synchronize()
    assert res.error()[0] == 0
    rng = np.random.default_rng(17)
    stream = torch.cuda.current_stream().cuda_stream
    # the second call is smaller: fewer heads and fewer records
    for heads, k, layer in ((128, 2048, 0), (64, 512, 1)):
        print(f"[noalloc] heads={heads} k={k} layer={layer}", flush=True)
        q = torch.from_numpy(bf16_bits(rng, (w.num_req, heads, 576)).view(np.int16)).to(dev)
        idx = slots[layer][:, :k].contiguous()
        out_a = torch.full((w.num_req, heads, 512), float("nan"), dtype=torch.float32, device=dev)
        lse_a = torch.full((w.num_req, heads), float("nan"), dtype=torch.float32, device=dev)
        out_b, lse_b = out_a.clone(), lse_a.clone()
        res.attend_mla(layer, q, idx, 1.0 / 24.0, out_a, lse_a)
        rc = hs.hisparse_attend_mla_noalloc(res.h, layer, q.data_ptr(), heads, idx.data_ptr(), k, 1.0 / 24.0,
                                            out_b.data_ptr(), lse_b.data_ptr(), stream)
        assert rc == hs.HS_OK
        torch.cuda.synchronize()
        a, b = out_a.cpu().numpy(), out_b.cpu().numpy()
        assert np.all(np.isfinite(a)) and np.array_equal(a, b), f"outputs differ (heads {heads}, k {k})"
        assert np.array_equal(lse_a.cpu().numpy(), lse_b.cpu().numpy()), f"lse differs (heads {heads}, k {k})"
    # argument errors are those of the allocating entry point
    assert hs.hisparse_attend_mla_noalloc(res.h, 5, q.data_ptr(), 64, idx.data_ptr(), 512, 1.0, out_b.data_ptr(),
                                          0, stream) == hs.HS_E_LAYER
    assert hs.hisparse_attend_mla_noalloc(res.h, 0, q.data_ptr(), 96, idx.data_ptr(), 512, 1.0, out_b.data_ptr(),
                                          0, stream) == hs.HS_E_INVAL
    res.close()
    pool.free()


def test_noalloc_refuses_partials_beyond_its_area(hs):
    """64 requests x 1024 heads x k = 2048 needs 64 * 1024 * 258 floats' worth
    of partials (one chunk), more than the 64 MiB area: HS_E_SCRATCH, nothing
    launched, and the allocating entry point still takes the same call."""
    w = tg.MLA.replace(name="noalloc_big", num_req=64, num_layers=1, L_ctx=4096, B=2048, k=2048, steps=1)
    tr = tg.trace(w)
    pool = make_pool(hs, w)
    res = make_resolver(hs, w, pool)
    dev = torch.device("cuda:0")
    slots = torch.empty((w.num_req, w.k), dtype=torch.int32, device=dev)
    res.resolve(0, torch.from_numpy(tr[0, 0]).to(dev), slots)
    heads = 1024
    q = torch.zeros((w.num_req, heads, 576), dtype=torch.int16, device=dev)
    out = torch.empty((w.num_req, heads, 512), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    assert w.num_req * heads * 258 * 4 > hs.HS_SCRATCH_BYTES
    rc = hs.hisparse_attend_mla_noalloc(res.h, 0, q.data_ptr(), heads, slots.data_ptr(), w.k, 1.0,
                                        out.data_ptr(), 0, stream)
    assert rc == hs.HS_E_SCRATCH
    res.attend_mla(0, q, slots, 1.0, out)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(out.cpu().numpy()))
    res.close()
    pool.free()
