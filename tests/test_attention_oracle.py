"""Pins of the float64 sparse MLA decode attention used to check the consumer kernel."""
import math

import numpy as np

from oracle.attention import D_QK, D_V, bf16_to_f64, mla_decode


def rand_bits(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    u = x.view(np.uint32)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16       # round to nearest even
    return u.astype(np.uint16)


def test_bf16_decode_exact():
    assert bf16_to_f64(np.array([0x3F80, 0xBF80, 0x4000, 0x0000], np.uint16)).tolist() == [1.0, -1.0, 2.0, 0.0]


def test_single_record_returns_its_values():
    rng = np.random.default_rng(1)
    q, rec = rand_bits(rng, (2, 3, D_QK)), rand_bits(rng, (2, 1, D_QK))
    out, lse = mla_decode(q, rec, 0.1)
    assert np.array_equal(out, np.broadcast_to(bf16_to_f64(rec)[:, :, :D_V], out.shape))
    s = (bf16_to_f64(q) * bf16_to_f64(rec)).sum(-1) * 0.1
    assert np.allclose(lse, s, rtol=0, atol=1e-12)


def test_zero_query_averages_values():
    rng = np.random.default_rng(2)
    rec = rand_bits(rng, (1, 37, D_QK))
    out, lse = mla_decode(np.zeros((1, 4, D_QK), np.uint16), rec, 0.05)
    mean = bf16_to_f64(rec)[0, :, :D_V].mean(axis=0)
    assert np.allclose(out[0], mean[None, :], rtol=0, atol=1e-13)
    assert np.allclose(lse, math.log(37), atol=1e-13)


def test_matches_explicit_loops_and_is_order_free():
    rng = np.random.default_rng(3)
    R, H, k = 2, 2, 9
    q, rec = rand_bits(rng, (R, H, D_QK)), rand_bits(rng, (R, k, D_QK))
    out, lse = mla_decode(q, rec, 0.07)
    qf, rf = bf16_to_f64(q), bf16_to_f64(rec)
    for r in range(R):
        for h in range(H):
            sc = [0.07 * sum(qf[r, h, d] * rf[r, j, d] for d in range(D_QK)) for j in range(k)]
            mx = max(sc)
            w = [math.exp(v - mx) for v in sc]
            z = sum(w)
            for d in (0, 1, 255, 511):
                ref = sum(w[j] * rf[r, j, d] for j in range(k)) / z
                assert abs(out[r, h, d] - ref) < 1e-12
            assert abs(lse[r, h] - (mx + math.log(z))) < 1e-12
    perm = rng.permutation(k)
    out2, lse2 = mla_decode(q, rec[:, perm], 0.07)
    assert np.allclose(out2, out, rtol=0, atol=1e-12) and np.allclose(lse2, lse, atol=1e-12)
