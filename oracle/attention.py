"""Sparse MLA decode attention over the selected records, in float64 -- TEST INFRASTRUCTURE ONLY.

The consumer that RESOLVE serves: sparse attention reads exactly the k
selected KV records of each request and layer and computes ordinary
attention over them; placement does not change the math (blog "Inference
Systems Infrastructure Notes (6): HiSparse", section 5 "Exact"; pith
"Core claim").  For an MLA-style latent record (576 bf16 elements: a
512-element compressed KV followed by a 64-element rotary key) the absorbed
decode form is used: the query of each head is already projected into the
576-element record space, scores are dot products with whole records, and
the values are the first 512 elements of the same records (the published
MLA decode formulation).

    s[h, j] = scale * sum_d q[h, d] * rec_j[d]             d < 576
    p[h, j] = exp(s[h, j] - max_j s[h, j]) / sum_j exp(...)
    out[h, d] = sum_j p[h, j] * rec_j[d]                   d < 512
    lse[h] = max_j s[h, j] + log(sum_j exp(s[h, j] - max_j s[h, j]))

Inputs are bf16 bit patterns (uint16); everything is computed in float64.
"""
from __future__ import annotations

import numpy as np

D_QK = 576
D_V = 512


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def mla_decode(q_bits: np.ndarray, rec_bits: np.ndarray, scale: float):
    """q_bits [R][H][576] uint16, rec_bits [R][k][576] uint16 -> (out [R][H][512], lse [R][H]) float64."""
    q = bf16_to_f64(q_bits)
    rec = bf16_to_f64(rec_bits)
    s = np.matmul(q, np.swapaxes(rec, 1, 2)) * scale          # [R][H][k]
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    out = np.matmul(e / z, rec[:, :, :D_V])                   # [R][H][512]
    lse = (m + np.log(z))[..., 0]
    return out, lse


def error_bound(q_bits: np.ndarray, rec_bits: np.ndarray, scale: float) -> np.ndarray:
    """Per-element bound for a kernel that forms scores in float32 from bf16
    inputs, keeps softmax in float32, rounds the probabilities to bf16
    before the value product (relative error at most 2^-9 each) and may
    round partial outputs over subsets of the records, each normalised by
    its own sum, to fp16 (relative 2^-11, of a value bounded by that subset's
    sum_j p_j |rec_j[d]| / sum_j p_j):
        |err[h, d]| <= 2^-8 * sum_j p[h, j] * |rec_j[d]| + 1e-6
    (2^-9 + 2^-11 of the same sum leave a quarter of the 2^-8 for the float32
    score, exponent and normalisation errors, which for scores of a few units
    are near 1e-5 relative; the 1e-6 covers fp16 subnormal spacing)."""
    q = bf16_to_f64(q_bits)
    rec = bf16_to_f64(rec_bits)
    s = np.matmul(q, np.swapaxes(rec, 1, 2)) * scale
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    p = e / e.sum(axis=-1, keepdims=True)
    return 2.0 ** -8 * np.matmul(p, np.abs(rec[:, :, :D_V])) + 1e-6
