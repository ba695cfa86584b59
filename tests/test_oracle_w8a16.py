"""Pins for the oracle's weight-only block-FP8 GEMM (CPU only).

Pins: exact rational brute force on small shapes and at sampled positions;
a closed form (unit weights, unit scales: row sums of the activation, taken
with math.fsum); agreement with the W8A8 oracle when the activation is a
dequantised FP8 tensor with power-of-two scales (a special case both
formulas must give identically); block locality of the weight scales.
"""

import math

import numpy as np
import pytest

from oracle import e4m3_decode, gemm_ref, gemm_w8a16_ref, gemm_w8a16_ref_at
from exact import gemm_w8a16_exact
import workloads


def _bf16_values(m, k, seed):
    """bf16-representable activation values: N(0,1) with a few large and tiny
    magnitudes, rounded to bf16 through torch."""
    import torch
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[rng.random((m, k)) < 0.02] *= 300.0
    x[rng.random((m, k)) < 0.02] *= 1e-4
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


def _sum_abs_terms(a, w_q, w_s):
    w = np.abs(e4m3_decode(w_q) * np.repeat(np.repeat(w_s.astype(np.float64), 128, axis=0)[: w_q.shape[0]], 128, axis=1))
    return np.abs(a.astype(np.float64)) @ w.T


@pytest.mark.parametrize("m,n,k,seed", [(1, 128, 128, 1), (2, 130, 256, 2), (3, 5, 384, 3)])
def test_w8a16_ref_exact_brute_force(m, n, k, seed):
    a = _bf16_values(m, k, seed)
    w_q = workloads.random_codes((n, k), seed + 1)
    w_s = workloads.random_scales((-(-n // 128), k // 128), seed + 2)
    got = gemm_w8a16_ref(a, w_q, w_s)
    exact = np.array([float(v) for v in gemm_w8a16_exact(a, w_q, w_s)]).reshape(m, n)
    assert np.all(np.abs(got - exact) <= 2.0 ** -50 * _sum_abs_terms(a, w_q, w_s))


def test_w8a16_ref_at_matches_brute_force():
    m, n, k = 4, 300, 256
    a = _bf16_values(m, k, 11)
    w_q = workloads.random_codes((n, k), 12)
    w_s = workloads.random_scales((-(-n // 128), k // 128), 13)
    rng = np.random.default_rng(0)
    rows, cols = rng.integers(0, m, 30), rng.integers(0, n, 30)
    got = gemm_w8a16_ref_at(a, w_q, w_s, rows, cols)
    exact = np.array([float(v) for v in gemm_w8a16_exact(a, w_q, w_s, rows, cols)])
    bound = 2.0 ** -50 * _sum_abs_terms(a, w_q, w_s)[rows, cols]
    assert np.all(np.abs(got - exact) <= bound)


def test_w8a16_ref_unit_weights_give_row_sums():
    m, n, k = 3, 200, 512
    a = _bf16_values(m, k, 21)
    w_q = np.full((n, k), 0x38, dtype=np.uint8)  # e4m3fn 1.0
    w_s = np.ones((-(-n // 128), k // 128), dtype=np.float32)
    got = gemm_w8a16_ref(a, w_q, w_s)
    for i in range(m):
        row = math.fsum(float(v) for v in a[i])
        tol = 2.0 ** -50 * float(np.sum(np.abs(a[i], dtype=np.float64)))
        assert np.all(np.abs(got[i] - row) <= tol)


def test_w8a16_ref_agrees_with_w8a8_on_dequantised_activation():
    # A = dec(codes) * 2^e exactly (4 significant bits, inside bf16's range):
    # the weight-only product of A must equal the W8A8 product of (codes, 2^e).
    m, n, k = 3, 260, 384
    a_q = workloads.random_codes((m, k), 31)
    e = np.random.default_rng(32).integers(-6, 7, size=(m, k // 128))
    a_s = np.ldexp(np.ones((m, k // 128), dtype=np.float32), e).astype(np.float32)
    a = e4m3_decode(a_q) * np.repeat(a_s.astype(np.float64), 128, axis=1)
    w_q = workloads.random_codes((n, k), 33)
    w_s = workloads.random_scales((-(-n // 128), k // 128), 34)
    got = gemm_w8a16_ref(a, w_q, w_s)
    ref = gemm_ref(a_q, a_s, w_q, w_s)
    assert np.all(np.abs(got - ref) <= 2.0 ** -48 * _sum_abs_terms(a, w_q, w_s))


def test_w8a16_ref_weight_scale_block_locality():
    m, n, k = 2, 300, 256
    a = _bf16_values(m, k, 41)
    w_q = workloads.random_codes((n, k), 42)
    w_s = workloads.random_scales((3, 2), 43)
    base = gemm_w8a16_ref(a, w_q, w_s)
    w_s2 = w_s.copy()
    w_s2[1, :] *= 2.0  # weight rows 128..255 only
    got = gemm_w8a16_ref(a, w_q, w_s2)
    assert np.array_equal(got[:, :128], base[:, :128]) and np.array_equal(got[:, 256:], base[:, 256:])
    assert np.allclose(got[:, 128:256], 2.0 * base[:, 128:256], rtol=1e-14, atol=0)
