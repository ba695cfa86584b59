"""Pins for the oracle's block-scaled GEMM (CPU only).

Pins: exact brute force (integer group sums, Fraction scales) on tiny shapes
and on the whole tiny case; a closed form for constant codes; the scale = 1
special case against torch's float64 matmul (library routine); an identity
weight; block locality and linearity of the weight scales.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, gemm_ref, gemm_ref_at, quant_act_ref, quant_weight_ref
from exact import gemm_exact
import workloads


def _sum_abs_terms(a_q, a_s, w_q, w_s):
    a = np.abs(e4m3_decode(a_q) * np.repeat(a_s.astype(np.float64), 128, axis=1))
    w = np.abs(e4m3_decode(w_q) * np.repeat(np.repeat(w_s.astype(np.float64), 128, axis=0)[: w_q.shape[0]], 128, axis=1))
    return a @ w.T


def _random_problem(m, n, k, seed):
    a_q = workloads.random_codes((m, k), seed)
    w_q = workloads.random_codes((n, k), seed + 1)
    a_s = workloads.random_scales((m, k // 128), seed + 2)
    w_s = workloads.random_scales((-(-n // 128), k // 128), seed + 3)
    return a_q, a_s, w_q, w_s


@pytest.mark.parametrize("m,n,k,seed", [(1, 128, 128, 1), (2, 256, 256, 2), (2, 200, 384, 3), (3, 1, 128, 4)])
def test_gemm_ref_exact_brute_force_small(m, n, k, seed):
    a_q, a_s, w_q, w_s = _random_problem(m, n, k, seed)
    got = gemm_ref(a_q, a_s, w_q, w_s)
    exact = np.array([float(v) for v in gemm_exact(a_q, a_s, w_q, w_s)]).reshape(m, n)
    bound = 2.0 ** -50 * _sum_abs_terms(a_q, a_s, w_q, w_s)
    assert np.all(np.abs(got - exact) <= bound)


def test_gemm_ref_exact_brute_force_whole_tiny_case():
    a, w = workloads.tiny_inputs()
    a_q, a_s = quant_act_ref(a)
    w_q, w_s = quant_weight_ref(w)
    got = gemm_ref(a_q, a_s, w_q, w_s)
    exact = np.array([float(v) for v in gemm_exact(a_q, a_s, w_q, w_s)]).reshape(got.shape)
    bound = 2.0 ** -50 * _sum_abs_terms(a_q, a_s, w_q, w_s)
    assert np.all(np.abs(got - exact) <= bound)
    # the quantised product approximates the unquantised one (sanity, not a
    # pin): two 3-bit-mantissa roundings give a few percent relative rms error
    fp = a.float().numpy().astype(np.float64) @ w.astype(np.float64).T
    assert np.sqrt(np.mean((got - fp) ** 2)) < 0.08 * np.sqrt(np.mean(fp ** 2))


def test_gemm_ref_at_matches_brute_force():
    a_q, a_s, w_q, w_s = _random_problem(5, 300, 512, 9)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, 5, 40)
    cols = rng.integers(0, 300, 40)
    got = gemm_ref_at(a_q, a_s, w_q, w_s, rows, cols)
    exact = np.array([float(v) for v in gemm_exact(a_q, a_s, w_q, w_s, rows, cols)])
    bound = 2.0 ** -50 * _sum_abs_terms(a_q, a_s, w_q, w_s)[rows, cols]
    assert np.all(np.abs(got - exact) <= bound)


def test_gemm_ref_closed_form_constant_codes():
    m, n, k = 3, 256, 640
    a_code, w_code = 0x3B, 0xC5  # 1.375 and -(1.625 * 2^1) = -3.25
    sa, sw = np.float32(0.75), np.float32(2.0 ** -7 * 3)
    a_q = np.full((m, k), a_code, np.uint8)
    w_q = np.full((n, k), w_code, np.uint8)
    a_s = np.full((m, k // 128), sa, np.float32)
    w_s = np.full((2, k // 128), sw, np.float32)
    got = gemm_ref(a_q, a_s, w_q, w_s)
    want = k * 1.375 * -3.25 * float(sa) * float(sw)
    assert np.all(got == want)


def test_gemm_ref_unit_scales_equal_plain_matmul():
    a_q, _, w_q, _ = _random_problem(4, 384, 768, 21)
    a_s = np.ones((4, 6), np.float32)
    w_s = np.ones((3, 6), np.float32)
    got = gemm_ref(a_q, a_s, w_q, w_s)
    ref = torch.from_numpy(e4m3_decode(a_q)) @ torch.from_numpy(e4m3_decode(w_q)).T
    assert np.array_equal(got, ref.numpy())  # every group sum is exact in fp64


def test_gemm_ref_identity_weight():
    m, k = 3, 384
    a = workloads.activation(m, 384, k)
    a_q, a_s = quant_act_ref(a)
    w_q = np.zeros((k, k), np.uint8)
    np.fill_diagonal(w_q, 0x38)  # 1.0
    w_s = np.ones((3, 3), np.float32)
    got = gemm_ref(a_q, a_s, w_q, w_s)
    want = e4m3_decode(a_q) * np.repeat(a_s.astype(np.float64), 128, axis=1)
    assert np.array_equal(got, want)


def test_gemm_ref_weight_scale_block_locality_and_linearity():
    m, n, k = 2, 384, 512
    a_q, a_s, w_q, w_s = _random_problem(m, n, k, 33)
    base = gemm_ref(a_q, a_s, w_q, w_s)
    b, g = 1, 2
    w_s2 = w_s.copy()
    w_s2[b, g] *= 2
    moved = gemm_ref(a_q, a_s, w_q, w_s2)
    diff = moved - base
    outside = np.ones(n, bool)
    outside[b * 128 : (b + 1) * 128] = False
    assert np.all(diff[:, outside] == 0)
    # inside the block the change is exactly that group's term
    cols = np.arange(b * 128, (b + 1) * 128)
    term = (e4m3_decode(a_q[:, g * 128 : (g + 1) * 128]) @ e4m3_decode(w_q[cols, g * 128 : (g + 1) * 128]).T)
    term = term * a_s[:, g : g + 1].astype(np.float64) * float(w_s[b, g])
    # (moved - base) cancels the other groups: compare within fp64 rounding of
    # the full sums
    tol = 2.0 ** -48 * _sum_abs_terms(a_q, a_s, w_q, w_s2)[:, cols]
    assert np.all(np.abs(diff[:, cols] - term) <= tol)
    assert np.all(np.abs(term) > 0)


def test_gemm_ref_activation_scale_row_locality():
    m, n, k = 3, 256, 384
    a_q, a_s, w_q, w_s = _random_problem(m, n, k, 44)
    base = gemm_ref(a_q, a_s, w_q, w_s)
    a_s2 = a_s.copy()
    a_s2[1, 0] *= 4
    moved = gemm_ref(a_q, a_s2, w_q, w_s)
    assert np.array_equal(moved[[0, 2]], base[[0, 2]])
    assert not np.array_equal(moved[1], base[1])


def test_gemm_ref_rejects_bad_shapes():
    a_q, a_s, w_q, w_s = _random_problem(3, 128, 256, 1)
    with pytest.raises(ValueError):
        gemm_ref(a_q, a_s.T, w_q, w_s)
    with pytest.raises(ValueError):
        gemm_ref(a_q, a_s, w_q[:, :128], w_s)
