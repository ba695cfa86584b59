"""Pins for the oracle's two-stage scoring (CPU only).

Pins: the bf16 key is monotone against the values torch decodes from the
bit patterns (every finite pattern); top-k against a brute-force Python sort
by (value, -index) on small rows with heavy ties and signed zeros, and
k = V giving the full order; rescoring against exact rational dot products
(Fractions) and its pick against the brute-force maximum.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16_key, rescore_ref, topk_ref


def _finite_bf16_bits():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return b[(b & 0x7F80) != 0x7F80]


def test_bf16_key_is_monotone_in_value():
    bits = _finite_bf16_bits()
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    key = bf16_key(bits)
    order = np.argsort(key, kind="stable")
    v = vals[order]
    assert np.all(v[1:] >= v[:-1])  # non-decreasing values along increasing keys
    assert len(np.unique(key)) == len(key)  # injective
    z = bf16_key(np.array([0x8000, 0x0000], dtype=np.uint16))
    assert z[0] + 1 == z[1]  # -0 directly below +0


def _brute_topk(bits_row, k):
    vals = torch.from_numpy(bits_row.view(np.int16)).view(torch.bfloat16).float().numpy()
    # (value, is +0 over -0, -index): the stated order, from decoded values
    sign0 = [0 if (b == 0x8000) else 1 for b in bits_row]
    items = sorted(range(len(bits_row)), key=lambda i: (vals[i], sign0[i], -i), reverse=True)
    return items[:k]


@pytest.mark.parametrize("v,k,seed", [(50, 5, 1), (64, 64, 2), (300, 17, 3), (1000, 1, 4), (257, 100, 5)])
def test_topk_ref_brute_force_with_ties(v, k, seed):
    rng = np.random.default_rng(seed)
    pool = np.array([0x3F80, 0x3F80, 0xBF80, 0x0000, 0x8000, 0x4000, 0x3F81, 0xC000, 0x0001], dtype=np.uint16)
    bits = rng.choice(pool, size=(3, v))  # few distinct values: many ties
    bits[1] = rng.integers(0, 1 << 16, size=v).astype(np.uint16)
    bits[1][(bits[1] & 0x7F80) == 0x7F80] &= 0x807F
    idx, vals = topk_ref(bits, k)
    for i in range(3):
        assert list(idx[i]) == _brute_topk(bits[i], k)
        assert np.array_equal(vals[i], bits[i][idx[i]])


def _exact_dot(hrow, wrow):
    return sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(hrow, wrow))


def test_rescore_ref_exact_and_pick():
    rng = np.random.default_rng(9)
    m, v, k, kk = 2, 40, 256, 7
    h = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    w = torch.from_numpy(rng.standard_normal((v, k)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    # two vocabulary rows with equal, clearly largest scores for row 0: the
    # pick must be the lower index
    w[3] = torch.from_numpy((2.0 * h[0]).astype(np.float32)).to(torch.bfloat16).float().numpy()
    w[5] = w[3]
    idx = np.stack([rng.permutation(v)[:kk] for _ in range(m)])
    idx[0, :2] = [5, 3]
    scores, pick = rescore_ref(h, w, idx)
    for i in range(m):
        exact = [_exact_dot(h[i], w[j]) for j in idx[i]]
        for j in range(kk):
            assert abs(scores[i, j] - float(exact[j])) <= 2.0 ** -50 * float(np.abs(h[i]) @ np.abs(w[idx[i, j]]))
        best = max(range(kk), key=lambda j: (exact[j], -idx[i, j]))
        assert pick[i] == idx[i, best]
    assert pick[0] == 3  # the tie between rows 3 and 5 goes to row 3


def _pattern_rank(b):
    """The stated order read off a bf16 bit pattern directly: every pattern
    with the sign bit clear ranks above every pattern with it set; among the
    former a larger 15-bit magnitude field ranks higher, among the latter
    lower. NaN and infinity patterns take their place by the same rule."""
    b = int(b)
    mag = b & 0x7FFF
    return (1, mag) if b < 0x8000 else (0, -mag)


def _brute_topk_any_pattern(bits_row, k):
    items = sorted(range(len(bits_row)), key=lambda i: (_pattern_rank(bits_row[i]), -i), reverse=True)
    return items[:k]


def test_pattern_rank_is_the_value_order_on_non_nan_patterns():
    # the tuple rank above is the numeric order (infinities at the ends, +0
    # over -0) wherever a value exists: checked against torch's decoding
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    nan = ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    b = b[~nan]
    vals = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    order = sorted(range(b.size), key=lambda i: _pattern_rank(b[i]))
    v = vals[order]
    assert np.all(v[1:] >= v[:-1])
    assert np.isneginf(v[0]) and np.isposinf(v[-1])


@pytest.mark.parametrize("v,k,seed", [(64, 10, 11), (300, 64, 12), (1000, 256, 13), (97, 97, 14)])
def test_topk_ref_on_inf_and_nan_patterns(v, k, seed):
    rng = np.random.default_rng(seed)
    special = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0xFFFF, 0x7FFF, 0x0000, 0x8000, 0x3F80, 0xBF80],
                       dtype=np.uint16)
    bits = np.stack([
        rng.integers(0, 1 << 16, size=v).astype(np.uint16),  # every pattern class, NaN and Inf included
        rng.choice(special, size=v),  # mostly infinities, NaNs and zeros: many ties
        np.where(rng.random(v) < 0.5, rng.choice(special, size=v), rng.integers(0, 1 << 16, size=v)).astype(np.uint16),
    ])
    idx, vals = topk_ref(bits, k)
    for i in range(bits.shape[0]):
        assert list(idx[i]) == _brute_topk_any_pattern(bits[i], k)
        assert np.array_equal(vals[i], bits[i][idx[i]])
