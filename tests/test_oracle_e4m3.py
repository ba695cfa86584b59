"""Pins for the oracle's e4m3fn codec (CPU only).

The codec is fixed by the OCP 8-bit floating point specification, not by the
pages (which only say "FP8", page 2 section 8). Pins: torch's own
float8_e4m3fn type (a library routine), the spec's spot values, ties worked
by hand, exact-rational brute force.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_encode_rne, e4m3_values
from exact import E4M3_POS, e4m3_nearest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_encode(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_for_all_256_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero
    assert math.copysign(1.0, ours[0x80]) == -1.0 and math.copysign(1.0, ours[0x00]) == 1.0


def test_decode_spot_values_from_spec():
    with open(os.path.join(GOLDEN, "e4m3_spot.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 15
    vals = e4m3_values()
    for code_s, val_s in rows:
        code = int(code_s, 16)
        if val_s == "nan":
            assert np.isnan(vals[code])
        else:
            want = float.fromhex(val_s)
            assert vals[code] == want and math.copysign(1, vals[code]) == math.copysign(1, want), hex(code)


def test_decode_matches_integer_bitfield_brute_force():
    vals = e4m3_values()
    for c in range(0x7F):
        assert Fraction(vals[c]) == E4M3_POS[c]
        assert Fraction(vals[c | 0x80]) == -E4M3_POS[c]


def _critical_points():
    pos = e4m3_values()[:0x7F]
    pts = [0.0, 448.0]
    for i in range(0x7F):
        pts.append(pos[i])
        if i < 0x7E:
            mid = np.float32((pos[i] + pos[i + 1]) / 2)
            pts += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e4))]
    pts += [1e-30, 1e-40, 2.0 ** -149, 447.99997, 2.0 ** -10, 3 * 2.0 ** -10]
    pts = np.array(pts, dtype=np.float32)
    return np.concatenate([pts, -pts])


def test_encode_critical_points_match_torch_cast():
    pts = _critical_points()
    assert np.array_equal(e4m3_encode_rne(pts), _torch_encode(pts))


def test_encode_hand_ties():
    # a list, not a dict: -0.0 and 0.0 are equal keys
    cases = [(2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (432.0, 0x7E), (1.0625, 0x38), (1.1875, 0x3A),
             (-1.0625, 0xB8), (-0.0, 0x80), (0.0, 0x00), (-1e-6, 0x80), (448.0, 0x7E), (-448.0, 0xFE)]
    got = e4m3_encode_rne(np.array([v for v, _ in cases], np.float32))
    assert [int(c) for c in got] == [c for _, c in cases]


def test_encode_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3_encode_rne(e4m3_decode(codes).astype(np.float32)), codes)


def test_encode_random_values_against_rational_brute_force():
    rng = np.random.default_rng(123)
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), size=600)).astype(np.float32)
    signs = rng.choice([-1.0, 1.0], size=600).astype(np.float32)
    v = np.minimum(mags, np.float32(448)) * signs
    got = e4m3_encode_rne(v)
    for x, c in zip(v, got):
        assert int(c) == e4m3_nearest(Fraction(float(x)), bool(np.signbit(x))), float(x)


def test_encode_random_values_against_torch_cast():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(200000) * 60).astype(np.float32)
    v = np.clip(v, -448, 448)
    assert np.array_equal(e4m3_encode_rne(v), _torch_encode(v))


def test_encode_rejects_out_of_range_and_nonfinite():
    with pytest.raises(ValueError):
        e4m3_encode_rne(np.array([448.5], np.float32))
    with pytest.raises(ValueError):
        e4m3_encode_rne(np.array([np.nan], np.float32))
    with pytest.raises(ValueError):
        e4m3_encode_rne(np.array([-np.inf], np.float32))
