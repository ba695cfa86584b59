"""Pins for the oracle's activation and weight quantisers (CPU only).

Pins: hand-derived groups in tests/golden/quant_act_cases.txt, invariants of
the scale rule (sign symmetry, power-of-two equivariance, block locality)
and exact-rational brute force on small inputs.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import quant_act_ref, quant_weight_ref
from exact import quant_group_exact
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "quant_act_cases.txt")) as f:
        for ln in f:
            ln = ln.strip()
            if not ln or ln.startswith("#"):
                continue
            key, _, rest = ln.partition(" ")
            if key == "case":
                cur = {"name": rest, "values": {}, "fill": 0.0, "codes": {}, "codefill": 0}
                cases.append(cur)
            elif key == "values":
                for tok in rest.split():
                    i, v = tok.split(":")
                    cur["values"][int(i)] = float.fromhex(v)
            elif key == "fill":
                cur["fill"] = float.fromhex(rest)
            elif key == "scale":
                cur["scale"] = float.fromhex(rest)
            elif key == "codes":
                for tok in rest.split():
                    i, c = tok.split(":")
                    cur["codes"][int(i)] = int(c, 16)
            elif key == "codefill":
                cur["codefill"] = int(rest, 16)
    return cases


CASES = _load_cases()


def _group(case):
    x = np.full(128, case["fill"], dtype=np.float32)
    for i, v in case["values"].items():
        x[i] = v
    return x


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_quant_act_golden_cases(case):
    x = _group(case)
    # every golden value is bf16-exact
    assert np.array_equal(torch.from_numpy(x).to(torch.bfloat16).float().numpy(), x)
    codes, s = quant_act_ref(x[None, :])
    assert s.dtype == np.float32 and s.shape == (1, 1)
    assert s[0, 0] == np.float32(case["scale"])
    want = np.full(128, case["codefill"], dtype=np.uint8)
    for i, c in case["codes"].items():
        want[i] = c
    assert np.array_equal(codes[0], want), (case["name"], codes[0][:8], want[:8])


def test_golden_cases_agree_with_rational_brute_force():
    for case in CASES:
        s, codes = quant_group_exact(_group(case))
        assert s == Fraction(case["scale"]), case["name"]


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def test_quant_act_against_rational_brute_force():
    # bf16 activations with outliers, tiny and huge magnitudes, exact zeros
    rng = np.random.default_rng(11)
    a = rng.standard_normal((3, 512)).astype(np.float32)
    a[0, :128] *= 1e-3
    a[1, 128:256] *= 3e4
    a[2, 256:384] = 0.0
    a[2, 300] = -2.0 ** -40
    a[0, 5] *= 20
    a[1, 400] *= 20
    a = _bf16(a)
    codes, s = quant_act_ref(a)
    for m in range(a.shape[0]):
        for g in range(a.shape[1] // 128):
            es, ecodes = quant_group_exact(a[m, g * 128 : (g + 1) * 128])
            assert Fraction(float(s[m, g])) == es, (m, g)
            assert list(codes[m, g * 128 : (g + 1) * 128]) == ecodes, (m, g)


def test_quant_act_sign_flip_only_flips_sign_bits():
    a, _ = workloads.tiny_inputs()
    c1, s1 = quant_act_ref(a)
    c2, s2 = quant_act_ref(-a)
    assert np.array_equal(s1, s2)
    assert np.array_equal(c1 ^ 0x80, c2)


@pytest.mark.parametrize("j", [-5, -1, 1, 7])
def test_quant_act_power_of_two_equivariance(j):
    a = workloads.activation(4, 512, 1024).float().numpy()
    c1, s1 = quant_act_ref(a)
    c2, s2 = quant_act_ref(a * np.float32(2.0 ** j))
    assert np.array_equal(c1, c2)
    assert np.array_equal(s2, s1 * np.float32(2.0 ** j))


def test_quant_act_scale_recovers_group_max():
    # the largest entry of a group always maps to +-448 (code 0x7E/0xFE)
    a = workloads.activation(8, 7168, 5120).float().numpy()
    codes, s = quant_act_ref(a)
    g = a.reshape(8, 40, 128)
    idx = np.argmax(np.abs(g), axis=2)
    top = np.take_along_axis(codes.reshape(8, 40, 128), idx[..., None], axis=2)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)
    amax = np.take_along_axis(np.abs(g), idx[..., None], axis=2)[..., 0]
    assert np.all(s * np.float32(448) <= amax * np.float32(1 + 2 ** -22))
    assert np.all(s * np.float32(448) >= amax * np.float32(1 - 2 ** -22))


def test_quant_act_empty_and_bad_shapes():
    codes, s = quant_act_ref(np.zeros((0, 256), np.float32))
    assert codes.shape == (0, 256) and s.shape == (0, 2)
    with pytest.raises(ValueError):
        quant_act_ref(np.zeros((2, 100), np.float32))


def test_quant_weight_against_rational_brute_force():
    rng = np.random.default_rng(3)
    w = (0.02 * rng.standard_normal((130, 256))).astype(np.float32)
    w[129, 200] = 0.9  # outlier in the partial last row block
    codes, s = quant_weight_ref(w)
    assert s.shape == (2, 2)
    for b in range(2):
        for g in range(2):
            blk = w[b * 128 : min(b * 128 + 128, 130), g * 128 : (g + 1) * 128]
            es, ecodes = quant_group_exact(blk.reshape(-1))
            assert Fraction(float(s[b, g])) == es, (b, g)
            got = codes[b * 128 : min(b * 128 + 128, 130), g * 128 : (g + 1) * 128].reshape(-1)
            assert list(got) == ecodes, (b, g)


def test_quant_weight_block_locality():
    w = workloads.weight(300, 384)
    c1, s1 = quant_weight_ref(w)
    w2 = w.copy()
    w2[130, 260] = 5.0  # block (1, 2)
    c2, s2 = quant_weight_ref(w2)
    changed_s = np.argwhere(s1 != s2)
    assert changed_s.tolist() == [[1, 2]]
    diff_rows, diff_cols = np.nonzero(c1 != c2)
    assert diff_rows.min() >= 128 and diff_rows.max() < 256
    assert diff_cols.min() >= 256 and diff_cols.max() < 384


def test_quant_weight_matches_activation_rule_on_single_row_blocks():
    # a weight with N=1 has 1x128 blocks, i.e. exactly the activation rule
    w = workloads.weight(1, 1024)
    cw, sw = quant_weight_ref(w)
    ca, sa = quant_act_ref(w)
    assert np.array_equal(cw, ca) and np.array_equal(sw, sa)
