"""Exhaustive CPU check of the quotients the quantisation kernels use.

The kernels (activation quantisation and the quantisation fused into the
GEMM) form x / s as a correctly rounded reciprocal of s followed by one
fma-based correction (Markstein's method) instead of an IEEE division per
value, for every group whose amax is at least 2^-96; the quantisation inside
the fused GEMM uses a two-term reciprocal instead (two operations per value,
no clamp). `quotient_check.c` runs both in host fp32 (libm's correctly
rounded fmaf) for every bf16 amax >= 2^-96 and every bf16 x in [0, amax],
rounds them to e4m3 and counts code mismatches against the IEEE division,
which must be zero (for the fused form: except the sign of a zero).

The harness's own e4m3 rounding is pinned to the oracle's encoder on the
codec's critical points, and a build without the correction step must
report mismatches, so the check can fail.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import e4m3_encode_rne, e4m3_values

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "quotient_check.c")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


def _build(tmp_path, *defines):
    exe = str(tmp_path / ("qc" + "".join(d.lower() for d in defines)))
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", *[f"-D{d}" for d in defines], SRC, "-lm", "-o", exe]
    subprocess.run(cmd, check=True)
    return exe


def _run_check(exe):
    env = dict(os.environ, OMP_NUM_THREADS=str(min(16, os.cpu_count() or 1)))
    proc = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, env=env, timeout=600)
    fields = proc.stdout.split()
    stats = {fields[i]: int(fields[i + 1]) for i in range(0, len(fields), 2)}
    return proc.returncode, stats, proc.stderr


def _expected_pairs():
    # positive x patterns 0..p for every amax pattern p, plus the negative x
    # patterns 0..p on every 17th amax
    first, last = 31 << 7, 0x7F7F
    p = np.arange(first, last + 1, dtype=np.int64)
    return int(np.sum(p + 1) + np.sum((p + 1)[p % 17 == 0]))


def test_harness_encoder_matches_oracle_on_critical_points(tmp_path):
    exe = _build(tmp_path)
    vals = e4m3_values()[:0x7F]  # non-negative finite codes
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids]).astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    down = np.nextafter(pts, np.float32(-np.inf))
    pts = np.concatenate([pts, up, down, [np.float32(460.0), np.float32(3e38)]])
    pts = pts[pts >= 0]
    pts = np.concatenate([pts, -pts]).astype(np.float32)
    text = "\n".join(float(v).hex() for v in pts) + "\n"
    out = subprocess.run([exe, "encode"], input=text, stdout=subprocess.PIPE, text=True, check=True).stdout
    got = np.array([int(t) for t in out.split()], dtype=np.int64)
    want = e4m3_encode_rne(np.clip(pts, -448, 448)).astype(np.int64)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_corrected_quotient_gives_division_codes_for_every_bf16_pair(tmp_path):
    rc, stats, err = _run_check(_build(tmp_path))
    assert stats["pairs"] == _expected_pairs()
    assert stats["code_differs"] == 0, err[:2000]
    # the fused GEMM's two-term-reciprocal quotient: same codes except the
    # sign of a zero, never above 448 (1 + 2^-23)
    assert stats["gemm_code_differs"] == 0
    assert stats["gemm_qmax_over"] == 0
    assert rc == 0
    # the quotients themselves do differ sometimes: the code, not the fp32
    # value, is what the check establishes
    assert stats["quotient_differs"] > 0


def test_check_fails_without_the_correction_step(tmp_path):
    rc, stats, _ = _run_check(_build(tmp_path, "UNCORRECTED"))
    assert rc == 1 and stats["code_differs"] > 0
