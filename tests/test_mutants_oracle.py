"""The oracle's pins can fail: each plausible mistake planted in a copy of
the oracle (in a child process; the files are untouched) is caught by at
least one pin. The mistakes: quantising by multiplying with a reciprocal
instead of dividing, a wrong all-zero-group scale, a signed instead of an
absolute group maximum, per-row instead of per-block weight scales, ties
away from zero, a lost negative-zero sign, a wrong subnormal exponent or
exponent bias in the decode table, transposed or mis-indexed weight scales,
the activation scale of the wrong group, a dropped group, ties to the higher
index in top-k and in the rescoring pick, and a missing weight scale in the
weight-only product. See oracle_mutants.py."""

import os
import subprocess
import sys

import pytest

from oracle_mutants import MUTANTS

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    proc = subprocess.run([sys.executable, os.path.join(HERE, "oracle_mutants.py"), name], stdout=subprocess.PIPE,
                          stderr=subprocess.STDOUT, text=True, timeout=600)
    # pytest exit status 1: tests ran and at least one failed
    assert proc.returncode == 1, proc.stdout[-3000:]
