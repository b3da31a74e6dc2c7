"""Oracle against hand-worked examples stored under tests/golden/."""

import glob
import os

import numpy as np
import pytest

import oracle
from cases import load_golden

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "handworked_*.txt")))


def test_fixtures_present():
    assert len(GOLDEN) >= 3


@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(p) for p in GOLDEN])
def test_oracle_matches_handworked(path):
    fmt, Q, X, d, offs, lens, exp = load_golden(path)
    got = oracle.maxsim(fmt, Q, X, offs, lens, d=d)
    assert np.array_equal(got, exp), (got, exp)
