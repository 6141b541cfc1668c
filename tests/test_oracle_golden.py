"""Oracle regression: the oracle's results on the small seeded inputs frozen in
tests/golden/ (written by tests/golden/make_golden.py, which calls only the oracle). These
guard the oracle against unintended changes; they are not pins against the pages."""
import os
import sys

import numpy as np
import pytest

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, HERE)
import make_golden  # noqa: E402


def _read(name):
    out = {}
    with open(os.path.join(HERE, name + ".txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            label, *vals = line.split()
            out[label] = np.array([float(v) for v in vals])
    return out


@pytest.mark.parametrize("name,arrays", make_golden.cases(), ids=lambda c: c if isinstance(c, str) else "")
def test_oracle_matches_frozen_fixture(name, arrays):
    stored = _read(name)
    assert set(stored) == {label for label, _ in arrays}
    for label, a in arrays:
        np.testing.assert_allclose(np.asarray(a, np.float64).ravel(), stored[label], rtol=1e-12,
                                   atol=1e-14, err_msg=f"{name}:{label}")
