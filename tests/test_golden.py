"""Oracle against the stored E2M1 fixtures (each fixture cites its source in its header)."""
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_e2m1_code_table():
    rows = _rows("e2m1_codes.txt")
    assert len(rows) == 16
    for code, s, e, m, value in rows:
        code = int(code)
        assert code == (int(s) << 3) | (int(e, 2) << 1) | int(m)
        assert oracle.e2m1_value(code) == float(value)


def test_e2m1_midpoints():
    for x, code in _rows("e2m1_midpoints.txt"):
        assert int(oracle.e2m1_encode([np.float32(x)])[0]) == int(code), x
        assert int(oracle.e2m1_encode([np.float32(-float(x))])[0]) == int(code) | 8, x
