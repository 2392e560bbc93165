"""The CPU oracle against its pins (library routines, format constants, brute force,
closed forms, invariants the pages fix).  No GPU needed."""
import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_e4m3_reference_points_golden():
    """The oracle's E4M3 codec against reference points of the OCP E4M3FN format
    (tests/golden/e4m3_reference_points.txt)."""
    import os

    import numpy as np

    from oracle import moe_oracle as O
    path = os.path.join(os.path.dirname(__file__), "golden", "e4m3_reference_points.txt")
    n = 0
    for line in open(path, encoding="utf-8"):
        line = line.split("#")[0].strip()
        if not line:
            continue
        f = line.split()
        if f[0] == "MID":
            lo, hi, v = int(f[1], 16), int(f[2], 16), float(f[3])
            assert O.e4m3_decode(np.uint8(lo)) < v < O.e4m3_decode(np.uint8(hi))
            want = lo if (lo & 1) == 0 else hi
            assert int(O.e4m3_encode(v)) == want, line
        elif f[0] == "SAT":
            assert int(O.e4m3_encode(float(f[2]))) == int(f[1], 16), line
        else:
            code, v = int(f[0], 16), float(f[1])
            got = float(O.e4m3_decode(np.uint8(code)))
            assert got == v and np.signbit(got) == np.signbit(v), line
            assert int(O.e4m3_encode(v)) == code, line
        n += 1
    assert n >= 19
