"""Host-only checks of the parity diagnostics (fp16 ulp distance and
bit-equality), against values fixed by the binary16 format itself."""
import numpy as np
import pytest

from parity import diagnostics, ordered16

pytestmark = pytest.mark.cpu


def h(bits):
    return np.array(bits, dtype=np.uint16).view(np.float16)


def test_ordered16_counts_representable_values():
    one, next_one = h([0x3C00]), h([0x3C01])
    assert abs(int(ordered16(next_one)[0] - ordered16(one)[0])) == 1
    # +0 and -0 are the same value
    assert ordered16(h([0x0000]))[0] == ordered16(h([0x8000]))[0] == 0
    # smallest subnormals on either side of zero are two values apart
    assert int(ordered16(h([0x0001]))[0] - ordered16(h([0x8001]))[0]) == 2
    # 65504 (largest finite) to inf is one step; 2048 and 2050 are adjacent (spacing 2)
    assert int(ordered16(h([0x7C00]))[0] - ordered16(h([0x7BFF]))[0]) == 1
    assert int(ordered16(np.float16([2050.0]))[0] - ordered16(np.float16([2048.0]))[0]) == 1
    # ordering agrees with the values over every finite pattern
    u = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    v = u.view(np.float16)
    fin = np.isfinite(v)
    order = np.argsort(v[fin].astype(np.float64), kind="stable")
    o = ordered16(v[fin])[order]
    assert np.all(np.diff(o) >= 0)


def test_diagnostics_on_known_differences():
    r16 = np.array([1.0, 2.0, -3.0, 0.5], dtype=np.float16)
    g = r16.copy()
    g[1] = h([0x4001])[0]          # one ulp above 2.0
    g[2] = np.float16(-3.0 - 3 * 2.0 ** -9)   # three ulps below -3 (spacing 2^-9 in [2, 4))
    d = diagnostics(g, r16.astype(np.float64), ref16=r16)
    assert d["elements"] == 4
    assert d["bit_equal_frac"] == 0.5
    assert d["max_ulp"] == 3
    assert d["frac_within_1ulp"] == 0.75
