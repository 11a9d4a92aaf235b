"""Pins for the oracle's e4m3 codec (CPU only).

What fixes the codec independently of the oracle's own code:
  * hand-derived points in tests/golden/e4m3_points.txt;
  * a second, enumerative construction of the 256-code table;
  * exhaustive round trip, midpoint ties and monotonicity;
  * torch's float8_e4m3fn cast (a library routine used only as a check).
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _points():
    out = []
    with open(os.path.join(GOLDEN, "e4m3_points.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            val, code = line.split()[:2]
            out.append((float(val), int(code, 16)))
    return out


@pytest.mark.parametrize("value,code", _points())
def test_golden_encode(value, code):
    got = int(e4m3.encode(np.float32(value).astype(np.float64))[()])
    assert got == code, f"{value!r}: got {got:#04x} want {code:#04x}"


def test_golden_decode_roundtrip_of_points():
    for value, code in _points():
        if abs(value) < 448 and value == e4m3.round_to_e4m3_value(value):
            assert e4m3.decode(np.uint8(code)) == value


def test_table_by_enumeration():
    """Build the set of e4m3 values a second way: every normal
    +-2^(e) * (1 + m/8) for e in -6..8 and every subnormal +-m * 2^-9, minus
    the NaN slot (e = 8, m = 7)."""
    normals = {s * 2.0 ** e * (1 + m / 8) for s in (1, -1) for e in range(-6, 9)
               for m in range(8) if not (e == 8 and m == 7)}
    subn = {s * m * 2.0 ** -9 for s in (1, -1) for m in range(8)}
    expect = normals | subn
    table = e4m3.DECODE_TABLE
    finite = table[~np.isnan(table)]
    assert set(finite.tolist()) == expect
    assert len(expect) == 253              # 254 non-NaN codes, +0 and -0 equal
    assert np.isnan(table[0x7F]) and np.isnan(table[0xFF])
    assert np.isnan(table).sum() == 2
    assert table[0x7E] == 448.0 and table[0xFE] == -448.0
    assert table[0x08] == 2.0 ** -6 and table[0x01] == 2.0 ** -9
    assert math.copysign(1.0, table[0x80]) == -1.0 and table[0x80] == 0.0


def test_exhaustive_roundtrip():
    codes = np.array([c for c in range(256) if c not in e4m3.NAN_CODES], np.uint8)
    back = e4m3.encode(e4m3.decode(codes))
    assert np.array_equal(back, codes)


def test_midpoints_tie_to_even_and_neighbours():
    """Between every pair of adjacent non-negative e4m3 values: the midpoint
    goes to the code with even mantissa; one float32 ulp either side goes to
    the nearer value."""
    vals = np.array(sorted(set(np.abs(e4m3.DECODE_TABLE[~np.isnan(e4m3.DECODE_TABLE)]))))
    for lo, hi in zip(vals[:-1], vals[1:]):
        mid = (lo + hi) / 2
        c_lo, c_hi = int(e4m3.encode(lo)), int(e4m3.encode(hi))
        want = c_lo if c_lo % 2 == 0 else c_hi
        assert int(e4m3.encode(mid)) == want, (lo, hi)
        below = np.nextafter(np.float32(mid), np.float32(0)).astype(np.float64)
        above = np.nextafter(np.float32(mid), np.float32(1e9)).astype(np.float64)
        assert int(e4m3.encode(below)) == c_lo
        assert int(e4m3.encode(above)) == c_hi


def test_saturation_and_sign():
    for y in [448.0, 448.5, 463.99, 464.0, 464.01, 479.0, 480.0, 512.0, 1e6, 3.4e38]:
        assert int(e4m3.encode(y)) == 0x7E
        assert int(e4m3.encode(-y)) == 0xFE
    assert int(e4m3.encode(-0.0)) == 0x80
    assert int(e4m3.encode(-1e-12)) == 0x80
    assert int(e4m3.encode(1e-12)) == 0x00


def test_monotone():
    g = np.random.default_rng(0)
    y = np.sort(np.concatenate([g.standard_normal(20000) * 10.0 ** g.uniform(-4, 3, 20000),
                                np.linspace(-500, 500, 20001)]))
    v = e4m3.decode(e4m3.encode(y))
    assert np.all(np.diff(v) >= 0)


def test_against_torch_float8_cast():
    """torch's float8_e4m3fn cast rounds to nearest even; inside [-448, 448]
    it must agree with the oracle bit for bit."""
    g = np.random.default_rng(1)
    y = np.concatenate([
        g.standard_normal(200000).astype(np.float32) * np.float32(30),
        (g.standard_normal(50000) * 1e-3).astype(np.float32),
        np.float32(e4m3.DECODE_TABLE[np.isfinite(e4m3.DECODE_TABLE)]),
    ])
    y = np.clip(y, -448, 448).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3.encode(y.astype(np.float64))
    assert np.array_equal(got, ref)
