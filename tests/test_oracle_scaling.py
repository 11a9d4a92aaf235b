"""Pins for the oracle's group scaling (CPU only): hand-derived points,
power-of-two exactness, scaling invariance, partial blocks, and a plain
per-group loop that restates the rule element by element."""
import os

import numpy as np
import pytest

from oracle import e4m3, scaling

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    rows = []
    with open(os.path.join(GOLDEN, "scaling_points.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, vals, scale, codes = line.split()
            rows.append((kind, [float(v) for v in vals.split(",")], float(scale),
                         [int(c, 16) for c in codes.split(",")]))
    return rows


@pytest.mark.parametrize("kind,vals,scale,codes", _golden())
def test_golden_groups(kind, vals, scale, codes):
    width = 128 if kind == "1x128" else 32
    x = np.zeros((1, width), np.float32)
    x[0, :len(vals)] = vals
    if kind == "1x128":
        q, s = scaling.quantize_1x128(x)
        assert s.shape == (1, 1) and float(s[0, 0]) == scale
    else:
        q, e = scaling.quantize_mx(x)
        assert e.shape == (1, 1) and int(e[0, 0]) == int(scale)
    assert q[0, :len(codes)].tolist() == codes
    assert np.all(q[0, len(vals):] == 0)


def _loop_1x128(x):
    """Per-group restatement with Python scalars (float32 via numpy scalars)."""
    rows, cols = x.shape
    q = np.zeros((rows, cols), np.uint8)
    s = np.zeros((cols // 128, rows), np.float32)
    for r in range(rows):
        for g in range(cols // 128):
            grp = x[r, g * 128:(g + 1) * 128]
            amax = np.float32(max(abs(float(v)) for v in grp))
            sc = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(448.0))
            s[g, r] = sc
            for i, v in enumerate(grp):
                q[r, g * 128 + i] = e4m3.encode(float(np.float32(v / sc)))
    return q, s


def test_1x128_matches_loop():
    g = np.random.default_rng(3)
    x = (g.standard_normal((5, 256)) * np.exp(g.uniform(-8, 8, (5, 1)))).astype(np.float32)
    x[2, 128:] = 0.0
    x[3, :128] = -0.0
    q, s = scaling.quantize_1x128(x)
    q2, s2 = _loop_1x128(x)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_1x128_layout_is_kblock_major():
    x = np.zeros((3, 384), np.float32)
    x[1, 128 + 5] = 448.0 * 4          # row 1, group 1 -> s = 4
    x[2, 256] = -448.0 / 8             # row 2, group 2 -> s = 1/8
    q, s = scaling.quantize_1x128(x)
    assert s.shape == (3, 3)
    assert s[1, 1] == 4.0 and s[2, 2] == 0.125
    assert np.count_nonzero(s != 1.0) == 2
    assert q[1, 133] == 0x7E and q[2, 256] == 0xFE


def test_power_of_two_exact_roundtrip():
    """Groups whose amax is 448 * 2^j get s = 2^j exactly, and inputs that are
    e4m3 values times 2^j come back bit-exactly."""
    g = np.random.default_rng(4)
    vals = e4m3.DECODE_TABLE[np.isfinite(e4m3.DECODE_TABLE)]
    for j in (-20, -7, 0, 3, 11):
        x = g.choice(vals, size=(4, 256)) * 2.0 ** j
        x[:, 0] = 448.0 * 2.0 ** j
        x[:, 128] = -448.0 * 2.0 ** j
        x = x.astype(np.float32)
        q, s = scaling.quantize_1x128(x)
        assert np.all(s == np.float32(2.0 ** j))
        assert np.array_equal(e4m3.decode(q) * 2.0 ** j, x.astype(np.float64))


def test_scaling_invariance_and_amax_maps_to_448():
    g = np.random.default_rng(5)
    x = g.standard_normal((8, 512)).astype(np.float32)
    q, s = scaling.quantize_1x128(x)
    for j in (-5, 4):
        q2, s2 = scaling.quantize_1x128(x * np.float32(2.0 ** j))
        assert np.array_equal(q, q2) and np.array_equal(s2, s * np.float32(2.0 ** j))
    grp = x.reshape(8, 4, 128)
    idx = np.argmax(np.abs(grp), axis=-1)
    qg = q.reshape(8, 4, 128)
    picked = np.take_along_axis(qg, idx[..., None], -1)[..., 0]
    assert np.all((picked == 0x7E) | (picked == 0xFE))


def test_128x128_blocks_and_partial_tail():
    g = np.random.default_rng(6)
    w = g.standard_normal((200, 256)).astype(np.float32)   # 200 rows: blocks 128 + 72
    w[130, 200] = 448.0 * 16
    q, s = scaling.quantize_128x128(w)
    assert s.shape == (2, 2)
    assert s[1, 1] == 16.0                      # amax of the cut block, valid rows only
    # every block restated with the 1x128 rule on its flattened contents
    for rb in range(2):
        for cb in range(2):
            blk = w[rb * 128:(rb + 1) * 128, cb * 128:(cb + 1) * 128]
            amax = np.float32(np.abs(blk).max())
            assert s[rb, cb] == np.float32(amax / np.float32(448))
            y = (blk / s[rb, cb]).astype(np.float64)
            assert np.array_equal(q[rb * 128:(rb + 1) * 128, cb * 128:(cb + 1) * 128],
                                  e4m3.encode(y))


def test_batched_shapes():
    g = np.random.default_rng(7)
    x = g.standard_normal((3, 130, 256)).astype(np.float32)
    q, s = scaling.quantize_1x128(x)
    assert q.shape == x.shape and s.shape == (3, 2, 130)
    for b in range(3):
        qb, sb = scaling.quantize_1x128(x[b])
        assert np.array_equal(q[b], qb) and np.array_equal(s[b], sb)
    q, s = scaling.quantize_128x128(x)
    assert s.shape == (3, 2, 2)
    for b in range(3):
        qb, sb = scaling.quantize_128x128(x[b])
        assert np.array_equal(q[b], qb) and np.array_equal(s[b], sb)


def test_zero_groups():
    x = np.zeros((2, 256), np.float32)
    x[1, :128] = -0.0
    q, s = scaling.quantize_1x128(x)
    assert np.all(s == 1.0)
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0x80) and np.all(q[1, 128:] == 0)
    q, e = scaling.quantize_mx(x)
    assert np.all(e == 0)


def test_mx_exponent_closed_form():
    """E = floor(log2 amax) - 8: amax in [2^j, 2^(j+1)) gives byte j - 8 + 127,
    so amax * 2^-E lands in [256, 512)."""
    for j in range(-60, 60, 7):
        for frac in (1.0, 1.5, 1.999):
            amax = np.float32(frac * 2.0 ** j)
            E = int(scaling.mx_exponent(amax))
            assert E == j - 8
            assert 256 <= float(amax) * 2.0 ** -E < 512
    # clamping at both ends of E8M0
    assert int(scaling.mx_exponent(np.float32(2.0 ** -130))) == -127
    assert int(scaling.mx_exponent(np.float32(1e-45))) == -127


def test_mx_saturates_and_is_exact_for_powers_of_two():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 500.0 * 2.0 ** 10       # scaled 500 -> saturates to 448
    x[0, 1] = 2.0 ** 10               # scaled 1.0 -> exact
    q, e = scaling.quantize_mx(x)
    assert int(e[0, 0]) == 127 + 10 and q[0, 0] == 0x7E and q[0, 1] == 0x38
    g = np.random.default_rng(8)
    vals = e4m3.DECODE_TABLE[np.isfinite(e4m3.DECODE_TABLE)]
    x = g.choice(vals, size=(6, 64))
    x[:, 0] = 448.0
    x[:, 32] = -256.0
    x = (x * 2.0 ** -3).astype(np.float32)
    q, e = scaling.quantize_mx(x)
    assert np.all(e == 127 - 3)
    assert np.array_equal(e4m3.decode(q) * 2.0 ** -3, x.astype(np.float64))
