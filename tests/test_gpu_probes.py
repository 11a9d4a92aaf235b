"""GPU probes of the gfx950 facts the kernels rely on.

  * lane layout of v_mfma_f32_16x16x128_f8f6f4 and 32x32x64 (operands and
    result), checked with random exactly-summable e4m3 operands;
  * the E8M0 scale operands of v_mfma_scale_*: which lane's byte scales which
    32-element chunk, and the bias 127;
  * v_cvt_pk_fp8_f32: round-to-nearest-even, saturation and the sign of zero,
    compared with the oracle's encoder on a sweep through every e4m3 midpoint;
  * v_cvt_pk_bf16_f32 (the BF16 output conversion): round-to-nearest-even
    on ties, overflow, subnormals and signed zeros, against torch's CPU cast;
  * e4m3 subnormal operands times normal ones are used exactly by the FP8
    MFMA (scaled and unscaled); products of two subnormals are reported;
  * how one MFMA rounds its 128-product sum (informational).
Expected values come from the oracle's e4m3 table and the stated hypotheses.
"""
import ctypes
import os

import numpy as np
import pytest

from oracle import e4m3

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "gpu_probes", "libfg8_probes.so")


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(LIB):
        raise RuntimeError("probe library not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    for name in ("probe_mfma16", "probe_mfma32", "probe_mfma16_scaled", "probe_mfma32_scaled",
                 "probe_mfma16_acc", "probe_mfma32_acc", "probe_cvt_fp8", "probe_cvt_bf16",
                 "probe_copy"):
        getattr(lib, name).restype = ctypes.c_int
    return torch, lib


def _stream(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


SMALL = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 1.5, -1.5, 2.0, -2.0, 3.0, -3.0, 4.0, -4.0])


def _codes(g, shape):
    return e4m3.encode(g.choice(SMALL, size=shape))


def _run_mfma(torch, lib, fn, a_lanes, b_lanes, nres, sa=None, sb=None):
    dev = "cuda"
    a = torch.from_numpy(np.ascontiguousarray(a_lanes)).to(dev)
    b = torch.from_numpy(np.ascontiguousarray(b_lanes)).to(dev)
    d = torch.full((64, nres), float("nan"), dtype=torch.float32, device=dev)
    if sa is None:
        rc = getattr(lib, fn)(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                              ctypes.c_void_p(d.data_ptr()), _stream(torch))
    else:
        ta = torch.from_numpy(sa.astype(np.int32)).to(dev)
        tb = torch.from_numpy(sb.astype(np.int32)).to(dev)
        rc = getattr(lib, fn)(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                              ctypes.c_void_p(ta.data_ptr()), ctypes.c_void_p(tb.data_ptr()),
                              ctypes.c_void_p(d.data_ptr()), _stream(torch))
    assert rc == 0
    torch.cuda.synchronize()
    return d.cpu().numpy().astype(np.float64)


# Layout of the 16x16x128 form: lane l = i + 16 g holds row (or column) i;
# its bytes 0-15 are K = 16 g .. 16 g + 15 and bytes 16-31 are
# K = 64 + 16 g .. 64 + 16 g + 15.  Result register v of lane l is
# D[4 (l // 16) + v][l % 16].  With scales, the byte of lane i + 16 c scales
# row i's 32-element K block c (K = 32 c .. 32 c + 31).
def _k16(l, byte):
    g = l // 16
    return 16 * g + byte if byte < 16 else 64 + 16 * g + (byte - 16)


def _lanes16(mat):                      # mat [16 rows][128 k] codes -> [64][32]
    out = np.zeros((64, 32), np.uint8)
    for l in range(64):
        for byte in range(32):
            out[l, byte] = mat[l % 16, _k16(l, byte)]
    return out


def _unlanes16(d):                      # [64][4] -> D[16][16]
    D = np.zeros((16, 16))
    for l in range(64):
        for v in range(4):
            D[4 * (l // 16) + v, l % 16] = d[l, v]
    return D


# 32x32x64: lane l = i + 32 g holds row i; bytes 0-15 are K = 16 g .. +15 and
# bytes 16-31 are K = 32 + 16 g .. +15.  Result register v of lane l is
# D[8 (v // 4) + 4 (l // 32) + v % 4][l % 32].  The scale byte of lane
# i + 32 c scales row i's K block c (K = 32 c .. 32 c + 31).
def _k32(l, byte):
    g = l // 32
    return 16 * g + byte if byte < 16 else 32 + 16 * g + (byte - 16)


def _lanes32(mat):                      # [32][64] -> [64][32]
    out = np.zeros((64, 32), np.uint8)
    for l in range(64):
        for byte in range(32):
            out[l, byte] = mat[l % 32, _k32(l, byte)]
    return out


def _unlanes32(d):
    D = np.zeros((32, 32))
    for l in range(64):
        for v in range(16):
            D[8 * (v // 4) + 4 * (l // 32) + v % 4, l % 32] = d[l, v]
    return D


def _scaled(mat_codes, bytes_, rows):
    """Dequantize with the lane-held E8M0 bytes: lane i + rows*c scales row i,
    K block c."""
    out = e4m3.decode(mat_codes).copy()
    for l in range(64):
        i, c = l % rows, l // rows
        out[i, 32 * c:32 * c + 32] *= 2.0 ** (int(bytes_[l]) - 127)
    return out


def test_mfma16x16x128_layout(env):
    torch, lib = env
    g = np.random.default_rng(100)
    for _ in range(3):
        A, B = _codes(g, (16, 128)), _codes(g, (16, 128))
        d = _run_mfma(torch, lib, "probe_mfma16", _lanes16(A), _lanes16(B), 4)
        want = e4m3.decode(A) @ e4m3.decode(B).T
        assert np.array_equal(_unlanes16(d), want)


def test_mfma32x32x64_layout(env):
    torch, lib = env
    g = np.random.default_rng(101)
    for _ in range(3):
        A, B = _codes(g, (32, 64)), _codes(g, (32, 64))
        d = _run_mfma(torch, lib, "probe_mfma32", _lanes32(A), _lanes32(B), 16)
        want = e4m3.decode(A) @ e4m3.decode(B).T
        assert np.array_equal(_unlanes32(d), want)


def test_mfma16_scaled_e8m0(env):
    """The scale byte (op_sel 0 = bits 7:0; bits 31:8 ignored) of lane i + 16 c
    scales row i's K block c by 2^(byte - 127), for A and for B."""
    torch, lib = env
    g = np.random.default_rng(102)
    A, B = _codes(g, (16, 128)), _codes(g, (16, 128))
    sa = g.integers(125, 130, size=64)   # sums stay exact in FP32
    sb = g.integers(125, 130, size=64)
    d = _run_mfma(torch, lib, "probe_mfma16_scaled", _lanes16(A), _lanes16(B), 4,
                  sa | (0x55 << 8), sb | (0x33 << 8))     # upper bytes must be ignored
    assert np.array_equal(_unlanes16(d), _scaled(A, sa, 16) @ _scaled(B, sb, 16).T)
    # byte 127 on every lane is the unscaled product
    d1 = _run_mfma(torch, lib, "probe_mfma16_scaled", _lanes16(A), _lanes16(B), 4,
                   np.full(64, 127), np.full(64, 127))
    assert np.array_equal(_unlanes16(d1), e4m3.decode(A) @ e4m3.decode(B).T)


def test_mfma32_scaled_e8m0(env):
    torch, lib = env
    g = np.random.default_rng(103)
    A, B = _codes(g, (32, 64)), _codes(g, (32, 64))
    sa = g.integers(125, 130, size=64)   # sums stay exact in FP32
    sb = g.integers(125, 130, size=64)
    d = _run_mfma(torch, lib, "probe_mfma32_scaled", _lanes32(A), _lanes32(B), 16, sa, sb)
    assert np.array_equal(_unlanes32(d), _scaled(A, sa, 32) @ _scaled(B, sb, 32).T)


def _cvt_sweep():
    vals = np.unique(np.abs(e4m3.DECODE_TABLE[np.isfinite(e4m3.DECODE_TABLE)]))
    mids = (vals[:-1] + vals[1:]) / 2
    pts = [vals, mids]
    for m in mids.astype(np.float32):
        pts.append([np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))])
    pts.append([448.5, 463.9, 464.0, 464.1, 479.0, 480.0, 500.0, 512.0, 1e4, 3e38,
                1e-30, 2.0 ** -10, 2.0 ** -11, 1.4e-45, 0.0])
    g = np.random.default_rng(104)
    pts.append(g.standard_normal(4000) * 10.0 ** g.uniform(-4, 2.5, 4000))
    x = np.concatenate([np.ravel(p) for p in pts]).astype(np.float32)
    x = np.concatenate([x, -x])
    if x.size % 2:
        x = np.append(x, np.float32(1.0))
    return x


@pytest.mark.parametrize("clamp", [1, 0])
def test_cvt_pk_fp8_f32(env, clamp):
    torch, lib = env
    x = _cvt_sweep()
    tx = torch.from_numpy(x).cuda()
    out = torch.zeros(x.size // 2, dtype=torch.int32, device="cuda")
    rc = lib.probe_cvt_fp8(ctypes.c_void_p(tx.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                           ctypes.c_int(x.size // 2), ctypes.c_int(clamp), _stream(torch))
    assert rc == 0
    w = out.cpu().numpy().view(np.uint32)
    got = np.empty(x.size, np.uint8)
    got[0::2] = w & 0xFF
    got[1::2] = (w >> 8) & 0xFF
    want = e4m3.encode(x.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    msg = "; ".join(f"{x[i]!r}: hw {got[i]:#04x} oracle {want[i]:#04x}" for i in bad[:12])
    if clamp:
        assert bad.size == 0, msg
    else:
        # without a pre-clamp only out-of-range magnitudes may differ
        assert np.all(np.abs(x[bad]) > 448), msg
        print(f"\nunclamped cvt differs on {bad.size} values: {msg}")


def _bf16_sweep():
    g = np.random.default_rng(105)
    hi = g.integers(0, 1 << 16, 6000, dtype=np.uint32) << 16
    pts = [hi,                                    # BF16 values themselves
           hi | 0x8000,                           # exact ties: even and odd neighbours
           hi | 0x7FFF, hi | 0x8001,              # just below / above the tie
           g.integers(0, 1 << 32, 20000, dtype=np.uint64).astype(np.uint32),
           np.array([0x00000001, 0x00008000, 0x00018000, 0x007FFFFF, 0x00800000,  # subnormals
                     0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF,                       # overflow edge
                     0x7F800000, 0x3F808000, 0x3F818000, 0x00000000], np.uint32)]
    u = np.concatenate(pts).astype(np.uint32)
    u = np.concatenate([u, u ^ 0x80000000])       # both signs
    x = u.view(np.float32)
    x = x[np.isfinite(x) | np.isinf(x)]           # NaNs are checked on their own
    if x.size % 2:
        x = np.append(x, np.float32(1.0))
    return x


def test_cvt_pk_bf16_f32(env):
    torch, lib = env
    x = _bf16_sweep()
    tx = torch.from_numpy(x).cuda()
    out = torch.zeros(x.size // 2, dtype=torch.int32, device="cuda")
    rc = lib.probe_cvt_bf16(ctypes.c_void_p(tx.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                            ctypes.c_int(x.size // 2), _stream(torch))
    assert rc == 0
    w = out.cpu().numpy().view(np.uint32)
    got = np.empty(x.size, np.uint16)
    got[0::2] = w & 0xFFFF
    got[1::2] = w >> 16
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(got != want)[0]
    msg = "; ".join(f"{x.view(np.uint32)[i]:#010x}: hw {got[i]:#06x} torch {want[i]:#06x}"
                    for i in bad[:12])
    assert bad.size == 0, msg
    # NaN in, NaN out (exponent all ones, mantissa not zero)
    nan = np.array([np.nan, -np.nan], np.float32)
    tn = torch.from_numpy(nan).cuda()
    o = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert lib.probe_cvt_bf16(ctypes.c_void_p(tn.data_ptr()), ctypes.c_void_p(o.data_ptr()),
                              ctypes.c_int(1), _stream(torch)) == 0
    wn = int(o.cpu().numpy().view(np.uint32)[0])
    for h in (wn & 0xFFFF, wn >> 16):
        assert (h & 0x7F80) == 0x7F80 and (h & 0x7F) != 0, hex(h)


def _one_product(torch, lib, ca, cb, scaled=False):
    A = np.zeros((16, 128), np.uint8)
    B = np.zeros((16, 128), np.uint8)
    A[0, 5], B[0, 5] = ca, cb
    if scaled:
        d = _run_mfma(torch, lib, "probe_mfma16_scaled", _lanes16(A), _lanes16(B), 4,
                      np.full(64, 127), np.full(64, 127))
    else:
        d = _run_mfma(torch, lib, "probe_mfma16", _lanes16(A), _lanes16(B), 4)
    return _unlanes16(d)[0, 0]


@pytest.mark.parametrize("scaled", [False, True])
def test_mfma_keeps_e4m3_subnormal_inputs(env, scaled):
    """An e4m3 subnormal operand (exponent field 0, mantissa m != 0, value
    m * 2^-9) times a normal one contributes its exact product: the FP8 MFMA
    does not flush it.  A product of two subnormals (m1 m2 2^-18) must come out
    either exact or zero; which one is printed."""
    torch, lib = env
    assert _one_product(torch, lib, 0x08, 0x38, scaled) == 2.0 ** -6      # normal x 1
    assert _one_product(torch, lib, 0x88, 0x40, scaled) == -(2.0 ** -5)
    for sub in (0x01, 0x04, 0x07, 0x81):
        val = e4m3.decode_code(sub)
        for other, oval in ((0x38, 1.0), (0x48, 4.0), (0xB0, -0.5)):
            got = _one_product(torch, lib, sub, other, scaled)
            assert got == val * oval, f"code {sub:#04x} x {oval} gave {got!r}"
            got = _one_product(torch, lib, other, sub, scaled)
            assert got == val * oval, f"{oval} x code {sub:#04x} gave {got!r}"
    seen = []
    for ca, cb in ((0x01, 0x01), (0x07, 0x05), (0x84, 0x03)):
        want = e4m3.decode_code(ca) * e4m3.decode_code(cb)
        got = _one_product(torch, lib, ca, cb, scaled)
        assert got in (want, 0.0), f"{ca:#04x} x {cb:#04x} gave {got!r}, exact {want!r}"
        seen.append("exact" if got == want else "zero")
    print(f"\nsubnormal x subnormal products (scaled={scaled}): {seen}")


def test_mfma_internal_sum_informational(env):
    """126 products of 2^-12 (normal operands) then +-448*448 at the end of the
    128-K chunk: an exact accumulator returns 126 * 2^-12, a left-to-right FP32
    one 2^-5.  Either is inside the derived bound (128 roundings of 2^-24)."""
    torch, lib = env
    A = np.zeros((16, 128), np.uint8)
    B = np.zeros((16, 128), np.uint8)
    A[0, :] = 0x08                     # 2^-6
    B[0, :] = 0x08
    A[0, 126], A[0, 127] = 0x7E, 0xFE  # +-448
    B[0, 126], B[0, 127] = 0x7E, 0x7E
    d = _run_mfma(torch, lib, "probe_mfma16", _lanes16(A), _lanes16(B), 4)
    got = _unlanes16(d)[0, 0]
    exact = 126 * 2.0 ** -12
    print(f"\nMFMA chunk sum: got {got!r}, exact {exact!r}")
    assert abs(got - exact) <= 128 * 2.0 ** -24 * (2 * 448 * 448 + 126 * 2.0 ** -12)


def _row0_dot(torch, lib, terms):
    """D[0][0] of one 16x16x128 MFMA whose row 0 of A and column 0 of B hold
    the given (k, code_a, code_b) terms and zeros elsewhere."""
    A = np.zeros((16, 128), np.uint8)
    B = np.zeros((16, 128), np.uint8)
    for k, ca, cb in terms:
        A[0, k], B[0, k] = ca, cb
    return _unlanes16(_run_mfma(torch, lib, "probe_mfma16", _lanes16(A), _lanes16(B), 4))[0, 0]


def test_mfma_alignment_informational(env):
    """How far below the largest product of a 16-wide K group a small product
    survives: +256 and -256 at K = 0, 1 cancel, and a third product x at K = 2
    (same group) or K = 16 (next group) should come out as x.  Printed as a
    table of log2(|x|) -> result / x for x = 2^-j and +-1.5 * 2^-j."""
    torch, lib = env
    enc = lambda v: int(e4m3.encode(float(v)))
    big, nbig, one = enc(256.0), enc(-256.0), enc(1.0)
    rows = []
    for j in range(0, 19):
        a, b = min(j, 9), j - min(j, 9)              # 2^-a (subnormal below 2^-6) times 2^-b
        line = [f"2^-{j:<2d}"]
        for mant, sign in ((1.0, 1), (1.5, 1), (1.5, -1)):
            a2, b2 = (a, b) if mant == 1.0 else (min(j, 8), j - min(j, 8))
            if b2 > 9:                               # 1.5 * 2^-j not a product of two codes
                line.append(f"{'-':>8s} {'-':>8s}")
                continue
            ca, cb = enc(sign * mant * 2.0 ** -a2), enc(2.0 ** -b2)
            want = sign * mant * 2.0 ** -j
            assert e4m3.decode_code(ca) * e4m3.decode_code(cb) == want
            same = _row0_dot(torch, lib, [(0, big, one), (1, nbig, one), (2, ca, cb)])
            other = _row0_dot(torch, lib, [(0, big, one), (1, nbig, one), (16, ca, cb)])
            line.append(f"{same / want:8.4f} {other / want:8.4f}")
        rows.append(" | ".join(line))
    print("\nx = 2^-j | (+1.0x) same-group next-group | (+1.5x) | (-1.5x), big products 2^8")
    print("\n".join(rows))


def _row0_dot_acc(torch, lib, form, terms, c00):
    """D[0][0] of one MFMA (16x16x128 or 32x32x64) whose accumulator input is
    zero except C[0][0] = c00, with the given (k, code_a, code_b) terms in row
    0 of A and column 0 of B."""
    rows, kk, nres = (16, 128, 4) if form == 16 else (32, 64, 16)
    A = np.zeros((rows, kk), np.uint8)
    B = np.zeros((rows, kk), np.uint8)
    for k, ca, cb in terms:
        A[0, k], B[0, k] = ca, cb
    lanes, unlanes = (_lanes16, _unlanes16) if form == 16 else (_lanes32, _unlanes32)
    C = np.zeros((64, nres), np.float32)
    C[0, 0] = c00                      # D[0][0] sits in register 0 of lane 0 in both forms
    dev = "cuda"
    a = torch.from_numpy(np.ascontiguousarray(lanes(A))).to(dev)
    b = torch.from_numpy(np.ascontiguousarray(lanes(B))).to(dev)
    c = torch.from_numpy(C).to(dev)
    d = torch.full((64, nres), float("nan"), dtype=torch.float32, device=dev)
    fn = getattr(lib, f"probe_mfma{form}_acc")
    assert fn(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
              ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(d.data_ptr()), _stream(torch)) == 0
    torch.cuda.synchronize()
    return unlanes(d.cpu().numpy().astype(np.float64))[0, 0]


@pytest.mark.parametrize("form", [16, 32])
def test_mfma_accumulator_input_is_added_in_fp32(env, form):
    """The accumulator input C stays out of the products' alignment window:
    C = 2^8 plus a product x = 2^-j gives exactly 2^8 + x for j = 0..15 (all
    representable in FP32), and C = 2^-10 survives beside a product 2^8.  So
    chaining MFMAs through C costs only FP32 rounding."""
    torch, lib = env
    enc = lambda v: int(e4m3.encode(float(v)))
    for j in range(16):
        a = min(j, 9)
        ca, cb = enc(2.0 ** -a), enc(2.0 ** -(j - a))
        got = _row0_dot_acc(torch, lib, form, [(0, ca, cb)], 256.0)
        assert got == 256.0 + 2.0 ** -j, f"form {form}, j={j}: {got!r}"
    got = _row0_dot_acc(torch, lib, form, [(0, enc(256.0), enc(1.0))], 2.0 ** -10)
    assert got == 256.0 + 2.0 ** -10


def test_copy_bandwidth_informational(env):
    torch, lib = env
    n = 1 << 28                        # 1 GiB of float32
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    st = _stream(torch)
    for _ in range(3):
        assert lib.probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                              ctypes.c_size_t(n // 4), ctypes.c_int(4096), st) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        lib.probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                       ctypes.c_size_t(n // 4), ctypes.c_int(4096), st)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    print(f"\ncopy 1 GiB: {ms:.3f} ms, {2 * 4 * n / ms / 1e6:.1f} GB/s (read+write)")
    assert torch.equal(dst[:1024], src[:1024])
