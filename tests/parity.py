"""Tolerances for comparing the HIP GEMMs with the float64 oracle.

FP32 outputs, the stated bar:   |g - C| <= 1e-3 * S + 1e-6,  S = sum_k |a_k b_k|.
FP32 outputs, the derived bar:  |g - C| <= eps_acc(K) * S + S_trunc  with
    eps_acc(K) = 2 * (128 + K/128 + 2) * 2^-24.
  Besides the alignment cut described next, the MFMA's group sums, the
  K/128 per-block FMAs and the two scale products give at most
  128 + K/128 + 2 FP32 roundings of relative size 2^-24 on partial sums
  bounded by S (a generous count); the factor 2 leaves room for
  non-nearest rounding.  A mis-indexed scale or a dropped K block is off by
  far more, so this bar is what catches them.
  The MXFP8 path is held to the stated bar only in FP32: it accumulates
  through the MFMA's C operand with E8M0 scales that may differ by many
  binades inside one 128-wide K chunk, and that internal sum loses more than
  the model below (measured up to ~5e-5 * S for exponent spreads of +-20
  binades, 20x inside the stated bar).
Inside one FP8 MFMA the 128 products are summed in groups of 16 consecutive
  K; within a group every product is aligned to the group's largest one and
  cut to 13 bits below it (the probe tests print this: with +-2^8 in a group,
  2^-5 survives, 1.5 * 2^-5 comes out as 2^-5 and 2^-6 vanishes, while the
  next group is unaffected).  Subnormal operands are otherwise used exactly.
  The derived bar therefore adds S_trunc = sum over groups of (sum_k
  |p_k| mod LSB_g, plus LSB_g once if any product is cut), LSB_g =
  2^(floor(log2 max_k |p_k|) - 12) (one bit of margin over the probe), with
  p_k the unscaled code products, times the group's scale product.
  S_trunc costs K products per output, so it is a lazy term (Trunc): every
  output is first held to eps_acc * S alone, and S_trunc is computed exactly
  for the outputs that exceed that, at any problem size.  No output is
  exempt from the derived bar.
BF16 outputs: within 1 BF16 ulp of the oracle rounded to BF16 (ordered-bit
  distance, +0 == -0), or, where FP32 accumulation alone moves a value near
  cancellation by more than that, |g - C| <= ulp_bf16(RNE(C)) + eps_acc * S
  + S_trunc, with S_trunc computed for exactly those outputs.  Such outputs
  are expected only near cancellation (|C| within a few hundred times the
  FP32 accumulation error); their count is printed and must stay below
  0.5% of the outputs (plus 4), so a systematic error cannot hide behind the
  second rule.
Fused gated epilogue (FP8 codes and 1x128 scales of h = silu(gate) * up):
  the GPU's gate and up values lie within the GEMM bar T = eps_acc * S +
  S_trunc of the oracle's; silu has slope below 1.1, so its h lies within
  Eh = 1.1 Tg (|up| + Tu) + |silu(gate)| Tu, plus 2^-20 relative for the
  FP32 evaluation.  Quantization is monotone, so the GPU's scale must lie
  between the scales of the smallest and largest amax that h can have, and
  each code, taken with the GPU's own scale, between the codes of
  (h - Eh) / s and (h + Eh) / s.  Codes and scales are integer-valued
  decisions made from FP32 values the oracle cannot reproduce bit for bit;
  these bounds are what any correct implementation satisfies.  The bounds
  are first taken with S_trunc = 0 (narrower); only groups that fail them
  are re-checked with S_trunc computed.
"""
import numpy as np

from oracle import activation, e4m3, gemm
from oracle.gemm import round_to_bf16

# outputs allowed off the 1-ulp rule (near cancellation), as a fraction
FALLBACK_FRACTION = 0.005


def eps_acc(K):
    return 2.0 * (128 + K // 128 + 2) * 2.0 ** -24


def bf16_bits_to_f32(bits):
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def _ordered(f32):
    u = np.asarray(f32, np.float32).view(np.int32).astype(np.int64)
    return np.where(u < 0, -(u & 0x7FFFFFFF), u)


def bf16_ulp_distance(a, b):
    """Distance in BF16 steps between BF16 values held as float32 (their low
    16 bits are zero), +0 == -0."""
    return np.abs(_ordered(a) - _ordered(b)) >> 16


# --------------------------------------------------------------- S_trunc
def trunc_pairs(qa, qb, group_scale, ms, ns):
    """S_trunc (module text) of the outputs (ms[i], ns[i]) of C = A B^T, from
    the e4m3 codes qa [M, K] and qb [N, K]; group_scale(ms, ns, g) gives the
    scale product of 16-group g for those outputs."""
    qa, qb = np.asarray(qa), np.asarray(qb)
    K = qa.shape[1]
    ms, ns = np.asarray(ms, np.int64), np.asarray(ns, np.int64)
    out = np.zeros(ms.size)
    if ms.size == 0:
        return out
    G = K // 16
    gi = np.arange(G)
    step = max(1, (1 << 22) // K)
    for c in range(0, ms.size, step):
        m, n = ms[c:c + step], ns[c:c + step]
        va = e4m3.DECODE_TABLE[qa[m].astype(np.intp)]
        vb = e4m3.DECODE_TABLE[qb[n].astype(np.intp)]
        p = np.abs(va * vb).reshape(-1, G, 16)              # exact dyadic products
        gmax = p.max(axis=2)
        live = gmax > 0
        e = np.floor(np.log2(np.where(live, gmax, 1.0)))
        lsb = np.where(live, np.ldexp(1.0, (e - 12).astype(np.int64)), 0.0)
        r = np.fmod(p, np.where(live, lsb, 1.0)[..., None]).sum(axis=2)
        bound = np.where(live, r + np.where(r > 0, lsb, 0.0), 0.0)
        out[c:c + step] = (bound * group_scale(m[:, None], n[:, None], gi[None, :])).sum(axis=1)
    return out


def trunc_bound(qa, qb, group_scale):
    """S_trunc of every output of C = A B^T (small problems; CPU pins)."""
    M, N = np.asarray(qa).shape[0], np.asarray(qb).shape[0]
    m, n = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    return trunc_pairs(qa, qb, group_scale, m.ravel(), n.ravel()).reshape(M, N)


class Trunc:
    """The S_trunc term of an output array, computed only where asked:
    fn(flat indices into `shape`) -> float64 values."""

    def __init__(self, shape, fn):
        self.shape = tuple(int(s) for s in shape)
        self._fn = fn

    @classmethod
    def zeros(cls, shape):
        return cls(shape, lambda idx: np.zeros(np.asarray(idx).size))

    @classmethod
    def of(cls, value, shape):
        """A Trunc for `value`: a Trunc (checked against shape), or an array /
        scalar broadcast to shape (tests of the helpers)."""
        if isinstance(value, Trunc):
            assert value.shape == tuple(shape), (value.shape, shape)
            return value
        arr = np.broadcast_to(np.asarray(value, np.float64), shape).ravel()
        return cls(shape, lambda idx: arr[idx])

    def at(self, flat_idx):
        return np.asarray(self._fn(np.asarray(flat_idx, np.int64)), np.float64)

    def __getitem__(self, key):
        base = np.arange(int(np.prod(self.shape)), dtype=np.int64).reshape(self.shape)[key]
        base = np.asarray(base)
        flat = base.ravel()
        return Trunc(base.shape, lambda idx: self._fn(flat[idx]))


class TruncRows(Trunc):
    """An output array whose row sets (first axis) take their S_trunc from
    separate Trunc objects (one per expert); unset rows have S_trunc = 0."""

    def __init__(self, shape):
        super().__init__(shape, self._eval)
        self._part = np.full(self.shape[0], -1, np.int64)
        self._local = np.zeros(self.shape[0], np.int64)
        self._parts = []

    def __setitem__(self, rows, t):
        idx = np.arange(self.shape[0])[rows]
        assert t.shape[0] == idx.size and t.shape[1:] == self.shape[1:], (t.shape, idx.size)
        self._part[idx] = len(self._parts)
        self._local[idx] = np.arange(idx.size)
        self._parts.append(t)

    def _eval(self, idx):
        inner = int(np.prod(self.shape[1:]))
        r, c = idx // inner, idx % inner
        out = np.zeros(idx.size)
        for p, t in enumerate(self._parts):
            sel = self._part[r] == p
            if sel.any():
                out[sel] = t.at(self._local[r[sel]] * inner + c[sel])
        return out


# --------------------------------------------------------------- checks
def check_f32(g, C, S, K, where="", derived=True, S_flush=0.0):
    """FP32 outputs: the stated bar on every output, and (derived=True) the
    derived bar eps_acc * S + S_trunc on every output, S_trunc computed for
    the outputs above eps_acc * S."""
    g = np.asarray(g, np.float64)
    C, S = np.asarray(C, np.float64), np.asarray(S, np.float64)
    assert np.all(np.isfinite(g)), f"{where}: non-finite output"
    err = np.abs(g - C)
    stated = err <= 1e-3 * S + 1e-6
    assert stated.all(), f"{where}: {np.count_nonzero(~stated)} outside 1e-3*S+1e-6; max err/S " \
                         f"{np.max(err / np.maximum(S, 1e-30)):.3e}"
    if derived:
        over = np.flatnonzero(err > eps_acc(K) * S)
        if over.size:
            F = Trunc.of(S_flush, g.shape).at(over)
            bad = err.ravel()[over] > eps_acc(K) * S.ravel()[over] + F + 1e-30
            assert not bad.any(), f"{where}: {np.count_nonzero(bad)} outside eps_acc*S+S_trunc " \
                                  f"(eps={eps_acc(K):.2e}); max err/S " \
                                  f"{np.max(err / np.maximum(S, 1e-30)):.3e}"
    return float(np.max(err / np.maximum(S, 1e-30))) if err.size else 0.0


def check_bf16(g_bits, C, S, K, where="", S_flush=0.0):
    """BF16 outputs: 1 ulp of RNE(C) on every output; the outputs that miss
    it must meet ulp + eps_acc * S + S_trunc (S_trunc computed for each of
    them) and be few.  Returns their count."""
    g = bf16_bits_to_f32(g_bits).astype(np.float64)
    C, S = np.asarray(C, np.float64), np.asarray(S, np.float64)
    assert np.all(np.isfinite(g)), f"{where}: non-finite output"
    ref = round_to_bf16(C)
    dist = bf16_ulp_distance(g.astype(np.float32), ref)
    miss = np.flatnonzero(dist > 1)
    if miss.size:
        _, e = np.frexp(np.abs(ref.ravel()[miss].astype(np.float64)))
        ulp = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
        F = Trunc.of(S_flush, g.shape).at(miss)
        err = np.abs(g.ravel()[miss] - C.ravel()[miss])
        bad = err > ulp + eps_acc(K) * S.ravel()[miss] + F
        assert not bad.any(), f"{where}: {np.count_nonzero(bad)} BF16 outputs fail " \
                              f"(max ulp dist {dist.max()})"
        limit = FALLBACK_FRACTION * g.size + 4
        assert miss.size <= limit, f"{where}: {miss.size} of {g.size} BF16 outputs are off " \
                                   f"the 1-ulp rule (limit {limit:.0f})"
    print(f"{where}: {miss.size} of {g.size} BF16 outputs off the 1-ulp rule", flush=True)
    return int(miss.size)


def ref_blockscaled(qa, sa, qb, sb):
    """Oracle (C, S) of the block-scaled product plus its S_trunc term."""
    A = gemm.dequant_1x128(qa, sa)
    B = gemm.dequant_128x128(qb, sb)
    C, S = gemm.matmul_with_base(A, B)
    sa64, sb64 = np.abs(np.asarray(sa, np.float64)), np.abs(np.asarray(sb, np.float64))
    scale = lambda m, n, g: sa64[g // 8, m] * sb64[n // 128, g // 8]
    N = C.shape[1]
    qa, qb = np.asarray(qa), np.asarray(qb)
    return C, S, Trunc(C.shape, lambda idx: trunc_pairs(qa, qb, scale, idx // N, idx % N))


def ref_mx(qa, ea, qb, eb):
    """Oracle (C, S, S_trunc) of one MX group: qa [M, K], ea [M, K/32], ..."""
    A = gemm.dequant_mx(qa, ea)
    B = gemm.dequant_mx(qb, eb)
    C, S = gemm.matmul_with_base(A, B)
    ea64 = np.asarray(ea, np.float64) - 127.0
    eb64 = np.asarray(eb, np.float64) - 127.0
    scale = lambda m, n, g: np.exp2(ea64[m, g // 2] + eb64[n, g // 2])
    N = C.shape[1]
    qa, qb = np.asarray(qa), np.asarray(qb)
    return C, S, Trunc(C.shape, lambda idx: trunc_pairs(qa, qb, scale, idx // N, idx % N))


def check_swiglu_quant(q, s, C, S, F, K, where=""):
    """q uint8 [R, H] and s float32 [H/128, R]: the GPU's codes and scales of
    h for R rows and H columns of h; C, S [R, 2H]: the oracle's product with
    the interleaved W1 (same column blocks, same order) and its base; F the
    S_trunc term of that product (a Trunc or an array)."""
    C, S = np.asarray(C, np.float64), np.asarray(S, np.float64)
    R, N2 = C.shape
    H = N2 // 2
    s_gpu = np.asarray(s, np.float32).astype(np.float64).T          # [R, H/128]
    assert s_gpu.shape == (R, H // 128)
    dq = e4m3.decode(np.asarray(q, np.uint8))
    h = activation.swiglu_interleaved(C)

    def outcome(T):
        g, u = activation.gate_up_of(C)
        Tg, Tu = activation.gate_up_of(T)
        E0 = 1.1 * Tg * (np.abs(u) + Tu) + np.abs(activation.silu(g)) * Tu
        Eh = E0 + 2.0 ** -20 * (np.abs(h) + E0)
        ha = np.abs(h).reshape(R, H // 128, 128)
        Eg = Eh.reshape(R, H // 128, 128)
        amax_lo = np.maximum(ha - Eg, 0.0).max(axis=2)
        amax_hi = (ha + Eg).max(axis=2)
        s_lo = np.float32(amax_lo / 448.0).astype(np.float64) * (1 - 2.0 ** -30)
        s_hi = np.float32(amax_hi / 448.0).astype(np.float64) * (1 + 2.0 ** -30)
        ok_s = ((s_gpu >= s_lo) & (s_gpu <= s_hi) & (amax_lo > 0)) | ((amax_lo == 0) & (
            (s_gpu == 1.0) | ((s_gpu <= s_hi) & (amax_hi > 0))))
        sf = np.repeat(s_gpu, 128, axis=1)
        lo_v = (h - Eh) / sf
        hi_v = (h + Eh) / sf
        lo_v = lo_v - np.abs(lo_v) * 2.0 ** -30
        hi_v = hi_v + np.abs(hi_v) * 2.0 ** -30
        lo = e4m3.round_to_e4m3_value(np.clip(lo_v, -1e4, 1e4))
        hi = e4m3.round_to_e4m3_value(np.clip(hi_v, -1e4, 1e4))
        ok_q = (dq >= lo) & (dq <= hi)
        return ok_s, ok_q

    ok_s, ok_q = outcome(eps_acc(K) * S)
    # groups (row, 128-column block of h) with a failing scale or code are
    # re-checked with S_trunc of their gate and up elements
    bad_grp = ~ok_s | ~ok_q.reshape(R, H // 128, 128).all(axis=2)
    if bad_grp.any():
        Ft = Trunc.of(F, C.shape)
        r, j = np.nonzero(bad_grp)
        cols = np.concatenate([np.arange(256 * jj, 256 * jj + 256) for jj in j])
        rows = np.repeat(r, 256)
        T = eps_acc(K) * S
        T[rows, cols] += Ft.at(rows * N2 + cols)
        ok_s, ok_q = outcome(T)
    assert ok_s.all(), f"{where}: {np.count_nonzero(~ok_s)} scales outside their bounds"
    assert ok_q.all(), f"{where}: {np.count_nonzero(~ok_q)} of {ok_q.size} codes outside their bounds"
    sf = np.repeat(s_gpu, 128, axis=1)
    return int(np.count_nonzero(dq != e4m3.round_to_e4m3_value(np.float32(h / sf))))


def ref_kgrouped(qa, sa, qb, sb, offsets):
    """Oracle (C, S, S_trunc) [G, M, N] of the K-grouped GEMM (1x128 scales
    on both operands)."""
    from oracle import backward
    C, S = backward.grouped_k(qa, sa, qb, sb, offsets)
    G, M, N = C.shape
    sa64, sb64 = np.abs(np.asarray(sa, np.float64)), np.abs(np.asarray(sb, np.float64))
    off = np.asarray(offsets, np.int64)
    qa, qb = np.asarray(qa), np.asarray(qb)

    def fn(idx):
        g, rem = idx // (M * N), idx % (M * N)
        out = np.zeros(idx.size)
        for gg in np.unique(g):
            k0, k1 = int(off[gg]), int(off[gg + 1])
            if k1 <= k0:
                continue
            sel = g == gg
            b0 = k0 // 128
            scale = lambda m, n, gi, b0=b0: sa64[b0 + gi // 8, m] * sb64[b0 + gi // 8, n]
            out[sel] = trunc_pairs(qa[:, k0:k1], qb[:, k0:k1], scale, rem[sel] // N, rem[sel] % N)
        return out

    return C, S, Trunc(C.shape, fn)
