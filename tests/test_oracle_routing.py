"""Pins for the oracle's routing -> contiguous layout step (CPU only): a
hand-worked example, invariants on random routings, degenerate cases, and
the gather+quantize reduced to the 1x128 quantizer."""
import numpy as np

from oracle import routing, scaling


def test_hand_worked_example():
    # 5 tokens, top-2 of 3 experts; expert 1 gets no token, token 3 repeats
    # expert 2, token 4 carries an out-of-range id.
    ids = np.array([[0, 2], [2, 0], [0, 0], [2, 2], [9, 0]])
    rt, be, off, cnt = routing.contiguous_layout(ids, 3, 512)
    assert cnt.tolist() == [4, 0, 3]
    assert off.tolist() == [0, 128, 128, 256]
    assert rt[:5].tolist() == [0, 1, 2, 4, -1]
    assert np.all(rt[4:128] == -1)
    assert rt[128:131].tolist() == [0, 1, 3] and np.all(rt[131:] == -1)
    assert be.tolist() == [0, 2, -1, -1]


def test_invariants_on_random_routings():
    g = np.random.default_rng(500)
    for T, k, E in [(300, 2, 6), (1000, 8, 32), (129, 2, 3)]:
        ids = np.argsort(g.random((T, E)), axis=1)[:, :k]        # distinct per token
        cap = routing.capacity(T, k, E)
        rt, be, off, cnt = routing.contiguous_layout(ids, E, cap)
        assert cnt.sum() == T * k and np.all(off % 128 == 0)
        for e in range(E):
            run = rt[off[e]:off[e + 1]]
            toks = run[run >= 0]
            assert toks.size == cnt[e]
            assert np.array_equal(toks, np.sort(toks))           # ascending token order
            assert np.all(run[cnt[e]:] == -1)                    # padding after the tokens
            assert np.array_equal(np.sort(toks), np.nonzero((ids == e).any(axis=1))[0])
            assert np.all(be[off[e] // 128:off[e + 1] // 128] == e)
        assert np.all(be[off[E] // 128:] == -1) and np.all(rt[off[E]:] == -1)


def test_capacity_is_enough_for_the_worst_routing():
    T, k, E = 100, 3, 5
    cap = routing.capacity(T, k, E)
    ids = np.tile(np.arange(k), (T, 1))                           # 3 experts get 100 each
    rt, be, off, cnt = routing.contiguous_layout(ids, E, cap)
    assert off[E] <= cap and cnt.tolist() == [100, 100, 100, 0, 0]


def test_gather_quantize_is_the_quantizer_on_gathered_rows():
    g = np.random.default_rng(501)
    x = g.standard_normal((40, 256)).astype(np.float32)
    ids = g.integers(0, 4, (40, 2))
    rt, be, off, cnt = routing.contiguous_layout(ids, 4, routing.capacity(40, 2, 4))
    q, s = routing.gather_quantize(x, rt)
    for r in (0, int(off[1]), int(off[2]) + 1):
        if rt[r] >= 0:
            qr, sr = scaling.quantize_1x128(x[rt[r]][None])
            assert np.array_equal(q[r], qr[0]) and np.array_equal(s[:, r], sr[:, 0])
    pad = rt < 0
    assert np.all(q[pad] == 0) and np.all(s[:, pad] == 1.0)


def test_token_rows_hand_worked():
    """The inverse map of the hand-worked routing: expert 0 holds tokens
    0, 1, 2, 4 in rows 0..3, expert 2 holds tokens 0, 1, 3 in rows 128..130;
    repeated ids and the out-of-range id 9 get -1."""
    ids = np.array([[0, 2], [2, 0], [0, 0], [2, 2], [9, 0]])
    tr = routing.token_rows(ids, 3, 512)
    assert tr.tolist() == [[0, 128], [129, 1], [2, -1], [130, -1], [-1, 3]]


def test_token_rows_invert_the_row_map():
    g = np.random.default_rng(12)
    for T, k, E in [(200, 4, 7), (97, 8, 3), (300, 2, 64)]:
        ids = g.integers(-1, E + 1, size=(T, k))
        m_cap = routing.capacity(T, k, E)
        rt, be, off, cnt = routing.contiguous_layout(ids, E, m_cap)
        tr = routing.token_rows(ids, E, m_cap)
        live = tr >= 0
        # every row that holds a token is named exactly once, by that token,
        # at a position whose id is the row's expert
        assert np.array_equal(np.sort(tr[live]), np.sort(np.nonzero(rt >= 0)[0]))
        t_idx, j_idx = np.nonzero(live)
        assert np.array_equal(rt[tr[live]], t_idx)
        assert np.array_equal(be[tr[live] // 128], ids[t_idx, j_idx])
        # -1 exactly where the id is out of range or repeats an earlier one
        for t in range(T):
            seen = set()
            for j in range(k):
                e = int(ids[t, j])
                dead = not (0 <= e < E) or e in seen
                seen.add(e)
                assert (tr[t, j] == -1) == dead
