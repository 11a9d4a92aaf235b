"""The seeded generators: deterministic, and with the structure each workload
asks for (row modifiers, routing without replacement, padded layout)."""
import numpy as np

import inputs
import moe_cases


def test_dense_cases_deterministic_and_shaped():
    a1, b1 = inputs.dense_case("tiny")
    a2, b2 = inputs.dense_case("tiny")
    assert a1.dtype == np.float32 and a1.shape == (64, 512) and b1.shape == (256, 512)
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2)
    big = np.abs(a1).max(axis=1)
    assert (big > 50).sum() == 1                     # exactly one x100 outlier row
    a, b = inputs.dense_case("skinny_a", N=256)
    assert a.shape == (64, 7168) and b.shape == (256, 7168)
    assert abs(b.std() * np.sqrt(7168) - 1) < 0.05   # N(0, 1/K)
    rms = np.sqrt((a.astype(np.float64) ** 2).mean(axis=1))
    assert rms.min() > 0.005 and rms.max() < 12      # log-uniform row factors in [0.01, 10]


def test_routing_distinct_and_skewed():
    r = inputs.zipf_topk_routing(3, 4096, 32, 8)
    assert r.shape == (4096, 8)
    assert all(len(set(row)) == 8 for row in r[:200])
    counts = np.bincount(r.ravel(), minlength=32)
    assert counts[0] > counts[31] * 2 and counts.sum() == 4096 * 8


def test_contiguous_layout_padding_and_order():
    r = inputs.zipf_topk_routing(3, 1000, 8, 2)
    lay = moe_cases.contiguous_layout(r, 8)
    assert lay.m_total % 128 == 0
    assert lay.block_expert.shape == (lay.m_total // 128,)
    assert np.all(np.diff(lay.block_expert) >= 0)
    assert lay.valid_rows == 2000
    for e in range(8):
        rows = np.repeat(lay.block_expert == e, 128)
        toks = lay.row_token[rows]
        live = toks[toks >= 0]
        assert live.size == lay.counts[e]
        assert np.all(np.diff(live) > 0)              # ascending token order
        assert np.all(toks[live.size:] == -1)         # padding at the end
    x = np.arange(1000 * 128, dtype=np.float32).reshape(1000, 128)
    a = moe_cases.gather_rows(x, lay.row_token)
    assert np.all(a[lay.row_token < 0] == 0)
    live = lay.row_token >= 0
    assert np.array_equal(a[live], x[lay.row_token[live]])


def test_contiguous_sources_shapes_and_determinism():
    c = inputs.ContiguousCase(tokens=300, hidden=256, inter=384, inter2=128, experts=5, topk=2,
                              workload=31)
    ids, x, w1, w2 = inputs.contiguous_sources(c)
    ids2, x2, _, _ = inputs.contiguous_sources(c)
    assert ids.shape == (300, 2) and x.shape == (300, 256)
    assert w1.shape == (5, 384, 256) and w2.shape == (5, 256, 128)
    assert np.array_equal(ids, ids2) and np.array_equal(x, x2)
    assert inputs.contiguous_a2(c, 640).shape == (640, 128)


def test_masked_case_counts_and_junk():
    c = inputs.MaskedCase(experts=6, cap=64, N=128, K=256)
    valid, a, b = inputs.masked_case(c)
    assert valid.shape == (6,) and valid.min() >= 0 and valid.max() <= 64
    for e in range(6):
        assert np.all(np.isfinite(a[e]))
        if valid[e] < 64:
            assert np.abs(a[e, valid[e]:]).max() > 1e20
