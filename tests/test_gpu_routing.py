"""Top-k routing -> contiguous layout + 1x128 quantize on the GPU against the
oracle (oracle/routing.py).  Index outputs and quantized bytes are integer
results: bit-exact."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp8_amd as fg8
import inputs
from oracle import gemm, routing, scaling
from parity import TruncRows, check_bf16, ref_blockscaled

pytestmark = pytest.mark.gpu


def _to_bf16(x):
    """float32 -> nearest bfloat16 bits (ties to even) and the float32 they
    hold; the test's inputs only (finite x)."""
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r, (r.astype(np.uint32) << 16).view(np.float32)


def _source(x, bf16):
    """(device tensor, float32 values the oracle sees)."""
    if bf16:
        bits, wide = _to_bf16(x)
        return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16), wide
    return torch.from_numpy(x).cuda(), x


def _run(x, ids, experts, m_cap=None, bf16=False):
    tx, wide = _source(np.ascontiguousarray(x, dtype=np.float32), bf16)
    tids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    print(f"routing: tokens={x.shape[0]} hidden={x.shape[1]} topk={ids.shape[1]} "
          f"experts={experts} m_cap={m_cap} bf16={bf16}", flush=True)
    out = fg8.moe_contiguous_layout_fp8(tx, tids, experts, m_cap)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}, wide


def _check_layout(got, ids, experts, m_cap):
    rt, be, off, cnt = routing.contiguous_layout(ids, experts, m_cap)
    assert np.array_equal(got["token_row"], routing.token_rows(ids, experts, m_cap))
    assert np.array_equal(got["row_token"], rt)
    assert np.array_equal(got["block_expert"], be)
    assert np.array_equal(got["expert_offsets"], off)
    assert np.array_equal(got["expert_counts"], cnt)
    return rt


def _check_rows(got, wide, rt, rows):
    q, s = routing.gather_quantize(wide, rt[rows])
    assert np.array_equal(got["q"][rows], q)
    assert np.array_equal(got["sa"][:, rows].view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("bf16", [False, True])
def test_hand_worked_example(dev, bf16):
    """The routing of the oracle's hand-worked pin: a repeated id, an
    out-of-range id and an expert nobody picks."""
    ids = np.array([[0, 2], [2, 0], [0, 0], [2, 2], [9, 0]], np.int32)
    x = np.random.default_rng(401).standard_normal((5, 256)).astype(np.float32)
    got, wide = _run(x, ids, 3, 512, bf16)
    rt = _check_layout(got, ids, 3, 512)
    assert list(got["expert_counts"]) == [4, 0, 3]
    _check_rows(got, wide, rt, np.arange(512))


EDGE = {
    # tokens, hidden, topk, experts, m_cap extra rows, id generator
    "one_token": (1, 128, 1, 1, 0, "uniform"),
    "ragged_bad_ids": (1000, 384, 4, 7, 0, "bad"),
    "one_hot_expert": (2050, 256, 2, 5, 0, "single"),
    "spare_capacity": (333, 128, 3, 4, 512, "uniform"),
    "max_experts": (300, 128, 8, 1024, 0, "uniform"),
    "topk_above_experts": (129, 128, 6, 3, 0, "uniform"),
    # more than 64 destinations per token and rows longer than one load chunk
    # of the scatter kernel (8192 BF16 / 4096 FP32 columns): its row-index
    # reloads between chunks and between groups of 64 destinations
    "topk_80_long_rows": (40, 8576, 80, 5, 0, "uniform"),
}


def _ids(kind, tokens, topk, experts, seed):
    g = np.random.default_rng(seed)
    if kind == "uniform":
        return g.integers(0, experts, size=(tokens, topk)).astype(np.int32)
    if kind == "bad":   # repeats, negative and too-large ids mixed in
        ids = g.integers(-2, experts + 3, size=(tokens, topk)).astype(np.int32)
        ids[::7, 1] = ids[::7, 0]
        return ids
    ids = np.full((tokens, topk), 3, np.int32)   # every token to expert 3 (twice)
    return ids


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("name", list(EDGE))
def test_edge_routings(dev, name, bf16):
    tokens, hidden, topk, experts, extra, kind = EDGE[name]
    ids = _ids(kind, tokens, topk, experts, 402 + len(name))
    x = np.random.default_rng(403).standard_normal((tokens, hidden)).astype(np.float32)
    x[::5] *= 100.0
    m_cap = routing.capacity(tokens, topk, experts) + extra
    assert fg8.moe_capacity(tokens, topk, experts) == m_cap - extra
    got, wide = _run(x, ids, experts, m_cap, bf16)
    rt = _check_layout(got, ids, experts, m_cap)
    _check_rows(got, wide, rt, np.arange(m_cap))


def test_token_ranges_spanning_several_chunks(dev):
    """A top-128 routing of 5000 tokens: the kernels cut the token axis into
    their maximum number of ranges, each spanning more than one staged chunk
    of ids, so the cross-range and cross-chunk rank bookkeeping is exercised.
    The layout is checked whole, the quantized rows on a sample."""
    T, H, k, E = 5000, 128, 128, 6
    g = np.random.default_rng(407)
    ids = g.integers(-1, E + 1, size=(T, k)).astype(np.int32)
    ids[::3] = np.arange(k) % E                     # every third token hits every expert
    x = g.standard_normal((T, H)).astype(np.float32)
    m_cap = routing.capacity(T, k, E)
    got, wide = _run(x, ids, E, m_cap, False)
    rt = _check_layout(got, ids, E, m_cap)
    off = got["expert_offsets"]
    rows = np.unique(np.clip(np.concatenate([off[:-1], off[1:] - 1, off[:-1] + got["expert_counts"],
                                             g.integers(0, int(off[-1]) + 256, 1500)]),
                             0, m_cap - 1))
    _check_rows(got, wide, rt, rows)


@pytest.mark.parametrize("bf16", [False, True])
def test_full_size_zipf(dev, bf16):
    """8192 tokens x 7168 hidden, top-8 of 32 experts with Zipf(1.1)
    popularity: the whole layout bit-exact; quantized rows bit-exact on a
    sample (run starts and ends, padding, random rows) against the oracle,
    and on every row against the plain 1x128 quantizer of the gathered rows."""
    T, H, k, E = 8192, 7168, 8, 32
    ids = inputs.zipf_topk_routing(3, T, E, k)
    x = inputs.rng(3, 0).standard_normal((T, H), dtype=np.float32)
    m_cap = routing.capacity(T, k, E)
    got, wide = _run(x, ids, E, m_cap, bf16)
    rt = _check_layout(got, ids, E, m_cap)
    off = got["expert_offsets"]
    edges = np.concatenate([off[:-1], off[:-1] + got["expert_counts"] - 1,
                            off[:-1] + got["expert_counts"], [m_cap - 1]])
    g = np.random.default_rng(404)
    rows = np.unique(np.clip(np.concatenate([edges, g.integers(0, m_cap, 160)]), 0, m_cap - 1))
    _check_rows(got, wide, rt, rows)
    # every row: the fused kernel equals the 1x128 quantizer run on the rows
    # gathered by the layout's row map
    gathered = torch.zeros((m_cap, H), dtype=torch.bfloat16 if bf16 else torch.float32,
                           device="cuda")
    src, _ = _source(x, bf16)
    live = torch.from_numpy(rt).cuda().long()
    keep = live >= 0
    gathered[keep] = src[live[keep]]
    q2, s2 = fg8.fp8_quantize(gathered, "1x128")
    torch.cuda.synchronize()
    assert np.array_equal(got["q"], q2.cpu().numpy())
    assert np.array_equal(got["sa"].view(np.uint32), s2.cpu().numpy().view(np.uint32))


def test_layout_feeds_the_contiguous_gemm(dev):
    """Routing kernel -> grouped_gemm_fp8_contiguous on the device, against
    the oracle's layout, quantizer and contiguous GEMM."""
    T, H, N, E, k = 700, 512, 384, 6, 2
    ids = inputs.zipf_topk_routing(31, T, E, k)
    x = inputs.rng(31, 0).standard_normal((T, H), dtype=np.float32)
    w = (inputs.rng(31, 1).standard_normal((E, N, H), dtype=np.float32) * H ** -0.5)
    qb, sb = scaling.quantize_128x128(w)
    tx, _ = _source(x, False)
    tids = torch.from_numpy(ids).cuda()
    lay = fg8.moe_contiguous_layout_fp8(tx, tids, E)
    d = fg8.grouped_gemm_fp8_contiguous(lay["q"], lay["sa"], torch.from_numpy(qb).cuda(),
                                        torch.from_numpy(sb).cuda(), lay["block_expert"])
    torch.cuda.synchronize()
    m_cap = routing.capacity(T, k, E)
    rt, be, _, _ = routing.contiguous_layout(ids, E, m_cap)
    qa, sa = routing.gather_quantize(x, rt)
    live = np.repeat(be >= 0, 128)
    C, S = gemm.grouped_contiguous(qa[live], sa[:, live], qb, sb, be[be >= 0])
    F = TruncRows(C.shape)
    for e in range(E):
        r = np.repeat(be[be >= 0] == e, 128)
        if r.any():
            F[r] = ref_blockscaled(qa[live][r], sa[:, live][:, r], qb[e], sb[e])[2]
    bits = d.view(torch.int16).cpu().numpy().view(np.uint16)[live]
    check_bf16(bits, C, S, H, "routing -> contiguous GEMM", S_flush=F)
