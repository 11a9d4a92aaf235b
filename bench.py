"""Benchmark of the fine-grained FP8 GEMM hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

One step is one pass of the activation path of the skinny dense workload
(64 x 2112 x 7168 and 64 x 24576 x 1536, A from N(0,1) with log-uniform row
factors in [0.01, 10], B from N(0, 1/K)): quantize A into 1x128 groups, then
the block-scaled GEMM against 128x128-scaled FP8 weights with BF16 output.
Weights are quantized once before timing, as an inference deployment stores
them; that quantization is measured on its own among the extras.  Inputs are
resident in HBM; every step uses a different copy of A, B and D so that the
256 MB last-level cache cannot serve them (rotation past 576 MB).

The JSON line also carries the roofline of the dominant kernel (the
64 x 2112 x 7168 GEMM, HBM-bound) timed per launch with HIP events on the
stream it runs on, the CPU oracle timed on a bounded sample of the same step,
and per-workload figures (prefill GEMMs, MoE contiguous W1/W2, masked, MXFP8
masked, quantize kernels) under "extra".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5033.0          # 256 CU x 8192 FLOP/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
ROTATE_BYTES = 576 << 20          # 2 x (256 MB MALL + 8 x 4 MB L2)
METRIC = "FP8 TFLOPS & % of FP8 MFMA peak: dense 64×2112×7168 and MoE grouped GEMM"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="", help="comma list of extra names to run (profiling)")
    return ap.parse_args()


def log(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def gemm_bytes(M, N, K, out_bytes=2):
    kb = K // 128
    return M * K + N * K + 4 * kb * M + 4 * (-(-N // 128)) * kb + out_bytes * M * N


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_skinny_64x2112x7168_traffic.md")
GEMM_SOURCE = os.path.join(ROOT, "moe_grouped_gemm_fp8_amd", "csrc", "gemm.hip")


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, scaled by the copy-kernel
    calibration recorded there; None when that summary was taken on a
    different gemm.hip than the one built here."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if ":" in line)
    digest = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if fields.get("source_sha256", "").strip() != digest:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"].strip())
    except (KeyError, ValueError):
        return None


def rotations(nbytes):
    return max(1, -(-ROTATE_BYTES // max(1, nbytes)))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the kernels "
              "run on one GPU's share of the work, and sharding N (dense) or the experts "
              "(grouped) across GPUs is not part of this library", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_grouped_gemm_fp8_amd as fg8
    from moe_grouped_gemm_fp8_amd import inputs

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    fg8._lib.lib()        # fail loudly if the HIP library is missing
    stream = torch.cuda.Stream()

    def graphs_for(fns):
        """Capture the callables (one step each, on successive rotation copies)
        as one graph per step plus one graph running all of them in order."""
        with torch.cuda.stream(stream):
            for f in fns:        # eager pass first: allocations, workspaces
                f()
        stream.synchronize()
        singles = []
        for f in fns:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                f()
            singles.append(g)
        whole = torch.cuda.CUDAGraph()
        with torch.cuda.graph(whole, stream=stream):
            for f in fns:
                f()
        torch.cuda.synchronize()
        return singles, whole

    def time_graphs(gs, steps, warmup):
        """Wall time per step of exactly `steps` steps (after `warmup`)."""
        singles, whole = gs
        R = len(singles)

        def run(n):
            for _ in range(n // R):
                whole.replay()
            for j in range(n % R):
                singles[j].replay()

        run(warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(steps)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def time_graph_launches(gs, n):
        """Average duration of one launch in steady state: HIP events on the
        launch stream around replays of the graph that runs every rotation
        copy back to back, divided by the launches it holds."""
        singles, whole = gs
        R = len(singles)
        reps = max(1, -(-n // R))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            whole.replay()
            e0.record(stream)
            for _ in range(reps):
                whole.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * R)

    def time_launches(fns, n):
        """Average duration of single launches, HIP events on the launch stream."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        with torch.cuda.stream(stream):
            for i in range(8):
                fns[i % len(fns)]()
            for i, (e0, e1) in enumerate(evs):
                e0.record(stream)
                fns[i % len(fns)]()
                e1.record(stream)
        torch.cuda.synchronize()
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
        return sum(ms) / len(ms), ms[len(ms) // 2], ms[int(len(ms) * 0.95)]

    # ------------------------------------------------------------ headline step
    shapes = [inputs.DENSE_CASES["skinny_a"], inputs.DENSE_CASES["skinny_b"]]
    sets = []
    for c in shapes:
        A, B = inputs.dense_case("skinny_a" if c.N == 2112 else "skinny_b")
        R = rotations(gemm_bytes(c.M, c.N, c.K) + 4 * c.M * c.K)
        tA = torch.from_numpy(A).to(dev)
        tB = torch.from_numpy(B).to(dev)
        qb, sb = fg8.fp8_quantize(tB, "128x128")
        del tB
        copies = []
        for r in range(R):
            copies.append(dict(
                A=tA.clone(), qb=qb.clone(), sb=sb.clone(),
                qa=torch.empty((c.M, c.K), dtype=torch.uint8, device=dev),
                sa=torch.empty((c.K // 128, c.M), dtype=torch.float32, device=dev),
                d=torch.empty((c.M, c.N), dtype=torch.bfloat16, device=dev)))
        sets.append((c, copies))
    R = max(len(cp) for _, cp in sets)
    flops_step = sum(2 * c.M * c.N * c.K for c, _ in sets)

    def step_fn(r):
        def f():
            for c, cp in sets:
                x = cp[r % len(cp)]
                fg8.fp8_quantize(x["A"], "1x128", q=x["qa"], scales=x["sa"])
                fg8.gemm_fp8_blockscaled(x["qa"], x["sa"], x["qb"], x["sb"], out=x["d"])
        return f

    gs = graphs_for([step_fn(r) for r in range(R)])
    t_step = time_graphs(gs, args.steps, args.warmup)
    value = flops_step / t_step / 1e12
    log(f"headline step {t_step * 1e6:.2f} us, {value:.1f} TFLOP/s ({R} rotation copies)")

    # dominant kernel: the 64 x 2112 x 7168 GEMM, per-launch events
    c0, cp0 = sets[0]

    def gemm_launch(r):
        x = cp0[r % len(cp0)]
        return lambda: fg8.gemm_fp8_blockscaled(x["qa"], x["sa"], x["qb"], x["sb"], out=x["d"])

    fns0 = [gemm_launch(r) for r in range(len(cp0))]
    avg_ms = time_graph_launches(graphs_for(fns0), 400)
    ev_avg, ev_med, ev_p95 = time_launches(fns0, 200)
    algo = gemm_bytes(c0.M, c0.N, c0.K)
    achieved = algo / (avg_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(),
                "kernel": "fg8::gemm_kernel, 64x32 tiles, two workgroups per CU, 2 K blocks "
                          "per stage, 7-way split-K (64x2112x7168, BF16 out)",
                "algorithmic_bytes": algo, "avg_us": round(avg_ms * 1e3, 3),
                "timing": "HIP events around back-to-back graph launches on the kernel's stream",
                "single_launch_us": {"avg": round(ev_avg * 1e3, 3), "median": round(ev_med * 1e3, 3),
                                     "p95": round(ev_p95 * 1e3, 3)},
                "tflops": round(2 * c0.M * c0.N * c0.K / (avg_ms * 1e-3) / 1e12, 1)}

    extra = {}
    if not args.no_extra:
        extra = run_extras(fg8, inputs, torch, np, dev, graphs_for, time_graphs, time_launches,
                           args)

    log(f"dominant kernel avg {avg_ms * 1e3:.2f} us -> {achieved:.0f} GB/s")
    cpu = None if args.no_cpu else cpu_baseline(np, inputs, sets)
    if cpu:
        log(f"cpu baseline {cpu}")

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3", "data": "synthetic",
        "config": {"workload": "dense skinny GEMMs 64x2112x7168 + 64x24576x1536: quantize A "
                               "(1x128) + block-scaled FP8 GEMM (B 128x128), BF16 out",
                   "M": 64, "N": [2112, 24576], "K": [7168, 1536], "rotation_copies": R,
                   "frac_of_fp8_peak": round(value / PEAK_FP8_TFLOPS, 5)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


def run_extras(fg8, inputs, torch, np, dev, graphs_for, time_graphs, time_launches, args):
    only = set(filter(None, args.only.split(",")))
    out = {}
    gen = torch.Generator(device=dev)

    def randn(shape, std=1.0, seed=0):
        gen.manual_seed(seed)
        t = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
        return t.mul_(std) if std != 1.0 else t

    def record(name, fns, flops=None, nbytes=None, steps=None):
        gs = graphs_for(fns)
        n = steps or 100
        t = time_graphs(gs, n, max(5, n // 10))
        avg, med, p95 = time_launches(fns, min(100, max(20, n)))
        r = {"ms_graph": round(t * 1e3, 4), "ms_event_avg": round(avg, 4),
             "ms_event_median": round(med, 4), "ms_event_p95": round(p95, 4)}
        # rates from the steady-state (graph) time per launch
        if flops:
            r["tflops"] = round(flops / t / 1e12, 1)
            r["frac_fp8_peak"] = round(r["tflops"] / PEAK_FP8_TFLOPS, 4)
        if nbytes:
            r["gbs"] = round(nbytes / t / 1e9, 1)
            r["frac_hbm"] = round(r["gbs"] / PEAK_HBM_GBS, 4)
        out[name] = r
        log(f"{name}: {r}")
        torch.cuda.empty_cache()

    def want(name):
        return not only or name in only

    # dense prefill GEMMs
    for nm in ("prefill_a", "prefill_b"):
        if not want(nm):
            continue
        c = inputs.DENSE_CASES[nm]
        qa, sa = fg8.fp8_quantize(randn((c.M, c.K), seed=11), "1x128")
        qb, sb = fg8.fp8_quantize(randn((c.N, c.K), c.K ** -0.5, seed=12), "128x128")
        R = rotations(gemm_bytes(c.M, c.N, c.K))
        cps = [(qa.clone(), sa.clone(), qb.clone(), sb.clone(),
                torch.empty((c.M, c.N), dtype=torch.bfloat16, device=dev)) for _ in range(R)]
        fns = [(lambda x=x: fg8.gemm_fp8_blockscaled(x[0], x[1], x[2], x[3], out=x[4])) for x in cps]
        record(f"{nm} {c.M}x{c.N}x{c.K}", fns, 2 * c.M * c.N * c.K, gemm_bytes(c.M, c.N, c.K))
        del cps, fns

    # MoE contiguous W1 / W2 (8192 tokens, top-8 of 32 experts, Zipf 1.1)
    if want("contiguous") or want("quantize"):
        cc = inputs.ContiguousCase()
        routing = inputs.zipf_topk_routing(cc.workload, cc.tokens, cc.experts, cc.topk)
        lay = inputs.contiguous_layout(routing, cc.experts)
        rt = torch.from_numpy(lay.row_token).to(dev)
        live = rt >= 0
        be = torch.from_numpy(lay.block_expert).to(dev)
        x = randn((cc.tokens, cc.hidden), seed=21)
        a1 = torch.zeros((lay.m_total, cc.hidden), dtype=torch.float32, device=dev)
        a1[live] = x[rt[live]]
        del x
        if want("quantize"):
            R = rotations(a1.numel() * 5)
            cp = [torch.empty_like(a1, dtype=torch.uint8) for _ in range(R)]
            sc = [torch.empty((cc.hidden // 128, lay.m_total), dtype=torch.float32, device=dev)
                  for _ in range(R)]
            fns = [(lambda i=i: fg8.fp8_quantize(a1, "1x128", q=cp[i], scales=sc[i])) for i in range(R)]
            record(f"quantize 1x128 {lay.m_total}x{cc.hidden}", fns,
                   nbytes=a1.numel() * 4 + a1.numel() + 4 * a1.numel() // 128)
            del cp, sc
        qa1, sa1 = fg8.fp8_quantize(a1, "1x128")
        del a1
        w1 = randn((cc.experts, cc.inter, cc.hidden), cc.hidden ** -0.5, seed=22)
        if want("quantize"):
            q = torch.empty_like(w1, dtype=torch.uint8)
            s = torch.empty((cc.experts, cc.inter // 128, cc.hidden // 128), dtype=torch.float32,
                            device=dev)
            record(f"quantize 128x128 {cc.experts}x{cc.inter}x{cc.hidden}",
                   [lambda: fg8.fp8_quantize(w1, "128x128", q=q, scales=s)],
                   nbytes=w1.numel() * 5 + 4 * w1.numel() // 16384)
            qx = torch.empty_like(w1, dtype=torch.uint8)
            ex = torch.empty((cc.experts, cc.inter, cc.hidden // 32), dtype=torch.uint8, device=dev)
            record(f"quantize mx1x32 {cc.experts}x{cc.inter}x{cc.hidden}",
                   [lambda: fg8.fp8_quantize(w1, "mx", q=qx, scales=ex)],
                   nbytes=w1.numel() * 5 + w1.numel() // 32)
            del q, s, qx, ex
        if not want("contiguous"):
            del w1, qa1, sa1
        else:
            qw1, sw1 = fg8.fp8_quantize(w1, "128x128")
            del w1
            d1 = torch.empty((lay.m_total, cc.inter), dtype=torch.bfloat16, device=dev)
            fl = 2 * lay.valid_rows * cc.inter * cc.hidden
            nb = (lay.m_total * cc.hidden + qw1.numel() + 4 * sa1.numel() + 4 * sw1.numel()
                  + 2 * d1.numel())
            record(f"moe contiguous W1 {lay.m_total}(valid {lay.valid_rows})x{cc.inter}x{cc.hidden}",
                   [lambda: fg8.grouped_gemm_fp8_contiguous(qa1, sa1, qw1, sw1, be, out=d1)], fl, nb,
                   steps=20)
            # the same W1 GEMM with the SiLU-gated activation and the 1x128
            # quantization of W2's input fused into the epilogue (the weight
            # rows read as interleaved gate / up blocks)
            qh = torch.empty((lay.m_total, cc.inter // 2), dtype=torch.uint8, device=dev)
            sh = torch.empty((cc.inter // 256, lay.m_total), dtype=torch.float32, device=dev)
            nb = (lay.m_total * cc.hidden + qw1.numel() + 4 * sa1.numel() + 4 * sw1.numel()
                  + qh.numel() + 4 * sh.numel())
            record(f"moe contiguous W1 + SiLU-gated activation + 1x128 quantize "
                   f"{lay.m_total}(valid {lay.valid_rows})x{cc.inter}x{cc.hidden}",
                   [lambda: fg8.grouped_gemm_fp8_contiguous_swiglu(qa1, sa1, qw1, sw1, be,
                                                                    q_out=qh, s_out=sh)],
                   fl, nb, steps=20)
            del qa1, sa1, qw1, sw1, d1, qh, sh
            a2 = randn((lay.m_total, cc.inter2), seed=23)
            a2[~live] = 0
            qa2, sa2 = fg8.fp8_quantize(a2, "1x128")
            del a2
            w2 = randn((cc.experts, cc.hidden, cc.inter2), cc.inter2 ** -0.5, seed=24)
            qw2, sw2 = fg8.fp8_quantize(w2, "128x128")
            del w2
            d2 = torch.empty((lay.m_total, cc.hidden), dtype=torch.bfloat16, device=dev)
            fl = 2 * lay.valid_rows * cc.hidden * cc.inter2
            nb = (qa2.numel() + qw2.numel() + 4 * sa2.numel() + 4 * sw2.numel() + 2 * d2.numel())
            record(f"moe contiguous W2 {lay.m_total}(valid {lay.valid_rows})x{cc.hidden}x{cc.inter2}",
                   [lambda: fg8.grouped_gemm_fp8_contiguous(qa2, sa2, qw2, sw2, be, out=d2)], fl, nb,
                   steps=20)
            del qa2, sa2, qw2, sw2, d2

    # MoE contiguous W1 with MXFP8 operands from BF16 sources (the training
    # pipeline: BF16 -> MXFP8 quantize -> grouped GEMM -> BF16)
    if want("mxcontig"):
        cc = inputs.ContiguousCase()
        routing = inputs.zipf_topk_routing(cc.workload, cc.tokens, cc.experts, cc.topk)
        lay = inputs.contiguous_layout(routing, cc.experts)
        rt = torch.from_numpy(lay.row_token).to(dev)
        live = rt >= 0
        be = torch.from_numpy(lay.block_expert).to(dev)
        x = randn((cc.tokens, cc.hidden), seed=21).bfloat16()
        a1 = torch.zeros((lay.m_total, cc.hidden), dtype=torch.bfloat16, device=dev)
        a1[live] = x[rt[live]]
        del x
        qa = torch.empty_like(a1, dtype=torch.uint8)
        ea = torch.empty((lay.m_total, cc.hidden // 32), dtype=torch.uint8, device=dev)
        record(f"quantize mx1x32 from bf16 {lay.m_total}x{cc.hidden}",
               [lambda: fg8.fp8_quantize(a1, "mx", q=qa, scales=ea)],
               nbytes=a1.numel() * 3 + a1.numel() // 32)
        del a1
        w1 = randn((cc.experts, cc.inter, cc.hidden), cc.hidden ** -0.5, seed=22).bfloat16()
        qw, ew = fg8.fp8_quantize(w1, "mx")
        del w1
        d1 = torch.empty((lay.m_total, cc.inter), dtype=torch.bfloat16, device=dev)
        fl = 2 * lay.valid_rows * cc.inter * cc.hidden
        nb = qa.numel() + ea.numel() + qw.numel() + ew.numel() + 2 * d1.numel()
        record(f"moe contiguous mxfp8 W1 {lay.m_total}(valid {lay.valid_rows})x{cc.inter}x{cc.hidden}",
               [lambda: fg8.grouped_gemm_mxfp8_contiguous(qa, ea, qw, ew, be, out=d1)], fl, nb,
               steps=20)
        del qa, ea, qw, ew, d1

    # MoE routing -> contiguous layout + 1x128 quantize of the BF16 token rows
    # into the rows that hold them (the step before the contiguous W1 GEMM).
    # Bytes: every token row read once, the ids, and the layout's codes,
    # scales, row map and its inverse written once.
    if want("route"):
        cc = inputs.ContiguousCase()
        ids = torch.from_numpy(inputs.zipf_topk_routing(cc.workload, cc.tokens, cc.experts,
                                                        cc.topk)).to(dev)
        x = randn((cc.tokens, cc.hidden), seed=21).bfloat16()
        cap = fg8.moe_capacity(cc.tokens, cc.topk, cc.experts)
        lay = fg8.moe_contiguous_layout_fp8(x, ids, cc.experts)
        valid = int(lay["expert_counts"].sum())
        nb = (2 * x.numel() + 8 * ids.numel() + cap * cc.hidden + 4 * cap * cc.hidden // 128
              + 4 * cap + 4 * cap // 128 + 8 * cc.experts + 4)
        record(f"moe routing + quantize 1x128 from bf16 into the layout {cc.tokens}x{cc.hidden} "
               f"top{cc.topk} of {cc.experts} (m_cap {cap}, routed {valid})",
               [lambda: fg8.moe_contiguous_layout_fp8(x, ids, cc.experts, out=lay)], nbytes=nb)
        del x, ids, lay

    # Training backward of W1: dY and X quantized along the token axis
    # (transposed codes), then the K-grouped weight-gradient GEMM over the
    # routing layout's expert row ranges, FP32 dW [32][4096][7168]
    if want("wgrad"):
        cc = inputs.ContiguousCase()
        ids = torch.from_numpy(inputs.zipf_topk_routing(cc.workload, cc.tokens, cc.experts,
                                                        cc.topk)).to(dev)
        xb = randn((cc.tokens, cc.hidden), seed=21).bfloat16()
        lay = fg8.moe_contiguous_layout_fp8(xb, ids, cc.experts)
        offs = lay["expert_offsets"]
        M = int(offs[-1].item())
        rt = lay["row_token"][:M].long()
        live = rt >= 0
        X = torch.zeros((M, cc.hidden), dtype=torch.bfloat16, device=dev)
        X[live] = xb[rt[live]]
        dy = randn((M, cc.inter), seed=25).bfloat16()
        dy[~live] = 0
        del xb, lay
        qx = torch.empty((cc.hidden, M), dtype=torch.uint8, device=dev)
        sx = torch.empty((M // 128, cc.hidden), dtype=torch.float32, device=dev)
        record(f"quantize 1x128 along tokens (transposed) from bf16 {M}x{cc.hidden}",
               [lambda: fg8.fp8_quantize(X, "1x128_t", q=qx, scales=sx)],
               nbytes=X.numel() * 3 + 4 * X.numel() // 128)
        qy, sy = fg8.fp8_quantize(dy, "1x128_t")
        del X, dy
        dw = torch.empty((cc.experts, cc.inter, cc.hidden), dtype=torch.float32, device=dev)
        valid = int(live.sum().item())
        fl = 2 * valid * cc.inter * cc.hidden
        nb = qy.numel() + qx.numel() + 4 * (sy.numel() + sx.numel()) + 4 * dw.numel()
        record(f"moe wgrad W1 k-grouped {cc.experts}x{cc.inter}x{cc.hidden} over {M} rows "
               f"(valid {valid}), FP32 out",
               [lambda: fg8.grouped_gemm_fp8_kgrouped(qy, sy, qx, sx, offs, out=dw)], fl, nb,
               steps=20)
        del qx, sx, qy, sy, dw

    # MoE masked, FP32 block scales and MXFP8
    if want("masked"):
        mc = inputs.MaskedCase()
        valid = inputs.masked_case_counts(mc)
        tv = torch.from_numpy(valid).to(dev)
        a = randn((mc.experts, mc.cap, mc.K), seed=31)
        b = randn((mc.experts, mc.N, mc.K), mc.K ** -0.5, seed=32)
        live_e = int((valid > 0).sum())
        fl = 2 * int(valid.sum()) * mc.N * mc.K
        qa, sa = fg8.fp8_quantize(a, "1x128")
        qb, sb = fg8.fp8_quantize(b, "128x128")
        nb = (int(valid.sum()) * mc.K + live_e * mc.N * mc.K + 4 * sa.numel() // mc.experts * live_e
              + 4 * sb.numel() // mc.experts * live_e + 2 * int(valid.sum()) * mc.N)
        R = rotations(nb)
        cps = [(qa.clone(), sa.clone(), qb.clone(), sb.clone(),
                torch.zeros((mc.experts, mc.cap, mc.N), dtype=torch.bfloat16, device=dev))
               for _ in range(R)]
        fns = [(lambda x=x: fg8.grouped_gemm_fp8_masked(x[0], x[1], x[2], x[3], tv, out=x[4]))
               for x in cps]
        record(f"moe masked {mc.experts}x{mc.cap}(valid {int(valid.sum())})x{mc.N}x{mc.K}",
               fns, fl, nb)
        del cps, fns, qa, sa, qb, sb
        qa, ea = fg8.fp8_quantize(a, "mx")
        qb, eb = fg8.fp8_quantize(b, "mx")
        nbx = nb + int(valid.sum()) * mc.K // 32 + live_e * mc.N * mc.K // 32
        cps = [(qa.clone(), ea.clone(), qb.clone(), eb.clone(),
                torch.zeros((mc.experts, mc.cap, mc.N), dtype=torch.bfloat16, device=dev))
               for _ in range(R)]
        fns = [(lambda x=x: fg8.gemm_mxfp8(x[0], x[1], x[2], x[3], tv, out=x[4])) for x in cps]
        record(f"moe masked mxfp8 {mc.experts}x{mc.cap}(valid {int(valid.sum())})x{mc.N}x{mc.K}",
               fns, fl, nbx)
        del cps, fns
    return out


def cpu_baseline(np, inputs, sets):
    """The oracle, as it stands, timed on this host on a bounded sample of the
    step: it quantizes A and runs the float64 GEMM for the 64 x 2112 x 7168
    shape (B quantized once outside the timing, as on the GPU)."""
    from oracle import gemm, scaling
    A, B = inputs.dense_case("skinny_a")
    qb, sb = scaling.quantize_128x128(B)
    flops = 2 * A.shape[0] * B.shape[0] * A.shape[1]
    n, t0 = 0, time.perf_counter()
    while True:
        qa, sa = scaling.quantize_1x128(A)
        gemm.gemm_blockscaled(qa, sa, qb, sb)
        n += 1
        el = time.perf_counter() - t0
        if el > 10.0 or n >= 200:
            break
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = os.cpu_count()
    return {"value": round(flops * n / el / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{n} oracle steps of quantize A 1x128 + float64 GEMM 64x2112x7168 "
                      f"({el:.1f} s)"}


if __name__ == "__main__":
    main()
