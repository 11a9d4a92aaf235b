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

Timing: W warmup steps and exactly K timed steps, each run as one captured
HIP graph that walks the rotation copies in order (so the figure does not
depend on K against the number of copies); the timed graph is replayed once
untimed first so that its upload is not timed.  The reported time per step
is the GPU time of the K steps, between HIP events recorded on the stream
around a replay of the K-step graph with a synchronization on both sides;
the host wall time around a replay is reported beside it (it adds the
latency of launching the graph, ~30 us, which weighs on short runs).  The JSON line also carries
the cold first step, the p50 / p95 of single steps, the roofline of every
kernel of the step (the dominant one under "roofline") timed per launch with
HIP events on the stream it runs on, the GPU, its observed shader clock and
the ROCm version, the CPU oracle timed on a bounded sample of the same step,
and per-workload figures under "extra" (prefill GEMMs, MoE contiguous,
masked and MXFP8 layouts, the routing step, the gated W1 epilogue, an
end-to-end MoE layer chain, the backward pieces and the quantize kernels).
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(1, os.path.join(ROOT, "tests"))     # the seeded input generators

PEAK_FP8_TFLOPS = 5033.0          # 256 CU x 8192 FLOP/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
ROTATE_BYTES = 576 << 20          # 2 x (256 MB MALL + 8 x 4 MB L2)
METRIC = "FP8 TFLOPS & % of FP8 MFMA peak: dense 64×2112×7168 and MoE grouped GEMM"
CSRC = os.path.join(ROOT, "moe_grouped_gemm_fp8_amd", "csrc")

# rocprofv3 FETCH_SIZE / WRITE_SIZE summaries of the step's GEMMs; each
# records the sha256 of the kernel source it was taken on
TRAFFIC_FILES = {
    "gemm 64x2112x7168": os.path.join(ROOT, "profiles", "gemm_skinny_64x2112x7168_traffic.md"),
    "gemm 64x24576x1536": os.path.join(ROOT, "profiles", "gemm_skinny_64x24576x1536_traffic.md"),
}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="", help="comma list of extra names to run (profiling)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the shader-clock sample (for runs under a profiler)")
    return ap.parse_args(argv)


def log(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def gemm_bytes(M, N, K, out_bytes=2):
    kb = K // 128
    return M * K + N * K + 4 * kb * M + 4 * (-(-N // 128)) * kb + out_bytes * M * N


def quant_bytes(rows, cols):
    """1x128 quantize of FP32 rows: 4 B read, 1 B code and 4/128 B scale written."""
    return rows * cols * 5 + 4 * rows * (cols // 128)


def measured_traffic(path):
    """HBM bytes per launch from a committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, scaled by the copy-kernel calibration recorded there; None when
    the summary is missing or was taken on a different kernel source than the
    one built here."""
    import hashlib
    try:
        text = open(path).read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if ":" in line)
    src = os.path.join(CSRC, fields.get("source_file", "gemm.hip").strip())
    try:
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    if fields.get("source_sha256", "").strip() != digest:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"].strip())
    except (KeyError, ValueError):
        return None


def rotations(nbytes):
    return max(1, -(-ROTATE_BYTES // max(1, nbytes)))


def percentile(sorted_vals, q):
    return sorted_vals[min(len(sorted_vals) - 1, int(round(q * (len(sorted_vals) - 1))))]


def environment(torch):
    """GPU, ROCm and host facts for the JSON line."""
    p = torch.cuda.get_device_properties(0)
    env = {"gpu": torch.cuda.get_device_name(0), "arch": getattr(p, "gcnArchName", ""),
           "cus": p.multi_processor_count, "torch": torch.__version__,
           "hip": getattr(torch.version, "hip", None)}
    try:
        env["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        env["rocm"] = None
    try:
        model = [ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo")
                 if ln.startswith("model name")]
        env["host_cpu"] = model[0] if model else None
    except OSError:
        env["host_cpu"] = None
    return env


def read_sclk_mhz():
    """Current shader clock of GPU 0 from rocm-smi (None if unavailable)."""
    try:
        r = subprocess.run(["rocm-smi", "-d", "0", "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=20)
        data = json.loads(r.stdout)
    except Exception:
        return None
    for card in data.values():
        if not isinstance(card, dict):
            continue
        for key, val in card.items():
            if "sclk" in key.lower():
                digits = "".join(ch for ch in str(val) if ch.isdigit() or ch == ".")
                try:
                    return float(digits)
                except ValueError:
                    return None
    return None


class Timer:
    """Graph capture and timing on one stream."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def capture(self, fns):
        """One graph that runs the callables in order (after an eager pass)."""
        torch = self.torch
        with torch.cuda.stream(self.stream):
            for f in fns:        # eager pass first: allocations, workspaces
                f()
        self.stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            for f in fns:
                f()
        torch.cuda.synchronize()
        return g

    def steps(self, step_fns, steps, warmup):
        """Time per step of exactly `steps` steps after `warmup` steps; step i
        runs step_fns[i % len(step_fns)].  Each phase is one graph.  Returns
        (wall, gpu, graph): wall is the host clock between two
        synchronizations around one replay of the timed graph; gpu is the
        time between HIP events recorded on the stream right before and
        after another replay (the steps' own duration, without the host's
        latency to launch the graph)."""
        torch = self.torch
        R = len(step_fns)
        timed = self.capture([step_fns[(warmup + i) % R] for i in range(steps)])
        warm = self.capture([step_fns[i % R] for i in range(warmup)]) if warmup else None
        timed.replay()                        # upload, untimed
        if warm is not None:
            warm.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        timed.replay()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            e0.record(self.stream)
            timed.replay()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return wall, e0.elapsed_time(e1) * 1e-3 / steps, timed

    def per_launch(self, fns, n):
        """Average duration of one launch in steady state: HIP events on the
        launch stream around replays of a graph that runs every callable
        back to back, divided by the launches it holds."""
        torch = self.torch
        g = self.capture(fns)
        reps = max(1, -(-n // len(fns)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            g.replay()
            e0.record(self.stream)
            for _ in range(reps):
                g.replay()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * len(fns))

    def singles(self, fns, n):
        """Durations (ms) of n single launches, each its own graph bracketed
        by HIP events; sorted."""
        torch = self.torch
        gs = [self.capture([f]) for f in fns]
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        with torch.cuda.stream(self.stream):
            for g in gs:
                g.replay()
            for i, (e0, e1) in enumerate(evs):
                e0.record(self.stream)
                gs[i % len(gs)].replay()
                e1.record(self.stream)
        torch.cuda.synchronize()
        return sorted(e0.elapsed_time(e1) for e0, e1 in evs)


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the kernels "
              "run on one GPU's share of the work, and sharding N (dense) or the experts "
              "(grouped) across GPUs is not part of this library", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import inputs
    import moe_grouped_gemm_fp8_amd as fg8

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    fg8._lib.lib()        # fail loudly if the HIP library is missing
    stream = torch.cuda.Stream()
    timer = Timer(torch, stream)
    env = environment(torch)

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

    def quant_fn(cp, r):
        x = cp[r % len(cp)]
        return lambda: fg8.fp8_quantize(x["A"], "1x128", q=x["qa"], scales=x["sa"])

    def gemm_fn(cp, r):
        x = cp[r % len(cp)]
        return lambda: fg8.gemm_fp8_blockscaled(x["qa"], x["sa"], x["qb"], x["sb"], out=x["d"])

    def step_fn(r):
        parts = [f(cp, r) for _, cp in sets for f in (quant_fn, gemm_fn)]

        def f():
            for p in parts:
                p()
        return f

    step_fns = [step_fn(r) for r in range(R)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        step_fns[0]()
    torch.cuda.synchronize()
    cold_us = (time.perf_counter() - t0) * 1e6

    t_wall, t_step, timed_graph = timer.steps(step_fns, args.steps, args.warmup)
    value = flops_step / t_step / 1e12
    log(f"headline step {t_step * 1e6:.2f} us (events), {t_wall * 1e6:.2f} us wall, "
        f"{value:.1f} TFLOP/s ({R} rotation copies, cold first step {cold_us:.0f} us)")
    single = timer.singles(step_fns, 200)
    # the shader clock while the timed graph runs (enqueued for about 1.5 s)
    sclk = None
    if not args.no_clock:
        with torch.cuda.stream(stream):
            for _ in range(max(1, min(4000, int(1.5 / (t_step * args.steps))))):
                timed_graph.replay()
        sclk = read_sclk_mhz()
        torch.cuda.synchronize()
    env["sclk_mhz_under_load"] = sclk
    del timed_graph

    # every kernel of the step on its own: per-launch events over back-to-back
    # launches of all rotation copies
    kernels = []
    for c, cp in sets:
        for kind, mk in (("quantize 1x128", quant_fn), ("gemm", gemm_fn)):
            name = f"{kind} {c.M}x{c.K}" if kind != "gemm" else f"gemm {c.M}x{c.N}x{c.K}"
            fns = [mk(cp, r) for r in range(len(cp))]
            avg_ms = timer.per_launch(fns, 400)
            sl = timer.singles(fns, 100)
            if kind == "gemm":
                algo = gemm_bytes(c.M, c.N, c.K)
                t = fg8.tile_choice(0, c.M, c.N, c.K)
                desc = (f"fg8 GEMM, {t['bm']}x{t['bn']} tiles, {t['splits']}-way split-K, "
                        f"{t['grid']} workgroups, BF16 out")
            else:
                algo = quant_bytes(c.M, c.K)
                desc = "fg8 1x128 quantize, FP32 in"
            achieved = algo / (avg_ms * 1e-3) / 1e9
            k = {"name": name, "bound": "hbm", "achieved": round(achieved, 1),
                 "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                 "traffic": measured_traffic(TRAFFIC_FILES[name]) if name in TRAFFIC_FILES
                 else None,
                 "kernel": desc, "algorithmic_bytes": algo, "avg_us": round(avg_ms * 1e3, 3),
                 "single_launch_us": {"median": round(percentile(sl, 0.5) * 1e3, 3),
                                      "p95": round(percentile(sl, 0.95) * 1e3, 3)}}
            if kind == "gemm":
                k["tflops"] = round(2 * c.M * c.N * c.K / (avg_ms * 1e-3) / 1e12, 1)
            kernels.append(k)
            log(f"{name}: {k['avg_us']} us, {k['achieved']} GB/s ({k['frac']:.3f} of HBM)")
    dominant = max(kernels, key=lambda k: k["avg_us"])
    roofline = {key: dominant[key] for key in ("bound", "achieved", "peak", "unit", "frac",
                                               "traffic")}
    roofline.update({"kernel": f"{dominant['name']}: {dominant['kernel']}",
                     "algorithmic_bytes": dominant["algorithmic_bytes"],
                     "avg_us": dominant["avg_us"],
                     "timing": "HIP events around back-to-back graph launches on the kernel's "
                               "stream", "all_kernels": kernels})

    extra = {}
    if not args.no_extra:
        extra = run_extras(fg8, inputs, torch, np, dev, timer, args)

    cpu = None if args.no_cpu else cpu_baseline(np, inputs, [c for c, _ in sets])
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
        "step_timing": {"events_us": round(t_step * 1e6, 3), "wall_us": round(t_wall * 1e6, 3),
                        "cold_first_step_us": round(cold_us, 1),
                        "single_step_us": {"p50": round(percentile(single, 0.5) * 1e3, 3),
                                           "p95": round(percentile(single, 0.95) * 1e3, 3)}},
        "env": env,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


def run_extras(fg8, inputs, torch, np, dev, timer, args):
    only = set(filter(None, args.only.split(",")))
    out = {}
    gen = torch.Generator(device=dev)

    def randn(shape, std=1.0, seed=0, dtype=torch.float32):
        gen.manual_seed(seed)
        t = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t if dtype == torch.float32 else t.to(dtype)

    def record(name, fns, flops=None, nbytes=None, steps=None):
        n = steps or 100
        _, t, g = timer.steps(fns, n, max(5, n // 10))
        del g
        sl = timer.singles(fns, min(100, max(20, n)))
        r = {"ms": round(t * 1e3, 4), "ms_single_p50": round(percentile(sl, 0.5), 4),
             "ms_single_p95": round(percentile(sl, 0.95), 4)}
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

    cc = inputs.ContiguousCase()
    moe_names = ("contiguous", "quantize", "chain", "mxcontig", "route", "wgrad")
    if any(want(n) for n in moe_names):
        ids = torch.from_numpy(inputs.zipf_topk_routing(cc.workload, cc.tokens, cc.experts,
                                                        cc.topk)).to(dev)

    def layout(x):
        """The routing step's contiguous layout (on the GPU) of token rows x."""
        lay = fg8.moe_contiguous_layout_fp8(x, ids, cc.experts)
        rt = lay["row_token"].long()
        return lay, rt, rt >= 0, int(lay["expert_counts"].sum().item())

    # MoE contiguous W1 / W2 (8192 tokens, top-8 of 32 experts, Zipf 1.1) in
    # the layout the routing step builds (m_cap rows; the blocks past the last
    # expert's run are skipped by the GEMM)
    if want("contiguous") or want("quantize"):
        x = randn((cc.tokens, cc.hidden), seed=21)
        lay, rt, live, valid = layout(x)
        m_cap = rt.shape[0]
        qa1, sa1, be = lay["q"], lay["sa"], lay["block_expert"]
        if want("quantize"):
            a1 = torch.zeros((m_cap, cc.hidden), dtype=torch.float32, device=dev)
            a1[live] = x[rt[live]]
            R = rotations(a1.numel() * 5)
            cp = [torch.empty_like(a1, dtype=torch.uint8) for _ in range(R)]
            sc = [torch.empty((cc.hidden // 128, m_cap), dtype=torch.float32, device=dev)
                  for _ in range(R)]
            fns = [(lambda i=i: fg8.fp8_quantize(a1, "1x128", q=cp[i], scales=sc[i]))
                   for i in range(R)]
            record(f"quantize 1x128 {m_cap}x{cc.hidden}", fns,
                   nbytes=quant_bytes(m_cap, cc.hidden))
            del cp, sc, a1
            w1 = randn((cc.experts, cc.inter, cc.hidden), cc.hidden ** -0.5, seed=22)
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
            del q, s, qx, ex, w1
        del x
        if want("contiguous"):
            qw1, sw1 = fg8.fp8_quantize(
                randn((cc.experts, cc.inter, cc.hidden), cc.hidden ** -0.5, seed=22), "128x128")
            d1 = torch.empty((m_cap, cc.inter), dtype=torch.bfloat16, device=dev)
            fl = 2 * valid * cc.inter * cc.hidden
            nb = (valid * cc.hidden + qw1.numel() + 4 * valid * cc.hidden // 128 + 4 * sw1.numel()
                  + 2 * valid * cc.inter)
            record(f"moe contiguous W1 {m_cap}(valid {valid})x{cc.inter}x{cc.hidden}",
                   [lambda: fg8.grouped_gemm_fp8_contiguous(qa1, sa1, qw1, sw1, be, out=d1)],
                   fl, nb, steps=20)
            # the same W1 GEMM with the SiLU-gated activation and the 1x128
            # quantization of W2's input fused into the epilogue (the weight
            # rows read as interleaved gate / up blocks)
            qh = torch.empty((m_cap, cc.inter // 2), dtype=torch.uint8, device=dev)
            sh = torch.empty((cc.inter // 256, m_cap), dtype=torch.float32, device=dev)
            nb = (valid * cc.hidden + qw1.numel() + 4 * valid * cc.hidden // 128 + 4 * sw1.numel()
                  + valid * cc.inter // 2 + 4 * valid * cc.inter // 256)
            record(f"moe contiguous W1 + SiLU-gated activation + 1x128 quantize "
                   f"{m_cap}(valid {valid})x{cc.inter}x{cc.hidden}",
                   [lambda: fg8.grouped_gemm_fp8_contiguous_swiglu(qa1, sa1, qw1, sw1, be,
                                                                    q_out=qh, s_out=sh)],
                   fl, nb, steps=20)
            del qw1, sw1, d1, qh, sh
            a2 = randn((m_cap, cc.inter2), seed=23)
            a2[~live] = 0
            qa2, sa2 = fg8.fp8_quantize(a2, "1x128")
            del a2
            qw2, sw2 = fg8.fp8_quantize(
                randn((cc.experts, cc.hidden, cc.inter2), cc.inter2 ** -0.5, seed=24), "128x128")
            d2 = torch.empty((m_cap, cc.hidden), dtype=torch.bfloat16, device=dev)
            fl = 2 * valid * cc.hidden * cc.inter2
            nb = (valid * cc.inter2 + qw2.numel() + 4 * valid * cc.inter2 // 128 + 4 * sw2.numel()
                  + 2 * valid * cc.hidden)
            record(f"moe contiguous W2 {m_cap}(valid {valid})x{cc.hidden}x{cc.inter2}",
                   [lambda: fg8.grouped_gemm_fp8_contiguous(qa2, sa2, qw2, sw2, be, out=d2)],
                   fl, nb, steps=20)
            del qa2, sa2, qw2, sw2, d2
        del lay, qa1, sa1, be, rt, live

    # One MoE expert layer end to end: routing of the BF16 token rows into
    # the contiguous layout with their 1x128 quantization, W1 with the gated
    # activation and the requantization of h fused, then W2 with BF16 out
    if want("chain"):
        xb = randn((cc.tokens, cc.hidden), seed=21, dtype=torch.bfloat16)
        lay, rt, live, valid = layout(xb)
        m_cap = rt.shape[0]
        qw1, sw1 = fg8.fp8_quantize(
            randn((cc.experts, cc.inter, cc.hidden), cc.hidden ** -0.5, seed=22), "128x128")
        qw2, sw2 = fg8.fp8_quantize(
            randn((cc.experts, cc.hidden, cc.inter2), cc.inter2 ** -0.5, seed=24), "128x128")
        qh = torch.empty((m_cap, cc.inter // 2), dtype=torch.uint8, device=dev)
        sh = torch.empty((cc.inter // 256, m_cap), dtype=torch.float32, device=dev)
        y = torch.empty((m_cap, cc.hidden), dtype=torch.bfloat16, device=dev)

        def chain():
            fg8.moe_contiguous_layout_fp8(xb, ids, cc.experts, out=lay)
            fg8.grouped_gemm_fp8_contiguous_swiglu(lay["q"], lay["sa"], qw1, sw1,
                                                   lay["block_expert"], q_out=qh, s_out=sh)
            fg8.grouped_gemm_fp8_contiguous(qh, sh, qw2, sw2, lay["block_expert"], out=y)
        fl = 2 * valid * cc.inter * cc.hidden + 2 * valid * cc.hidden * cc.inter2
        record(f"moe layer chain: routing + quantize (bf16 {cc.tokens}x{cc.hidden}, top{cc.topk} "
               f"of {cc.experts}) -> W1 + gated activation + requantize -> W2 (bf16 out)",
               [chain], fl, steps=10)
        del xb, lay, qw1, sw1, qw2, sw2, qh, sh, y

    # MoE contiguous W1 with MXFP8 operands from BF16 sources (the training
    # pipeline: BF16 -> MXFP8 quantize -> grouped GEMM -> BF16)
    if want("mxcontig"):
        xb = randn((cc.tokens, cc.hidden), seed=21, dtype=torch.bfloat16)
        lay, rt, live, valid = layout(xb)
        m_cap = rt.shape[0]
        a1 = torch.zeros((m_cap, cc.hidden), dtype=torch.bfloat16, device=dev)
        a1[live] = xb[rt[live]]
        be = lay["block_expert"]
        del xb, lay
        qa = torch.empty_like(a1, dtype=torch.uint8)
        ea = torch.empty((m_cap, cc.hidden // 32), dtype=torch.uint8, device=dev)
        record(f"quantize mx1x32 from bf16 {m_cap}x{cc.hidden}",
               [lambda: fg8.fp8_quantize(a1, "mx", q=qa, scales=ea)],
               nbytes=a1.numel() * 3 + a1.numel() // 32)
        del a1
        qw, ew = fg8.fp8_quantize(randn((cc.experts, cc.inter, cc.hidden), cc.hidden ** -0.5,
                                        seed=22, dtype=torch.bfloat16), "mx")
        d1 = torch.empty((m_cap, cc.inter), dtype=torch.bfloat16, device=dev)
        fl = 2 * valid * cc.inter * cc.hidden
        nb = valid * cc.hidden * (1 + 1 / 32) + qw.numel() + ew.numel() + 2 * valid * cc.inter
        record(f"moe contiguous mxfp8 W1 {m_cap}(valid {valid})x{cc.inter}x{cc.hidden}",
               [lambda: fg8.grouped_gemm_mxfp8_contiguous(qa, ea, qw, ew, be, out=d1)], fl, nb,
               steps=20)
        del qa, ea, qw, ew, d1, be

    # MoE routing -> contiguous layout + 1x128 quantize of the BF16 token rows
    # into the rows that hold them (the step before the contiguous W1 GEMM).
    # Bytes: every token row read once, the ids, and the layout's codes,
    # scales, row map and its inverse written once.
    if want("route"):
        xb = randn((cc.tokens, cc.hidden), seed=21, dtype=torch.bfloat16)
        cap = fg8.moe_capacity(cc.tokens, cc.topk, cc.experts)
        lay = fg8.moe_contiguous_layout_fp8(xb, ids, cc.experts)
        valid = int(lay["expert_counts"].sum())
        nb = (2 * xb.numel() + 8 * ids.numel() + cap * cc.hidden + 4 * cap * cc.hidden // 128
              + 4 * cap + 4 * cap // 128 + 8 * cc.experts + 4)
        record(f"moe routing + quantize 1x128 from bf16 into the layout {cc.tokens}x{cc.hidden} "
               f"top{cc.topk} of {cc.experts} (m_cap {cap}, routed {valid})",
               [lambda: fg8.moe_contiguous_layout_fp8(xb, ids, cc.experts, out=lay)], nbytes=nb)
        del xb, lay

    # Training backward of W1: dY and X quantized along the token axis
    # (transposed codes), then the K-grouped weight-gradient GEMM over the
    # routing layout's expert row ranges, FP32 dW [32][4096][7168]
    if want("wgrad"):
        xb = randn((cc.tokens, cc.hidden), seed=21, dtype=torch.bfloat16)
        lay, rt, live, valid = layout(xb)
        offs = lay["expert_offsets"]
        M = int(offs[-1].item())
        rt, live = rt[:M], live[:M]
        X = torch.zeros((M, cc.hidden), dtype=torch.bfloat16, device=dev)
        X[live] = xb[rt[live]]
        dy = randn((M, cc.inter), seed=25, dtype=torch.bfloat16)
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


def cpu_baseline(np, inputs, shapes, budget_s=15.0):
    """The oracle, as it stands, timed on this host on a bounded sample of the
    step: whole steps (quantize A 1x128 + float64 GEMM for both skinny
    shapes; B quantized once outside the timing, as on the GPU) repeated
    until the budget is spent."""
    from oracle import gemm, scaling
    ops = []
    flops = 0
    for c in shapes:
        A, B = inputs.dense_case("skinny_a" if c.N == 2112 else "skinny_b")
        qb, sb = scaling.quantize_128x128(B)
        ops.append((A, qb, sb))
        flops += 2 * c.M * c.N * c.K
    n, t0 = 0, time.perf_counter()
    while True:
        for A, qb, sb in ops:
            qa, sa = scaling.quantize_1x128(A)
            gemm.gemm_blockscaled(qa, sa, qb, sb)
        n += 1
        el = time.perf_counter() - t0
        if el > budget_s or n >= 200:
            break
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = os.cpu_count()
    return {"value": round(flops * n / el / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{n} oracle steps of quantize A 1x128 + float64 GEMM for 64x2112x7168 and "
                      f"64x24576x1536 ({el:.1f} s)"}


if __name__ == "__main__":
    main()
