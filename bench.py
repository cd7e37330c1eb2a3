#!/usr/bin/env python3
"""Benchmark of the A16W4 MoE layer on one MI355X.

A step is one pass of the whole layer over one batch: softmax top-k routing,
align/sort, grouped gate_up GEMM + SwiGLU, grouped down GEMM and the weighted
combine, with every input already resident in HBM. Steps rotate over
--sets independent weight sets and routings (like consecutive layers of a
model), so weights are streamed from HBM rather than served by the 256 MB
Infinity Cache. Default workload: decode, tokens=1 at the production
expert-parallel shape (H=3584, I=3072, 112 local experts, topk=15) with MXFP4
weights.

Prints one JSON line. `value` is tokens/s of the timed steps: HIP-graph
replays, each graph holding one step of every weight set back to back (as
the MoE layers of a captured model step run); `one_step_per_graph` is the
same with a graph replay per step. `roofline` is the
dominant kernel (the gate_up stage): algorithmic bytes (decode) or flops
(prefill) per launch over its average launch duration, timed with HIP events
on the launch stream around a graph of back-to-back launches cycling over the
weight sets; its `traffic` is the HBM bytes per launch that rocprofv3 counters
measured for the same kernel sources (profiles/traffic.json), else null.
`stage_us` is an eager breakdown into the monolithic call's two stage groups
(routing + align/sort + gate_up; down + combine), with events between the
launches, so it includes launch gaps. `warm` repeats one weight set every
step (the cold headline rotates over --sets). Prefill lines also carry the
shader clock under the MFMA load (from the committed SQ-counter profile) and
the peak at that clock. For the int4 workloads `requant` is the load-time
MXFP4 -> int4-g32 conversion of one weight set (every expert of w13 and w2, 8
experts per call into preallocated outputs): bytes read + written per pass
over its duration, against HBM peak. `cpu_baseline` is the CPU oracle on a
bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s + achieved HBM GB/s (decode) / MFMA % (prefill) at H3584,E112"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_t1",
                    help="decode_t1 (default), decode_t{4,7,16,32}, skewed_t{4,7,16,32}, "
                         "prefill_t1024, int4_t16, tp8_t1 (8-way tensor-parallel shard: E=896, I=384)")
    ap.add_argument("--sets", type=int, default=8, help="independent weight sets / routings")
    ap.add_argument("--eager", action="store_true", help="time eager launches, not graph replay")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


def copy_probe():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}))


class Layer:
    """Device buffers of one weight set + routing, and the launches of a step."""

    def __init__(self, moe, spec, T, fmt, seed, host=None, int4=False):
        import numpy as np
        import torch
        self.moe, self.T, self.fmt = moe, T, fmt
        s = spec
        H, I, E, k = s.H, s.I, s.E, s.topk
        self.H, self.I, self.E, self.k = H, I, E, k
        dev = torch.device("cuda")
        if host is not None:
            self.x = torch.from_numpy(host.x.view(np.int16)).view(torch.bfloat16).to(dev)
            self.logits = torch.from_numpy(host.logits).to(dev)
            w = [torch.from_numpy(a).to(dev) for a in (host.w13, host.w13_scale, host.w2, host.w2_scale)]
        else:
            g = torch.Generator(device=dev)
            g.manual_seed(seed)
            self.x = torch.randn((T, H), generator=g, device=dev).to(torch.bfloat16)
            self.logits = torch.randn((T, E), generator=g, device=dev)
            if s.hot:
                hot = torch.randperm(E, generator=g, device=dev)[: s.hot]
                self.logits[:, hot] += s.hot_bias
            w = [torch.randint(0, 256, (E, 2 * I, H // 2), generator=g, device=dev, dtype=torch.uint8),
                 torch.randint(s.scale_lo, s.scale_hi + 1, (E, 2 * I, H // 32), generator=g, device=dev,
                               dtype=torch.uint8),
                 torch.randint(0, 256, (E, H, I // 2), generator=g, device=dev, dtype=torch.uint8),
                 torch.randint(s.scale_lo, s.scale_hi + 1, (E, H, I // 32), generator=g, device=dev,
                               dtype=torch.uint8)]
        self.mx = w if (int4 and host is not None) else None  # set 0 keeps its MXFP4 tensors
        if int4:
            q13, s13 = moe.requantize_mxfp4_experts(w[0], w[1])
            q2, s2 = moe.requantize_mxfp4_experts(w[2], w[3])
            w = [q13, s13, q2, s2]
            torch.cuda.synchronize()
        self.w13, self.w13s, self.w2, self.w2s = w
        self.bm = moe.moe_default_block_m(T, k, E)
        self.bufs = moe.MonolithicBuffers(T, H, I, E, k, self.bm, dev)
        b = self.bufs
        self.ids, self.wts, self.out, self.ws = b.ids, b.weights, b.out, b.workspace
        self.sort = (b.sorted_ids, b.block_expert, b.expert_offsets, b.num_post_pad)

    def route_sort(self):
        self.moe.moe_route_align(self.logits, self.k, self.E, self.bm, True, self.ids, self.wts,
                                 out=self.sort)

    def forward(self, stages=7):
        s, be, _, npp = self.sort
        self.moe.moe_a16w4_forward(self.x, self.w13, self.w13s, self.w2, self.w2s, self.ids, self.wts,
                                   s, be, npp, self.bm, fmt=self.fmt, out=self.out, workspace=self.ws,
                                   stages=stages)

    def monolithic(self, stages=7):
        self.moe.moe_a16w4_forward_monolithic(self.x, self.logits, self.w13, self.w13s, self.w2, self.w2s,
                                              self.k, fmt=self.fmt, block_m=self.bm, bufs=self.bufs,
                                              stages=stages)

    def step(self):
        """One pass of the layer: routing, align/sort, gate_up + SwiGLU, down,
        combine (moe_a16w4_forward_monolithic)."""
        self.monolithic()

    def distinct_experts(self):
        import torch
        return int(torch.unique(self.ids).numel())


def stage1_launch_us(layers, moe, eager, fused_t1, reps=4):
    """Average duration of one gate_up launch: a HIP graph of launches cycling
    over every weight set (eager launches with --eager), timed with events on
    the stream the launches go to. With the one-token path the launch is the
    gate_up kernel that also routes (the monolithic call's first stage)."""
    import torch
    stream = torch.cuda.current_stream()
    n = len(layers) * reps
    if fused_t1:
        launch = lambda L: L.monolithic(moe.MOE_STAGE_GATE_UP)
    else:
        launch = lambda L: L.forward(moe.MOE_STAGE_GATE_UP)
    if eager:
        fn = lambda: [launch(layers[i % len(layers)]) for i in range(n)]
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                launch(layers[i % len(layers)])
        stream = torch.cuda.current_stream()
        fn = g.replay
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (3 * n)


def counter_clock_ghz(workload):
    """Shader clock under the MFMA load of the dominant prefill kernel, from
    the committed SQ-counter profile (profiles/sclk.json: SQ_BUSY_CYCLES per
    shader engine over the kernel's rocprofv3 duration). None without one."""
    path = os.path.join(ROOT, "profiles", "sclk.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    return rec if rec and rec.get("ghz") else None


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter's
    reading for a plain device copy). None when there is no summary for this
    workload, or the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("kernel") != kernel:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return rec["hbm_bytes_per_launch"]


def fused_t1(T, fmt, H, I, topk, E):
    """Whether the monolithic call takes the two-launch one-token path (the
    rule of t1_eligible in the C sources, restated for the label)."""
    return (T == 1 and fmt == 0 and E <= 128 and topk <= 64 and H % 256 == 0 and I % 128 == 0
            and H <= 4096 and I <= 4096)


def stage1_kernel_name(T, bm, fmt, H, I, topk, E):
    """Which gate_up kernel the library launches for this shape (the rule of
    gemv_resident_eligible / gemv_mfma_eligible / gemv_eligible / forward_stages
    in the C sources, restated for the label)."""
    if fused_t1(T, fmt, H, I, topk, E):
        return "route_gate_up_t1_kernel"
    rows = min(T, bm)
    cap16 = T * topk + min(T * topk, E) * 15  # align/sort capacity at 16-row blocks
    kmax = 4096 if fmt == 0 else 3584
    if (bm == 16 and rows > 1 and H <= kmax and I <= kmax and H % 512 == 0 and I % 512 == 0
            and (cap16 + 15) // 16 <= 512):
        return "gemv_resident_kernel"
    if (bm == 16 and rows > 1 and H <= 4096 and I <= 4096 and H % 64 == 0 and I % 64 == 0):
        return "gemv_mfma_x_kernel" if T > 12 else "stage1_gemv_mfma_kernel"
    if (bm <= 32 and fmt == 0 and rows <= 8 and H <= 4096 and I <= 4096
            and H % 256 == 0 and I % 128 == 0):
        return "stage1_gemv_kernel"
    P = T * topk
    if bm == 32 and H % 256 == 0 and I % 256 == 0 and P >= 32:
        if T <= (13 if fmt == 0 else 32):
            return f"prefill_direct_kernel<1, {fmt}>"
        return f"prefill_kernel<1, {fmt}, 2>" if P <= 48 * min(P, E) else f"prefill_kernel<1, {fmt}, 8>"
    return "stage1_unit_kernel" if bm <= 32 else "stage1_stream_kernel"


def weight_bytes_per_expert(H, I, fmt):
    sb = 1 if fmt == 0 else 2
    w13 = 2 * I * (H // 2) + 2 * I * (H // 32) * sb
    w2 = H * (I // 2) + H * (I // 32) * sb
    return w13, w2


def requant_rate(moe, mx, passes=5):
    """Time the load-time requant of every expert of one weight set (w13 and
    w2, 8 experts per call into preallocated outputs), HIP events on the
    current stream. Free device memory is read before and after the timed
    loop: the calls allocate nothing."""
    import torch
    outs = [(torch.empty_like(w), torch.empty(s.shape, dtype=torch.bfloat16, device=w.device))
            for w, s in ((mx[0], mx[1]), (mx[2], mx[3]))]
    pairs = [((mx[0], mx[1]), outs[0]), ((mx[2], mx[3]), outs[1])]
    nbytes = sum(w.numel() + s.numel() + q.numel() + 2 * sb.numel() for (w, s), (q, sb) in pairs)

    def one_pass():
        calls = 0
        for (w, s), (q, sb) in pairs:
            for lo in range(0, w.shape[0], 8):
                moe.mxfp4_to_int4g32_requant(w, s, lo, min(lo + 8, w.shape[0]), q, sb)
                calls += 1
        return calls
    one_pass()
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(passes):
        calls = one_pass()
    e1.record()
    e1.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    ms = e0.elapsed_time(e1) / passes
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"bytes_per_pass": nbytes, "ms_per_pass": round(ms, 4), "achieved": round(gbps, 1),
            "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "calls_per_pass": calls,
            "experts_per_call": 8, "device_bytes_allocated_during_loop": free0 - free1}


def cpu_baseline(wl, spec, seconds, fmt_name):
    """The CPU oracle (test infrastructure) timed on this host, tokens/s: the
    same bounded sample (routing + align/sort of every token, the forward of
    up to 4 of them) on all host cores and on one core, each the median of 3
    timed runs; a run repeats the sample to about seconds / 6."""
    import numpy as np
    import oracle
    T = wl.x.shape[0]
    n_tok = T if T <= 4 else 2
    tokens = np.arange(n_tok, dtype=np.int32)

    def sample():
        ids, w = oracle.route_topk(wl.logits, spec.topk)
        oracle.align_sort(ids, spec.E, 16)
        oracle.moe_forward(wl.x, wl.w13, wl.w13_scale, wl.w2, wl.w2_scale, oracle.FMT_MXFP4, ids, w,
                           I=spec.I, tokens=tokens if n_tok < T else None)

    def median_rate(threads):
        oracle.set_num_threads(threads)
        t0 = time.perf_counter()
        sample()  # also sizes the runs
        one = time.perf_counter() - t0
        reps = max(1, int(seconds / 6 / max(one, 1e-6)))
        rates = []
        for _ in range(3):
            t0 = time.perf_counter()
            for _ in range(reps):
                sample()
            rates.append(reps * n_tok / (time.perf_counter() - t0))
        return float(np.median(rates)), reps

    all_cores = oracle.num_threads()
    v_all, reps_all = median_rate(all_cores)
    v_one, reps_one = median_rate(1)
    oracle.set_num_threads(all_cores)
    return {"value": round(v_all, 4), "unit": "tokens/s", "cores": all_cores, "kind": "oracle",
            "one_core": {"value": round(v_one, 4), "cores": 1},
            "sample": f"median of 3 runs of {reps_all} (all cores) / {reps_one} (one core) x (route + "
                      f"align/sort of all {T} tokens + forward of {n_tok} token(s)) of the {fmt_name} "
                      f"workload, weight set 0"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the layer here is one "
              "expert-parallel rank's share and this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return

    import numpy as np
    import torch

    import mxfp4_grouped_gemm_amd as moe
    import synth

    specs = synth.specs()
    if args.workload not in specs or args.workload == "tiny":
        raise SystemExit(f"unknown workload {args.workload}")
    spec = specs[args.workload]
    int4 = args.workload.startswith("int4")
    fmt = moe.MOE_W_INT4G32 if int4 else moe.MOE_W_MXFP4
    T = spec.T
    host = synth.make(spec)
    layers = [Layer(moe, spec, T, fmt, seed=1000 + i, host=host if i == 0 else None, int4=int4)
              for i in range(args.sets)]
    torch.cuda.synchronize()
    R = len(layers)

    # routing of each set (for the algorithmic byte counts)
    for L in layers:
        L.route_sort()
    torch.cuda.synchronize()
    distinct = [L.distinct_experts() for L in layers]

    # ---- headline: graph replay (or eager) of whole steps
    graphs = chain = None
    if not args.eager:
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for L in layers:  # warm the launch path once outside capture
                L.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for L in layers:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                L.step()
            graphs.append(g)
        # The R sets' steps back to back in one graph, as the MoE layers of
        # consecutive decoder layers run inside one captured model step: the
        # host-side cost of starting a graph is paid once per R steps.
        chain = torch.cuda.CUDAGraph()
        with torch.cuda.graph(chain):
            for L in layers:
                L.step()
        torch.cuda.synchronize()

    def run_steps(n):
        """n whole steps over the sets in order: full passes as one replay of
        the chained graph, the rest as single-step replays (eager: launches)."""
        if graphs is None:
            for i in range(n):
                layers[i % R].step()
            return
        full, rem = divmod(n, R)
        for _ in range(full):
            chain.replay()
        for i in range(rem):
            graphs[i].replay()

    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(n)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    run_steps(args.warmup)
    torch.cuda.synchronize()
    ms_per_step = timed(run_steps, args.steps)

    # ---- the same steps with one graph replay per step (host-side start of
    # every replay inside the timed region), reported apart
    single_ms = None
    if graphs is not None:
        def run_single(n):
            for i in range(n):
                graphs[i % R].replay()
        run_single(args.warmup)
        torch.cuda.synchronize()
        single_ms = timed(run_single, args.steps)

    # ---- warm cache: one weight set every step (its weights partly served by
    # the Infinity Cache), R steps per graph like the headline, reported apart
    warm_ms = None
    if graphs is not None:
        warm = torch.cuda.CUDAGraph()
        with torch.cuda.graph(warm):
            for _ in range(R):
                layers[0].step()
        torch.cuda.synchronize()

        def run_warm(n):
            full, rem = divmod(n, R)
            for _ in range(full):
                warm.replay()
            for _ in range(rem):
                graphs[0].replay()
        run_warm(args.warmup)
        torch.cuda.synchronize()
        warm_ms = timed(run_warm, args.steps)

    # ---- per-stage timing (eager, events on the launch stream): the two
    # stage groups of the monolithic call
    nst = max(args.steps, 8)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nst)]
    for i in range(min(args.warmup, 4)):
        layers[i % R].step()
    torch.cuda.synchronize()
    for i in range(nst):
        L, e = layers[i % R], ev[i]
        e[0].record()
        L.monolithic(moe.MOE_STAGE_GATE_UP)
        e[1].record()
        L.monolithic(moe.MOE_STAGE_DOWN | moe.MOE_STAGE_COMBINE)
        e[2].record()
    torch.cuda.synchronize()
    stage_ms = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(2)] for e in ev])
    stage_avg = stage_ms.mean(axis=0)
    eager_ms = float(stage_ms.sum(axis=1).mean())

    H, I, E, k = spec.H, spec.I, spec.E, spec.topk
    P = T * k
    w13_b, w2_b = weight_bytes_per_expert(H, I, fmt)
    d_avg = float(np.mean(distinct))
    act_bytes_1 = T * H * 2 + P * I * 2            # x read, h written
    if fused_t1(T, fmt, H, I, k, E):
        act_bytes_1 += T * E * 4                    # the routing reads the logits
    stage1_bytes = d_avg * w13_b + act_bytes_1
    layer_bytes = d_avg * (w13_b + w2_b) + 2 * T * H * 2 + T * E * 4
    stage1_flops = 2.0 * P * (2 * I) * H
    layer_flops = 2.0 * P * 3 * I * H

    # ---- dominant kernel (gate_up): back-to-back launches over all sets,
    # HIP events on the launch stream, average duration per launch
    t1 = fused_t1(T, fmt, H, I, k, E)
    s1_us = stage1_launch_us(layers, moe, args.eager, t1)
    s1_sec = s1_us * 1e-6
    if spec.T >= 256:
        ach = stage1_flops / s1_sec / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None}
        # The published peak is quoted at 2.4 GHz. The shader clock this kernel
        # runs at comes from the committed rocprofv3 SQ counters of the same
        # kernel (busy cycles per shader engine over its duration); with it,
        # the peak at that clock.
        clk = counter_clock_ghz(args.workload)
        if clk:
            at_clock = BF16_MFMA_PEAK_TFLOPS * clk["ghz"] / 2.4
            roof["sclk_ghz_from_counters"] = clk["ghz"]
            roof["sclk_source"] = clk["source"]
            roof["peak_at_observed_clock"] = round(at_clock, 1)
            roof["frac_at_observed_clock"] = round(ach / at_clock, 4)
    else:
        ach = stage1_bytes / s1_sec / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": None}
    kname = stage1_kernel_name(T, layers[0].bm, fmt, H, I, k, E)
    roof["traffic"] = measured_traffic(args.workload, kname)
    roof["kernel"] = kname + " (grouped gate_up GEMM + SwiGLU)"
    roof["avg_us"] = round(s1_us, 2)
    roof["algorithmic_per_launch"] = (round(stage1_flops) if roof["bound"] == "mfma"
                                      else round(stage1_bytes))

    value = T / (ms_per_step * 1e-3)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "H": H, "I": I, "experts": E, "topk": k,
                   "weights": "int4_g32" if int4 else "mxfp4", "block_m": layers[0].bm,
                   "weight_sets": R,
                   "timing": "eager" if args.eager else f"hip_graph_replay ({R} steps per graph)",
                   "distinct_experts_avg": round(d_avg, 2)},
        "layer_hbm_gbps": round(layer_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "layer_tflops": round(layer_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "eager_ms_per_step": round(eager_ms, 5),
        "stage_us": {"route_sort_gate_up": round(stage_avg[0] * 1e3, 2),
                     "down_combine": round(stage_avg[1] * 1e3, 2)},
        "roofline": roof,
    }
    if single_ms is not None:
        line["one_step_per_graph"] = {"ms_per_step": round(single_ms, 5),
                                      "value": round(T / (single_ms * 1e-3), 2), "unit": "tokens/s",
                                      "note": "a graph replay per step (graph start in every step)"}
    if warm_ms is not None:
        line["warm"] = {"ms_per_step": round(warm_ms, 5), "value": round(T / (warm_ms * 1e-3), 2),
                        "unit": "tokens/s", "note": "one weight set replayed every step (Infinity Cache warm)"}
    if int4:
        line["requant"] = requant_rate(moe, layers[0].mx)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(host, spec, args.cpu_seconds,
                                            "int4_g32" if int4 else "MXFP4")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
