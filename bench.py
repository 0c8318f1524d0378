#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X: route -> dispatch layout + permute -> grouped SwiGLU expert
GEMM (+ shared experts) -> combine, through libmoe.so, on seeded synthetic inputs.

    python bench.py [--steps K] [--warmup W] [--workload 4] [--no-cpu-baseline]

Prints one JSON line. A step is one pass of the whole hot path over one batch whose inputs are
already resident in HBM. `value` is tokens per second (owned tokens / step time) over K steps on
one stream, the shared experts in the same launches as the routed ones (--overlap: the shared
experts, which need no routing, on a second stream while route and dispatch run). The per-phase
times and the roofline come from K more single-stream steps with HIP events between the
phases; the roofline object covers the dominant kernel, the gate/up grouped GEMM. cpu_baseline
times the plain CPU oracle on a bounded sample of the same workload. The default workload is the largest single-GPU
configuration, the Llama-4-Scout-shaped layer (N 8192, H 5120, 16 experts top-1 sigmoid, I 8192,
one shared expert, bf16). The `shuffle` object (outside the step; --shuffle adds it) times the
token-shuffle planner's table fit and plan on a stand-in routing trace and reports the locality
of the planned owners against contiguous sequence slices. --microbatches M also times the step
pipelined over M microbatches (the `microbatch` object).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s on 1 GPU; GEMM MFMA % of peak; permute/combine HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=100,
                   help="untimed steps first: the first few dozen steps after start-up run "
                        "up to 10%% slower than the steady state")
    p.add_argument("--workload", type=int, default=4,
                   help="1..5 (default 4: the Llama-4-Scout-shaped layer, the largest)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=0,
                   help="tokens in the oracle's timed sample (0 = automatic)")
    p.add_argument("--out", default="", help="also append the JSON line to this file")
    p.add_argument("--placement", choices=["contiguous", "correlated"], default="contiguous",
                   help="expert placement: contiguous, or the balanced partition of the "
                        "co-selection counts of this batch's routing (set-up, not timed)")
    p.add_argument("--graph", action="store_true",
                   help="time the step as replays of one HIP graph (the per-kernel times still "
                        "come from the eager steps)")
    p.add_argument("--route-from", choices=["x", "logits"], default=None,
                   help="default: logits for the correlated-routing workload (its co-selected "
                        "pairs are planted in the logits, which a router product of random x "
                        "and W_R would not reproduce), x otherwise. "
                        "x: the step starts from the token rows, with the router linear layer "
                        "on the device (its epilogue routes and counts where one workgroup "
                        "holds all of a token's logits); logits: the step starts from "
                        "precomputed router logits")
    p.add_argument("--overlap", action="store_true",
                   help="run the shared experts on a second stream during route and dispatch "
                        "(their own launches) instead of in the same launches as the routed ones")
    p.add_argument("--microbatches", type=int, default=1,
                   help="also time the step pipelined over this many microbatches (the "
                        "`microbatch` object; dst_rank = -1 workloads)")
    p.add_argument("--no-flush", action="store_true",
                   help="do not read a 1 GiB buffer (evicting L2 and the 256 MB MALL) before each "
                        "phase-timed step")
    p.add_argument("--plain-weights", action="store_true",
                   help="keep the expert weights in the plain K-contiguous layout instead of the "
                        "packed layout (moe_pack_weights, converted once at set-up)")
    p.add_argument("--shuffle", action="store_true",
                   help="also time the token-shuffle planner (not part of the step)")
    p.add_argument("--table1", action="store_true",
                   help="also report the Expert Coupling Table I statistics (dedup %%, GPUs per "
                        "token, same-GPU %%) on synthetic correlated routing (not part of the "
                        "step)")
    p.add_argument("--small-batch", action="store_true",
                   help="also time small batches (the tiny layer at 64 tokens, the "
                        "DeepSeek-V2-Lite-shaped layer at 64, 256 and 512 tokens) as the separate "
                        "launches (eager and as one HIP graph) and as the one-launch fused layer "
                        "(eager and as a graph); the `small_batch` object (not part of the step)")
    p.add_argument("--dense-reference", action="store_true",
                   help="also time the workload's shared-expert gate/up product as one dense "
                        "GEMM through this library and through torch.mm (the vendor library), "
                        "same shape and dtype (the `dense_reference` object, not part of the "
                        "step)")
    p.add_argument("--gemm-cus", type=int, default=0,
                   help="cap the grouped GEMM's persistent grid at this many compute units "
                        "(moe_set_gemm_max_cus; 0 = all): with fewer units busy the chip's power "
                        "limit allows a higher shader clock")
    p.add_argument("--copy-calibration-mb", type=int, default=0,
                   help="before warm-up, one device-to-device copy of this many MiB (a kernel of "
                        "known traffic to scale rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    a = p.parse_args()
    return a


def default_route_from(w):
    """Where the step's routing starts: the logits for a workload whose co-selection structure is
    planted in its logits (a router product of random x and W_R would not carry it), x (the
    router linear layer on the device) for the others."""
    return "logits" if w.hot_pairs else "x"


def measured_traffic(w, kernel_prefix):
    """HBM bytes per launch of the dominant kernel from the committed counter summary of this
    workload (its `traffic-record:` line), or None when there is none or the kernel's source
    code changed since the counters were taken."""
    import json as _json
    from dispatch_expert_gemm_amd.rocprof_summary import code_hash
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_ffn_gemm1_{w.name}.md")
    try:
        line = [x for x in open(path) if x.startswith("traffic-record:")][-1]
        rec = _json.loads(line.split(":", 1)[1])
        src = os.path.join(ROOT, "dispatch_expert_gemm_amd", "csrc", rec["source"])
        if code_hash(src) != rec["source_code_sha256"] or rec["kernel_prefix"] != kernel_prefix:
            return None
    except (OSError, IndexError, KeyError, ValueError):
        return None
    return rec["bytes_per_launch"]


def algorithmic(w, rows, pairs):
    """Algorithmic work of one step (what the method must move or compute)."""
    eb = w.elt_bytes
    t0, t1 = w.owned
    owned = t1 - t0
    S = w.n_shared
    d = {}
    d["route_bytes"] = w.N * w.E * 4 + (w.E * 4 if w.bias_std else 0) + w.N * w.k * 8
    out_rows = pairs if w.dedup else rows
    # permute: each token row needed by the partition read once, each dispatched row written once
    uniq = pairs if w.dst_rank >= 0 else w.N
    d["permute_bytes"] = (uniq + out_rows) * w.H * eb
    # combine: every owned slot's row read, shared outputs read, the output written
    slots = owned * w.k
    d["combine_bytes"] = (slots + S * owned + owned) * w.H * eb
    if w.dedup:   # expert-rank partials (read the rows, write one per pair), then owner sums
        src = pairs if w.expert == "identity" else rows
        d["combine_bytes"] = (src + 2 * pairs + S * w.N + w.N) * w.H * eb
    if w.expert == "swiglu":
        mrows = rows + S * w.N
        d["gemm1_flops"] = 2.0 * mrows * w.H * 2 * w.I
        d["gemm2_flops"] = 2.0 * mrows * w.I * w.H
        # every local expert's and shared expert's gate, up and down weights read once
        e_local = w.E // w.W if w.dst_rank >= 0 else w.E
        d["gemm_weight_bytes"] = (e_local + S) * 3 * w.I * w.H * eb
    return d


def cpu_baseline(w, host, n_tokens):
    """The oracle as it stands on the first n_tokens tokens of the workload (its own route,
    layout, expert FFN and combine), timed on the host cores."""
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    n = max(w.W, n_tokens - n_tokens % w.W)
    x = host["x"][:n].float().numpy()
    logits = np.asarray(host["logits"])[:n]
    experts, shared = {}, []
    if w.expert == "swiglu":
        wgu, wd = host["experts"]
        local = range(wgu.shape[0])
        first = 0 if w.dst_rank < 0 else w.dst_rank * (w.E // w.W)
        experts = {first + i: (wgu[i].float().numpy(), wd[i].float().numpy()) for i in local}
        if host.get("shared") and host["shared"][0] is not None:
            sgu, sd = host["shared"]
            shared = [(sgu[s].float().numpy(), sd[s].float().numpy()) for s in range(sgu.shape[0])]
    def one_pass(stages=None):
        clock = [time.perf_counter()]

        def mark(name):
            if stages is not None:
                now = time.perf_counter()
                stages[name] = round(now - clock[0], 4)
                clock[0] = now
        idx, wts = O.route(logits, host["bias"], w.k, w.gate)
        mark("route")
        lay = O.layout(idx, O.contiguous_placement(w.E, w.W), w.W)
        mark("layout")
        y = O.expert_outputs(x, lay, w.k, experts, identity=w.expert == "identity")
        sh = np.stack([O.swiglu_expert(x, *s) for s in shared]) if shared else None
        if w.dst_rank >= 0:
            y = np.nan_to_num(y)            # rows of other ranks' experts are not computed here
        mark("ffn")
        O.combine_a2a(y, lay, wts, shared=sh)
        mark("combine")

    # one pass with each stage timed on its own
    stages = {}
    one_pass(stages)

    # the sample is passed through the oracle repeatedly until about 10 s of CPU time (at most
    # 20 passes), so that the rate is not one short measurement
    passes, t0 = 0, time.perf_counter()
    while True:
        one_pass()
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or passes >= 20:
            break
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    return dict(value=n * passes / dt, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"first {n} of {w.N} tokens of {w.name}, {passes} passes: oracle route, "
                       f"layout, expert FFN (fp64) and combine; {dt:.1f} s",
                stages_s=stages,
                cpu_count=os.cpu_count(), affinity=affinity, blas_threads=int(threads))


def device_info() -> dict:
    """What the HIP runtime reports for the current device."""
    import torch

    from dispatch_expert_gemm_amd import moe
    cus, lds, clk, mclk = moe.moe_device_info()
    props = torch.cuda.get_device_properties(0)
    return dict(name=props.name, arch=getattr(props, "gcnArchName", ""), cus=cus,
                lds_kb_per_cu=lds // 1024, peak_clock_mhz=clk // 1000,
                mem_clock_mhz=mclk // 1000, hbm_gb=round(props.total_memory / 2 ** 30, 1))


def shuffle_planner(name: str) -> dict:
    """Token-shuffle planner on a stand-in routing trace (not part of the layer step): the tables
    fit on the trace's fit tokens under correlated placement (co-selection counts and
    Algorithm 1 through the library), then the plan of its T tokens; times from HIP events on
    the library's stream, and the locality of the position-m slots before and after."""
    import numpy as np
    import torch

    from dispatch_expert_gemm_amd import moe
    from dispatch_expert_gemm_amd import workloads as WL

    c = WL.SHUFFLE_TRACES[name]
    fit = [torch.from_numpy(a).cuda() for a in WL.gen_shuffle_trace(c, "fit")]
    p2, p1, cur = WL.gen_shuffle_trace(c, "eval")
    counts = moe.moe_coselect_counts(fit[2], c.E)
    group, _ = moe.moe_placement_partition(counts.cpu().numpy(), c.P)
    placement = torch.from_numpy(group).cuda()
    ws_fit = torch.empty(moe.lib().moe_shuffle_fit_workspace_bytes(c.E, c.P), dtype=torch.uint8,
                         device="cuda")
    ws_plan = torch.empty(moe.lib().moe_shuffle_plan_workspace_bytes(c.T), dtype=torch.uint8,
                          device="cuda")
    dp2, dp1 = torch.from_numpy(p2).cuda(), torch.from_numpy(p1).cuda()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            out = fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps, out

    fit_ms, (F, S, n) = timed(lambda: moe.moe_shuffle_fit(*fit, placement, c.E, c.P, ws_fit), 5)
    beta, w_max = 8.0, 0.9
    plan_ms, (_, _, owner, _, _) = timed(
        lambda: moe.moe_shuffle_plan(dp2, dp1, F, S, n, beta, w_max, ws_plan), 20)
    rank = group[cur]
    canon = np.arange(c.T) // (c.T // c.P)
    own = owner.cpu().numpy()
    return dict(trace=c.name, T=c.T, E=c.E, k=c.k, P=c.P, fit_tokens=c.fit_tokens,
                placement="correlated", beta=beta, w_max=w_max, fit_ms=round(fit_ms, 4),
                plan_ms=round(plan_ms, 4),
                locality_canonical_pct=round(100.0 * float((rank == canon[:, None]).mean()), 2),
                locality_shuffled_pct=round(100.0 * float((rank == own[:, None]).mean()), 2))


def dense_reference(w, steps=10, warmup=6) -> dict:
    """The shared expert's gate/up product of workload w (N x 2I x H, bf16) as one dense GEMM:
    this library's grouped GEMM with no routed groups (packed weights, SwiGLU epilogue) against
    torch.mm (the vendor GEMM, no epilogue) on the same operands. Milliseconds per launch from
    HIP events, back to back (warm caches)."""
    import torch

    from dispatch_expert_gemm_amd import moe
    M, H, I = w.N, w.H, w.I
    g = torch.Generator(device="cuda").manual_seed(w.seed)
    x = torch.randn(M, H, device="cuda", generator=g).to(torch.bfloat16)
    wgu = (torch.randn(1, 2 * I, H, device="cuda", generator=g) * H ** -0.5).to(torch.bfloat16)
    wd = (torch.randn(1, H, I, device="cuda", generator=g) * I ** -0.5).to(torch.bfloat16)
    wt = wgu[0].t().contiguous()
    wgu_p, wd_p = moe.moe_pack_weights(wgu, 2), moe.moe_pack_weights(wd, 1)
    h = torch.empty(1, M, I, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(1, M, H, dtype=torch.bfloat16, device="cuda")

    def ours():
        moe.moe_expert_ffn(None, None, 0, None, None, None, None, 0, shared_x=x,
                           shared_w_gate_up=wgu_p, shared_w_down=wd_p, shared_h=h, shared_y=y,
                           phases=1, weights_packed=True)

    def vendor():
        torch.mm(x, wt)

    out = dict(shape=f"{M} x {2 * I} x {H}", flops=2.0 * M * 2 * I * H)
    for name, fn in (("library", ours), ("torch_mm", vendor)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / steps
        out[name] = dict(ms=round(ms, 4), TFLOPs=round(out["flops"] / (ms * 1e-3) / 1e12, 1))
    return out


def small_batch(steps=50, warmup=20) -> list:
    """The layer at decode batch sizes, route from logits, every rank's share: the library's
    separate launches (eager, and replayed as one HIP graph) against the one-launch fused layer
    (moe_layer_fused, eager and as a graph). Milliseconds per step from HIP events around
    `steps` steps after `warmup`."""
    import torch

    from dispatch_expert_gemm_amd import workloads as WL
    from dispatch_expert_gemm_amd.layer import FusedLayerRun, MoELayerRun

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / steps

    def graph_of(fn):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    rows = []
    for cfg, N in ((1, 64), (2, 64), (2, 256), (2, 512)):
        w0 = WL.WORKLOADS[cfg]
        w = w0 if N == w0.N else WL.shrink(w0, N=N)
        multi = MoELayerRun(w)                       # packed weights where the shapes allow
        fused = FusedLayerRun(multi)                 # the same inputs and weights
        g_multi = graph_of(multi.step)
        g_fused = graph_of(fused.step)
        row = dict(workload=w.name, N=N,
                   multi_launch_ms=round(timed(multi.step), 4),
                   multi_launch_graph_ms=round(timed(g_multi.replay), 4),
                   fused_ms=round(timed(fused.step), 4),
                   fused_graph_ms=round(timed(g_fused.replay), 4),
                   fused_error=fused.error())
        row["fused_vs_graph"] = round(row["multi_launch_graph_ms"] / row["fused_graph_ms"], 3)
        rows.append(row)
        del multi, fused, g_multi, g_fused
        torch.cuda.empty_cache()
    return rows


TABLE1_TRACES = {2: "ec-top2-p8", 6: "ec-top6-p8"}


def table1(ranks=(8, 16, 32)) -> list:
    """Expert Coupling in MoE Pretraining, section II-B, Table I, on synthetic correlated routing:
    128 experts, top-2 and top-6 (the planner's stand-in traces: each token has a latent class
    that prefers 8 experts), EP8/16/32, contiguous placement against the correlated placement
    (co-selection counts of the trace's fit tokens on the device, then Algorithm 1), measured on
    the trace's evaluation tokens through the library's deduplicating layout: same-GPU % (tokens
    whose k experts sit on one rank), GPUs per token (dedup rows / tokens) and dedup % (1 - D /
    (N k)). The pages' printed row is reported beside each."""
    import numpy as np
    import torch

    from dispatch_expert_gemm_amd import moe
    from dispatch_expert_gemm_amd import workloads as WL
    golden = json.load(open(os.path.join(ROOT, "tests", "golden", "ec_table1.json")))["rows"]
    rows = []
    for k, name in TABLE1_TRACES.items():
        c = WL.SHUFFLE_TRACES[name]
        fit = torch.from_numpy(WL.gen_shuffle_trace(c, "fit")[2]).cuda()
        cur = torch.from_numpy(WL.gen_shuffle_trace(c, "eval")[2]).cuda()
        counts = moe.moe_coselect_counts(fit, c.E).cpu().numpy()
        for P in ranks:
            group, swaps = moe.moe_placement_partition(counts, P)
            for kind, pl in (("contiguous", None), ("correlated", group)):
                lay = moe.Layout(c.T, c.E, k, P, 8)
                moe.moe_dispatch_layout(lay, cur, None if pl is None else
                                        torch.from_numpy(pl).cuda())
                torch.cuda.synchronize()
                D = int(lay["pair_offsets"][P])
                per_tok = np.bincount(lay["pair_token"][:D].cpu().numpy(), minlength=c.T)
                ref = [r for r in golden if r["topk"] == k and r["EP"] == P and
                       r["placement"] == kind]
                rows.append(dict(topk=k, EP=P, placement=kind, tokens=c.T,
                                 same_gpu_pct=round(100.0 * float((per_tok == 1).mean()), 2),
                                 gpus_per_token=round(D / c.T, 3),
                                 dedup_pct=round(100.0 * (1 - D / (c.T * k)), 2),
                                 swaps=swaps if kind == "correlated" else 0,
                                 pages_table1=({x: ref[0][x] for x in ("same_gpu", "gpus",
                                                                       "dedup")}
                                               if ref else None)))
    return rows


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the hot path here "
              "is one GPU's share of the expert-parallel layer", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from dispatch_expert_gemm_amd import workloads as WL
    from dispatch_expert_gemm_amd.layer import MoELayerRun

    w = WL.WORKLOADS[args.workload]
    if args.route_from is None:
        args.route_from = default_route_from(w)
    args.fused_gate = args.route_from == "x"
    if args.fused_gate and not (w.H % 32 == 0 and w.E <= 256):
        print("the router linear layer needs H a multiple of 32 and E <= 256: use --route-from "
              "logits", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mb:
        # the source is written first, then a 1 GiB buffer evicts it from the 256 MB MALL, so
        # the copy reads and writes exactly its size in HBM
        n = args.copy_calibration_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        flush = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst, flush
    placement = None
    if args.placement == "correlated":
        from dispatch_expert_gemm_amd import moe
        probe = MoELayerRun(w)
        probe.route()
        counts = moe.moe_coselect_counts(probe.topk_idx, w.E).cpu().numpy()
        placement, _ = moe.moe_placement_partition(counts, w.W)
        del probe
    run = MoELayerRun(w, placement=placement, pack=False if args.plain_weights else None)
    if args.gemm_cus:
        from dispatch_expert_gemm_amd import moe
        moe.moe_set_gemm_max_cus(args.gemm_cus)
    run.route()
    run.dispatch()
    run.place_standins()

    names = ("route", "dispatch", "gemm1", "gemm2", "combine")

    do_route = run.gate_route if args.fused_gate else run.route

    def step(ev):
        ev[0].record()
        do_route()
        ev[1].record()
        run.dispatch()
        ev[2].record()
        run.ffn(phases=1)
        ev[3].record()
        run.ffn(phases=2)
        ev[4].record()
        run.combine()
        ev[5].record()

    # the step as the library runs it: one stream (or, with --overlap, the shared experts on a
    # second stream while route and dispatch run)
    overlap = args.overlap and run.swiglu and run.sw_gu is not None
    for _ in range(args.warmup):
        run.step(args.fused_gate, overlap)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run.step(args.fused_gate, overlap)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the same step pipelined over microbatches (route and dispatch of the next microbatch
    # beside the expert FFN of the current one), for comparison
    microbatch = None
    if args.microbatches > 1:
        from dispatch_expert_gemm_amd.layer import MicrobatchLayer
        mb = MicrobatchLayer(w, args.microbatches, full=run)
        for _ in range(args.warmup):
            mb.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            mb.step()
        torch.cuda.synchronize()
        mb_wall = time.perf_counter() - t0
        microbatch = dict(M=args.microbatches, tokens_per_microbatch=w.N // args.microbatches,
                          ms_per_step=round(mb_wall * 1e3 / args.steps, 5),
                          tokens_per_s=round((w.owned[1] - w.owned[0]) * args.steps / mb_wall, 1),
                          vs_whole_step=round(wall / mb_wall, 4))
        del mb

    # per-phase times from the same number of single-stream steps with events between phases
    # (shared and routed experts in the same launches: the launches the profiles cover)
    # each preceded (outside its events) by a read of 1 GiB, which leaves nothing of the step's
    # inputs in L2 or the 256 MB MALL. A read, not a write: a write would leave the MALL full of
    # dirty lines whose write-back the step's first kernels would pay (a 256 MB copy right after
    # a 1 GiB fill runs at 4.3 TB/s, after a 1 GiB read at 5.7)
    flush = None if args.no_flush else torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush_sink = torch.empty((), dtype=torch.float32, device="cuda")
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for _ in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()
    evs = [mk() for _ in range(args.steps)]
    for i in range(args.steps):
        if flush is not None:
            torch.amax(flush, 0, out=flush_sink)
        step(evs[i])
    torch.cuda.synchronize()
    del flush

    # the fused gate (router linear layer + route), timed on its own after the steps
    gate_ms = None
    if w.H % 32 == 0 and w.E <= 256:
        run.gate_route()
        torch.cuda.synchronize()
        ge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ge[0].record()
        for _ in range(10):
            run.gate_route()
        ge[1].record()
        torch.cuda.synchronize()
        gate_ms = ge[0].elapsed_time(ge[1]) / 10
        run.route()                         # leave the step's own routing in place

    # a plain device-to-device copy of 512 MiB (reads and writes 1 GiB of HBM): the measured
    # bandwidth the HBM-bound kernels are also compared with
    csrc = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    torch.cuda.synchronize()
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ce[0].record()
    for _ in range(5):
        cdst.copy_(csrc)
    ce[1].record()
    torch.cuda.synchronize()
    copy_gbs = 2 * csrc.numel() * 4 * 5 / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e9
    del csrc, cdst

    ms = {n: [] for n in names}
    for ev in evs:
        for j, n in enumerate(names):
            ms[n].append(ev[j].elapsed_time(ev[j + 1]))
    med = {n: float(np.median(v)) for n, v in ms.items()}
    mean = {n: float(np.mean(v)) for n, v in ms.items()}

    L = run.layout
    r = max(w.dst_rank, 0)
    rows = int(L["rank_counts"][r]) if w.dst_rank >= 0 else w.N * w.k
    pairs = (int(L["pair_counts"][r]) if w.dst_rank >= 0 else int(L["pair_offsets"][w.W]))
    alg = algorithmic(w, rows, pairs)
    t_owned = w.owned[1] - w.owned[0]
    ms_step = wall * 1e3 / args.steps
    value = t_owned * args.steps / wall
    if args.graph:
        g = run.capture(fused_gate=args.fused_gate, overlap_shared=overlap)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        gwall = time.perf_counter() - t0
        ms_step = gwall * 1e3 / args.steps
        value = t_owned * args.steps / gwall

    kernels = {}
    # with the route from x the route phase is the router linear layer plus the selection: it
    # reads x and W_R, writes the logits and the selection
    gate_bytes = (w.N * w.H * w.elt_bytes + w.E * w.H * 4 + w.N * w.E * 4 + w.N * w.k * 8)
    for n, key in (("route", "route_bytes"), ("dispatch", "permute_bytes"),
                   ("combine", "combine_bytes")):
        nbytes = gate_bytes if (n == "route" and args.fused_gate) else alg[key]
        gbs = nbytes / (mean[n] * 1e-3) / 1e9
        kernels[n] = dict(ms=round(mean[n], 5), GBps=round(gbs, 1),
                          frac_hbm=round(gbs / PEAK_HBM_GBS, 4),
                          frac_copy=round(gbs / copy_gbs, 4))
    kernels["route"]["from"] = "x" if args.fused_gate else "logits"
    kernels["copy_reference"] = dict(GBps=round(copy_gbs, 1),
                                     frac_hbm=round(copy_gbs / PEAK_HBM_GBS, 4))
    # routing statistics of the batch (Expert Coupling in MoE Pretraining, section II-B and
    # Table I: dispatched rows removed by deduplication, token-expert assignments served on the
    # token's own rank, per-rank load)
    slots = w.N * w.k
    rc = L["rank_counts"].cpu().numpy().astype(np.float64)
    sc = L["send_counts"].cpu().numpy().reshape(w.W, w.W)
    D = int(L["pair_offsets"][w.W])
    routing = dict(dedup_rows=D, dedup_pct=round(100.0 * (1 - D / slots), 2),
                   locality_pct=round(100.0 * float(np.trace(sc)) / slots, 2),
                   rank_load_ratio=round(float(rc.max() / rc.mean()), 3),
                   placement=args.placement)

    if gate_ms is not None:
        eb = w.elt_bytes
        g_bytes = w.N * w.H * eb + w.E * w.H * 4 + w.N * w.E * 4 + w.N * w.k * 8
        g_flops = 2.0 * w.N * w.H * w.E * (3 if w.dtype == "f32" else 2)
        kernels["gate_route"] = dict(ms=round(gate_ms, 5),
                                     GBps=round(g_bytes / (gate_ms * 1e-3) / 1e9, 1),
                                     frac_hbm=round(g_bytes / (gate_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                     mfma_TFLOPs=round(g_flops / (gate_ms * 1e-3) / 1e12, 1),
                                     in_step=bool(args.fused_gate))
    roofline = None
    if w.expert == "swiglu":
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
        for n in ("gemm1", "gemm2"):
            tf = alg[n + "_flops"] / (mean[n] * 1e-3) / 1e12
            kernels[n] = dict(ms=round(mean[n], 5), TFLOPs=round(tf, 1), frac_mfma=round(tf / peak, 4))
        g_ms = mean["gemm1"] + mean["gemm2"]
        g_fl = alg["gemm1_flops"] + alg["gemm2_flops"]
        compute_ms = g_fl / (peak * 1e12) * 1e3
        weight_ms = alg["gemm_weight_bytes"] / (PEAK_HBM_GBS * 1e9) * 1e3
        kernels["gemm_total"] = dict(ms=round(g_ms, 5), flops=g_fl,
                                     weight_bytes=alg["gemm_weight_bytes"],
                                     compute_bound_ms=round(compute_ms, 5),
                                     weight_stream_bound_ms=round(weight_ms, 5),
                                     frac_of_bound=round(max(compute_ms, weight_ms) / g_ms, 4))
        a1 = alg["gemm1_flops"] / (mean["gemm1"] * 1e-3) / 1e12
        key = "moe::ffn_gemm_bf16<2" if w.dtype == "bf16" else "moe::ffn_gemm_f32<2"
        roofline = dict(bound="mfma", achieved=round(a1, 2), peak=peak, unit="TFLOP/s",
                        frac=round(a1 / peak, 4), traffic=measured_traffic(w, key),
                        kernel=key, flops_per_launch=alg["gemm1_flops"],
                        avg_launch_ms=round(mean["gemm1"], 5))
    else:
        gbs = alg["combine_bytes"] / (mean["combine"] * 1e-3) / 1e9
        roofline = dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=round(gbs / PEAK_HBM_GBS, 4), traffic=None, kernel="combine",
                        bytes_per_launch=alg["combine_bytes"])
    # the committed kernel-duration and traffic summaries of this workload, if any
    for name, rel in (("profile", f"profiles/kernel_stats_{w.name}.md"),
                      ("traffic_profile", f"profiles/hbm_traffic_ffn_gemm1_{w.name}.md")):
        if os.path.exists(os.path.join(ROOT, rel)):
            roofline[name] = rel

    cpu = None
    if not args.no_cpu_baseline:
        # a sample of about 1-3 s of fp64 BLAS per oracle pass
        per_token = 6.0 * w.H * max(w.I, 1) * (w.k + w.n_shared)
        n = args.cpu_tokens or min(w.N, 4096, max(256, int(1.2e12 / per_token)))
        cpu = cpu_baseline(w, run.host, n)

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "N": w.N, "H": w.H, "E": w.E, "k": w.k, "W": w.W,
                   "I": w.I, "n_shared": w.n_shared, "gate": w.gate, "expert": w.expert,
                   "dedup": w.dedup, "dst_rank": w.dst_rank, "owned_tokens": t_owned,
                   "rows": rows, "dedup_rows": pairs,
                   "route_from": "x (router linear layer on the device)" if args.fused_gate
                   else "precomputed logits",
                   "weights": "packed once at set-up (moe_pack_weights)" if run.packed
                   else "plain K-contiguous layout",
                   "launch": ("hip graph replay" if args.graph else "eager launches") +
                   (", shared experts on a second stream" if overlap else "") +
                   (f", grouped GEMM capped at {args.gemm_cus} compute units"
                    if args.gemm_cus else "")},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "routing": routing,
        "microbatch": microbatch,
        "device": device_info(),
        "phase_timing": "single-stream steps, each after a 1 GiB read that evicts L2 and the MALL"
        if not args.no_flush
        else "single-stream steps, back to back",
    }
    if args.shuffle:
        res["shuffle"] = shuffle_planner("ec-top6-p8")
    if args.table1:
        res["table1"] = table1()
    if args.small_batch:
        res["small_batch"] = small_batch()
    if args.dense_reference and w.n_shared > 0 and w.dtype == "bf16":
        res["dense_reference"] = dense_reference(w)
    line = json.dumps(res)
    print(line, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
