"""Benchmark of the NVFP4 W4A16 routed-expert MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config C] [--only] [--gpus 1]

A step is one pass of the hot path over one batch of synthetic input:
router top-k + permutation and the layer forward (gate/up grouped GEMM +
SwiGLU, down grouped GEMM, routing-weighted combine), issued as one
moe_w4a16_route_forward call (one token: two kernel launches, the route
computed inside the gate/up kernel), or with --split as moe_route_topk
followed by moe_w4a16_forward.  Quantization is load time and is not in a
step.

Workloads (hidden 5120, intermediate 1536, 256 experts, top-8, one seeded
layer): decode with 1 token (the headline, default --config 1), decode with
8 tokens (MTP at 4 streams, shared router bias), a 1024-token prefill chunk
and a 16384-token prefill with Zipf(1.1) expert popularity.  All four are
measured in one run; the headline's fields are the top level of the JSON
line and the others sit under "configs" with the same fields.  Inputs are
resident in HBM before timing.  Decode workloads cycle through 16 distinct
device copies of the packed layer so that the 256 MB Infinity Cache cannot
serve the weights (a model has one such layer per MoE block); prefill
workloads read all of a layer's touched experts (GBs) per step and use one.
The timed region replays a HIP graph of `copies` consecutive steps at least
10 times (more when --steps asks for more steps; without --steps, 400 decode
steps and 200 prefill steps after 40 and 20 warm-up steps); "steps" is the
number of steps actually timed and "step_spread" gives p10/p50/p90 over the
replays.

Each workload also carries "roofline" (the dominant kernel, timed by HIP
events that its own launches stamp, against the roofline that binds it) and
"cpu_baseline" (the oracle timed on the host cores on a bounded sample of
the same workload, after all GPU work).  The top level adds
"achievable_peaks" (a 1 GiB device copy and an 8192^3 bf16 GEMM by the
torch/ROCm libraries, for context beside the spec peaks).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
METRIC = "MoE-layer tokens/s + weight GB/s (decode) and TFLOP/s (prefill), % roofline"


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", type=int, default=1,
                    help="headline workload index (1 = decode, 1 token); the others follow under \"configs\"")
    ap.add_argument("--only", action="store_true", help="measure the headline workload alone")
    ap.add_argument("--copies", type=int, default=None, help="layer copies cycled through (decode)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-peaks", action="store_true", help="skip the achievable-peak measurements")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget per workload")
    ap.add_argument("--prefill-variant", type=int, default=2,
                    help="grouped-GEMM kernels (moe_debug_set_prefill_variant): 0 register-staged, "
                         "1 LDS-pipelined, 2 chosen per product by rows per expert (default)")
    ap.add_argument("--split", action="store_true",
                    help="step = moe_route_topk + moe_w4a16_forward (two calls) instead of route_forward")
    ap.add_argument("--router", choices=("none", "fused", "separate"), default="none",
                    help="start the step from the BF16 router GEMM (router weights N(0, 1/H); the routing then "
                         "follows x, not the workload's drawn logits): fused = moe_router_route_topk + "
                         "moe_w4a16_forward, separate = moe_router_logits + moe_w4a16_route_forward")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM counter scaling)")
    ap.add_argument("--op", choices=("moe", "w4a4", "linear", "shared", "router"), default="moe",
                    help="moe: the routed layer (default); w4a4: the same layer with NVFP4 activations under "
                         "the static input scales (moe_w4a4_route_forward per step); "
                         "linear: a dense H x H NVFP4 projection "
                         "(moe_w4a16_linear); shared: the shared expert (moe_w4a16_shared_expert); "
                         "router: the BF16 router logits (moe_router_logits); all at the workload's "
                         "token count and shapes")
    return ap.parse_args()


def packed_bytes(N, K):
    return N * K // 2 + N * K // 16 + 4


def kernel_source_hash(kernel):
    from nvfp4_weight_only_moe_amd import pmc
    return pmc.kernel_source_hash(kernel)


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter profile, or None when
    there is none for this kernel/workload or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(f"{kernel}@{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer fits one MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch
    from nvfp4_weight_only_moe_amd import binding as B
    from nvfp4_weight_only_moe_amd import workloads as wls

    if args.op not in ("moe", "w4a4"):
        return bench_single(args, wls.WORKLOADS[args.config])
    B.moe_debug_set_prefill_variant(args.prefill_variant)
    torch.cuda.set_device(0)
    t0 = time.time()
    base, quant_ms = build_layer(wls.WORKLOADS[1])      # the one full-size layer of workloads 1-4
    log(f"layer packed ({time.time() - t0:.1f} s)")

    # the headline workload first, then the others in the same process
    cfgs = [args.config] if args.only else [args.config] + [c for c in (1, 2, 3, 4) if c != args.config]
    results = {}
    copies_cache = {}
    for cfg in cfgs:
        results[cfg] = bench_moe_config(args, cfg, base, copies_cache)
        torch.cuda.empty_cache()
    copies_cache.clear()

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 copies of 268435456 bytes (read 256 MiB, write 256 MiB each)")

    # what plain library work reaches on this GPU, beside the spec peaks the
    # roofline uses: a 1 GiB device copy (read + write) and a bf16 GEMM
    achievable = None if args.no_peaks else achievable_peaks()

    # the oracle on the host, per workload, after every GPU measurement
    if not args.no_cpu:
        for cfg in cfgs:
            results[cfg]["cpu_baseline"] = cpu_baseline(wls.WORKLOADS[cfg], args.cpu_seconds,
                                                        w4a4=args.op == "w4a4")
            log(f"cpu baseline {wls.WORKLOADS[cfg].name}: {results[cfg]['cpu_baseline']['value']} tokens/s")

    head = results[cfgs[0]]
    rec = {"metric": METRIC}
    rec.update({k: head[k] for k in ("value", "unit")})
    rec.update({"n_gpus": 1, "steps": head["steps"], "warmup": head["warmup"], "ms_per_step": head["ms_per_step"],
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                "data": "synthetic"})
    rec["config"] = head["config"]
    for key in ("roofline", "cpu_baseline", "steps_requested", "step_spread", "step_algorithmic_GBps",
                "step_hbm_frac", "weight_GBps", "step_TFLOPs", "step_mfma_frac", "eager_ms_per_step",
                "per_kernel_us"):
        rec[key] = head.get(key)
    rec["configs"] = {results[c]["config"]["workload"]: results[c] for c in cfgs[1:]}
    rec["quantize_pack_ms_total"] = round(quant_ms, 2)
    rec["achievable_peaks"] = achievable
    rec["gpu_clocks_after_timing"] = head.get("gpu_clocks_after_timing")
    print(json.dumps(rec), flush=True)


def build_layer(wl):
    """Generate the seeded fp32 masters of the full-size layer on the host and
    quantize them on the GPU (load time, not part of a step).  Returns the
    packed layer and the GPU quantize time in ms."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    from nvfp4_weight_only_moe_amd import binding as B
    from nvfp4_weight_only_moe_amd import workloads as wls

    dev = "cuda:0"
    threads = min(16, len(os.sched_getaffinity(0)))
    layer = {}
    quant_ms = 0.0
    for proj, name in ((wls.GATE, "gate"), (wls.UP, "up"), (wls.DOWN, "down")):
        n, k = wls.proj_shape(wl, proj)
        t = B.NVFP4Tensor.empty(wl.E, n, k, dev)
        batch = 32
        with ThreadPoolExecutor(threads) as ex:
            for e0 in range(0, wl.E, batch):
                ms = np.stack(list(ex.map(lambda e: wls.master(wl, proj, e), range(e0, e0 + batch))))
                w = torch.from_numpy(ms).to(dev)
                sl = B.NVFP4Tensor(t.codes[e0:e0 + batch], t.scales[e0:e0 + batch], t.global_scale[e0:e0 + batch])
                torch.cuda.synchronize()
                q0 = time.perf_counter()
                B.moe_w4a16_quantize_pack(w, out=sl)
                torch.cuda.synchronize()
                quant_ms += (time.perf_counter() - q0) * 1e3
                del w
        layer[name] = t
    flag = torch.zeros((4,), dtype=torch.int32, device=dev)
    for name in ("gate", "up", "down"):
        B.moe_w4a16_validate(layer[name], flag)
    return layer, quant_ms


def layer_copies(base, copies, cache):
    """`copies` distinct device copies of the packed layer (the first is the
    layer itself): a step cycles through them so the 256 MB Infinity Cache
    cannot serve the weights, as with a model's many MoE layers."""
    from nvfp4_weight_only_moe_amd import binding as B
    lst = cache.setdefault("copies", [base])
    while len(lst) < copies:
        lst.append({n: B.NVFP4Tensor(t.codes.clone(), t.scales.clone(), t.global_scale.clone())
                    for n, t in base.items()})
    return lst[:copies]


def bench_moe_config(args, cfg, base, cache):
    """One workload: graph-replayed steps (route + layer), per-kernel times,
    roofline of the dominant kernel."""
    import torch
    from nvfp4_weight_only_moe_amd import binding as B
    from nvfp4_weight_only_moe_amd import workloads as wls

    wl = wls.WORKLOADS[cfg]
    dev = "cuda:0"
    decode = wl.T <= 8
    steps_req = args.steps or (400 if decode else 200)
    warmup = args.warmup if args.warmup is not None else (40 if decode else 20)
    copies = args.copies or (16 if decode else 1)
    layers = layer_copies(base, copies, cache)
    torch.cuda.synchronize()

    xb, _ = wls.activations(wl)
    lg = wls.logits(wl)
    x_d = torch.from_numpy(xb.view(np.int16)).to(dev)
    lg_d = torch.from_numpy(lg).to(dev)
    route = B.Routing.empty(wl.T, wl.E, wl.k, dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.int16, device=dev)
    ws = B.forward_workspace(wl.T, wl.H, wl.I, wl.E, wl.k, dev)

    if args.router != "none":
        _, _, wb, _ = wls.router_problem(7, 1, wl.H, wl.E)
        wr_d = torch.from_numpy(wb.view(np.int16)).to(dev)
        rws = B.router_route_workspace(wl.T, wl.E, wl.k, dev)

    if args.op == "w4a4":
        sx, sh = wls.W4A4_INPUT_SCALES
        ws4 = torch.empty((max(B.moe_w4a4_workspace_size(wl.T, wl.H, wl.I, wl.E, wl.k), 256),), dtype=torch.uint8,
                          device=dev)

    def step(i):
        L = layers[i % copies]
        if args.op == "w4a4":
            B.moe_w4a4_route_forward(lg_d, x_d, L["gate"], L["up"], L["down"], wl.k, sx, sh, routing=route, out=out,
                                     ws=ws4)
        elif args.router == "fused":
            B.moe_router_route_topk(x_d, wr_d, wl.k, logits=lg_d, routing=route, ws=rws)
            B.moe_w4a16_forward(x_d, L["gate"], L["up"], L["down"], route, out=out, ws=ws)
        elif args.router == "separate":
            B.moe_router_logits(x_d, wr_d, out=lg_d)
            B.moe_w4a16_route_forward(lg_d, x_d, L["gate"], L["up"], L["down"], wl.k, routing=route, out=out, ws=ws)
        elif args.split:
            B.moe_route_topk(lg_d, wl.k, out=route)
            B.moe_w4a16_forward(x_d, L["gate"], L["up"], L["down"], route, out=out, ws=ws)
        else:
            B.moe_w4a16_route_forward(lg_d, x_d, L["gate"], L["up"], L["down"], wl.k, routing=route, out=out, ws=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ref_out = out.clone()
    counts = route.counts.cpu().numpy()
    U = int((counts > 0).sum())

    def timed(fn, n):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(n)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    n_eager = max(steps_req, copies)
    eager_ms = timed(lambda n: [step(i) for i in range(n)], n_eager)
    assert torch.equal(out, ref_out)

    # timed region: R replays of a graph of `copies` consecutive steps, at
    # least 10 so that the spread is over real samples; every replay is
    # bracketed by its own events (stream-ordered, no synchronisation between)
    graph_ms, spread, steps_timed = None, None, n_eager
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(2):
                step(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(copies):
                step(i)
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref_out):
            log(f"{wl.name}: graph replay output differs from eager: graph timing discarded")
        else:
            reps = max(10, -(-steps_req // copies))
            for _ in range(3):
                g.replay()
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            torch.cuda.synchronize()
            evs[0].record()
            for r in range(reps):
                g.replay()
                evs[r + 1].record()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out)
            per = sorted(evs[r].elapsed_time(evs[r + 1]) / copies * 1e3 for r in range(reps))
            graph_ms = evs[0].elapsed_time(evs[reps]) / (reps * copies)
            steps_timed = reps * copies
            q = lambda f: round(per[int(round(f * (len(per) - 1)))], 3)
            spread = {"p10_us": q(0.1), "p50_us": q(0.5), "p90_us": q(0.9), "samples": reps,
                      "steps_per_sample": copies}
    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    log(f"{wl.name}: {ms_per_step * 1e3:.2f} us/step over {steps_timed} steps (eager {eager_ms * 1e3:.2f})")

    # per-kernel times from events the launches stamp themselves
    n_prof = max(steps_req, 10)
    B.moe_profile_begin(64 * n_prof)
    for i in range(n_prof):
        step(i)
    prof = B.moe_profile_end()
    per_kernel_us = {k: round(v[1] / v[0] * 1e3, 3) for k, v in prof.items()}
    dominant = max(prof, key=lambda k: prof[k][1])
    dom_us = prof[dominant][1] / prof[dominant][0] * 1e3
    log(f"{wl.name}: per-kernel us {per_kernel_us}")
    clocks = gpu_clocks()

    H, I, T, k = wl.H, wl.I, wl.T, wl.k
    w_gu, w_d = 2 * packed_bytes(I, H), packed_bytes(H, I)
    alg_bytes_step = U * (w_gu + w_d) + T * H * 2 * 2 + T * wl.E * 4
    if args.router != "none":
        alg_bytes_step += wl.E * H * 2                  # the BF16 router weight
    flops_step = 6.0 * T * k * H * I
    # (algorithmic bytes, flops) per launch; the grouped GEMMs read every
    # touched expert's weights once and do 2 flops per weight per row
    kernel_work = {
        "dec_gateup": (U * w_gu + T * H * 2, None),
        "dec_gateup_route": (U * w_gu + T * H * 2 + T * wl.E * 4, None),
        "dec_down": (U * w_d + T * H * 2, None),
        "gemm_gateup": (U * w_gu + T * H * 2, 4.0 * T * k * H * I),
        "gemm_down": (U * w_d + T * H * 2, 2.0 * T * k * H * I),
        "router_route": (wl.E * H * 2 + T * H * 2 + T * wl.E * 4, None),
        "router_gemv": (wl.E * H * 2 + T * H * 2 + T * wl.E * 4, None),
    }
    work_bytes, work_flops = kernel_work.get(dominant, (alg_bytes_step, None))
    traffic = None if args.op == "w4a4" else measured_traffic(dominant, wl.name)   # counters are of W4A16 runs
    roofline = make_roofline(dominant, dom_us, work_bytes, work_flops, traffic)
    if decode and not args.no_peaks and args.router == "none":
        # what a kernel that only reads reaches on the same byte counts: the
        # two decode kernels' bytes, each alone (event-timed like the
        # kernels) and back to back (graph-replayed like the steps)
        gu_key = "dec_gateup_route" if "dec_gateup_route" in prof else "dec_gateup"
        ref = stream_reference([kernel_work[gu_key][0], kernel_work["dec_down"][0]], copies)
        dom_ref = ref["kernel_us"][0] if dominant == gu_key else ref["kernel_us"][1] if dominant == "dec_down" else None
        roofline["achievable"] = {
            "what": "plain streaming read of the same bytes (moe_bench_stream_read)",
            "kernel_bytes": ref["bytes"], "kernel_us": ref["kernel_us"],
            "dominant_kernel_frac": round(dom_ref / dom_us, 4) if dom_ref else None,
            "step_pair_us": ref["pair_us"],
            "step_frac": round(ref["pair_us"] / (ms_per_step * 1e3), 4),
        }
        log(f"{wl.name}: plain reads of the same bytes {ref}")
    sec = ms_per_step * 1e-3
    return {
        "value": round(T / sec, 2), "unit": "tokens/s", "steps": steps_timed, "steps_requested": steps_req,
        "warmup": warmup, "ms_per_step": round(ms_per_step, 6),
        "config": {"workload": wl.name, "T": T, "H": H, "I": I, "E": wl.E, "k": k, "layer_copies": copies,
                   "hip_graph": graph_ms is not None, "touched_experts": U,
                   "max_rows_per_expert": int(counts.max()),
                   "step_calls": ("w4a4_route_forward" if args.op == "w4a4" else
                                  "router_route_topk+forward" if args.router == "fused" else
                                  "router_logits+route_forward" if args.router == "separate" else
                                  "route_topk+forward" if args.split else "route_forward"),
                   "prefill_variant": None if decode else args.prefill_variant,
                   "activations": ("NVFP4 (W4A4, static input scales "
                                   f"{wls.W4A4_INPUT_SCALES[0]:.6g}, {wls.W4A4_INPUT_SCALES[1]:.6g})"
                                   if args.op == "w4a4" else "bf16 (W4A16)")},
        "roofline": roofline, "cpu_baseline": None, "step_spread": spread,
        "step_algorithmic_GBps": round(alg_bytes_step / sec / 1e9, 1),
        "step_hbm_frac": round(alg_bytes_step / sec / 1e9 / HBM_PEAK_GBPS, 4),
        "weight_GBps": round(U * (w_gu + w_d) / sec / 1e9, 1),
        "step_TFLOPs": round(flops_step / sec / 1e12, 3),
        "step_mfma_frac": round(flops_step / sec / 1e12 / BF16_PEAK_TFLOPS, 5),
        "eager_ms_per_step": round(eager_ms, 6), "per_kernel_us": per_kernel_us,
        "gpu_clocks_after_timing": clocks,
    }


def stream_reference(sizes, launches):
    """moe_bench_stream_read on the given byte counts (rounded down to 16):
    each size's per-launch time from the launches' own events (as the
    kernels' times), and the time of the sizes read back to back, from
    replays of a HIP graph of `launches` such sequences (as the steps).  The
    reads rotate through a pool of at least 1 GiB so that the 256 MB Infinity
    Cache cannot serve them."""
    import torch
    from nvfp4_weight_only_moe_amd import binding as B
    sizes = [int(b) // 16 * 16 for b in sizes]
    seq = sum(sizes)
    pool = torch.empty(max(1 << 30, 3 * seq), dtype=torch.uint8, device="cuda:0")
    pool.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    slots = max(1, (pool.numel() - seq) // seq + 1)

    def one(i):
        o = (i % slots) * seq
        for b in sizes:
            B.moe_bench_stream_read(pool[o:o + b], b, sink)
            o += b

    for i in range(4):
        one(i)
    torch.cuda.synchronize()
    # per-size event times (the profile merges launches by name: one size at a time)
    n = 20
    kernel_us = []
    for j, b in enumerate(sizes):
        B.moe_profile_begin(n)
        for i in range(n):
            o = (i % slots) * seq + sum(sizes[:j])
            B.moe_bench_stream_read(pool[o:o + b], b, sink)
        prof = B.moe_profile_end()
        c, ms = prof["stream_read"]
        kernel_us.append(round(ms / c * 1e3, 3))
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        one(0)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(launches):
            one(i)
    for _ in range(3):
        g.replay()
    reps = 10
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    pair_us = a.elapsed_time(e) / (reps * launches) * 1e3
    del g, pool
    return {"bytes": sizes, "kernel_us": kernel_us, "pair_us": round(pair_us, 3)}


def achievable_peaks():
    import torch
    dev = "cuda:0"

    def timed(fn, n):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(n)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    copy_ms = timed(lambda r: [dst.copy_(src) for _ in range(r)], 5)
    del src, dst
    m = 8192
    ga = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    gb = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    gc = ga @ gb
    mm_ms = timed(lambda r: [torch.matmul(ga, gb, out=gc) for _ in range(r)], 5)
    del ga, gb, gc
    res = {"hbm_copy_GBps": round(2 * n / (copy_ms * 1e-3) / 1e9, 1),
           "bf16_gemm_8192_TFLOPs": round(2.0 * m ** 3 / (mm_ms * 1e-3) / 1e12, 1)}
    log(f"achievable: {res}")
    return res


def cpu_baseline(wl, budget_s, w4a4=False):
    """The oracle (fp64 numpy, BLAS on the host's cores) on a bounded sample
    of the workload, expert quantization excluded.  Decode workloads: route +
    FFN + combine of the first tokens (1, or 2 of the 8), repeated within the
    budget.  Prefill workloads: the route of every token, then the experts
    one at a time in ascending index, each adding its weighted FFN rows into
    an fp64 [T, H] output, until the budget is spent; the rate counts the
    rows processed (k rows make one token).  w4a4: the W4A4 oracle (the
    activations and the hidden rows quantized under the static input
    scales)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from oracle import moe as omoe
    from oracle import w4a4 as ow4
    from nvfp4_weight_only_moe_amd import workloads as wls
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    threads = min(16, len(os.sched_getaffinity(0)))
    _, x = wls.activations(wl)
    logits = wls.logits(wl)

    def quantized(experts):
        todo = [(p, n, e) for p, n in ((wls.GATE, "gate"), (wls.UP, "up"), (wls.DOWN, "down")) for e in experts]
        with ThreadPoolExecutor(threads) as ex:
            res = list(ex.map(lambda a: oracle.quantize(wls.master(wl, a[0], a[2])), todo))
        layer = {n: ({}, {}, {}) for n in ("gate", "up", "down")}
        for (p, n, e), (c, s, g) in zip(todo, res):
            layer[n][0][e], layer[n][1][e], layer[n][2][e] = c, s, g
        return layer

    if wl.T <= 8:
        n_tok = 1 if wl.T == 1 else 2
        ids, _ = oracle.route_topk(logits[:n_tok], wl.k)
        experts = sorted(set(int(e) for e in ids.ravel()))
        layer = quantized(experts)
        runs, t_total = 0, 0.0
        while t_total < budget_s and runs < 50:
            t0 = time.perf_counter()
            ids_s, w_s = oracle.route_topk(logits[:n_tok], wl.k)
            if w4a4:
                ow4.moe_forward_w4a4(x[:n_tok], layer, ids_s, w_s, *wls.W4A4_INPUT_SCALES, tokens=range(n_tok))
            else:
                oracle.moe_forward(x[:n_tok], layer, ids_s, w_s, tokens=range(n_tok))
            t_total += time.perf_counter() - t0
            runs += 1
        rate = n_tok * runs / t_total
        sample = (f"{n_tok} of {wl.T} token(s): route + {'W4A4 ' if w4a4 else ''}SwiGLU FFN of {len(experts)} "
                  f"experts (dequantize + fp64) + combine, {runs} runs, {t_total:.1f} s; expert quantization excluded")
    else:
        t0 = time.perf_counter()
        ids, w = oracle.route_topk(logits, wl.k)
        t_route = time.perf_counter() - t0
        present = sorted(set(int(e) for e in ids.ravel()))
        out = np.zeros((wl.T, wl.H))
        if w4a4:
            t0 = time.perf_counter()
            xf = ow4.fake_quantize(x, wls.W4A4_INPUT_SCALES[0]).astype(np.float64)
            t_route += time.perf_counter() - t0
        else:
            xf = x.astype(np.float64)
        t_total, rows, done, i = t_route, 0, [], 0
        while i < len(present) and t_total < budget_s:
            batch = present[i:i + 4]
            layer = quantized(batch)                     # excluded from the time
            for e in batch:
                t0 = time.perf_counter()
                r, sl = np.nonzero(ids == e)
                wg, wu, wd = omoe.dequantize_expert(layer, e)
                y = (ow4.expert_ffn_w4a4(xf[r], wg, wu, wd, wls.W4A4_INPUT_SCALES[1]) if w4a4
                     else omoe.expert_ffn(xf[r], wg, wu, wd))
                out[r] += w[r, sl][:, None] * y
                t_total += time.perf_counter() - t0
                rows += r.size
                done.append(e)
            i += len(batch)
        rate = rows / wl.k / t_total
        sample = (f"route of all {wl.T} tokens{' and their activations quantized' if w4a4 else ''} ({t_route:.1f} s), "
                  f"then {len(done)} of {len(present)} touched experts "
                  f"one at a time (ascending index), {rows} of {wl.T * wl.k} (token, expert) rows, dequantize + "
                  f"fp64 SwiGLU FFN accumulated into an fp64 [T, H] output, {t_total:.1f} s; rate = rows / k / time; "
                  f"expert quantization excluded")
    return {"value": round(rate, 4), "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": sample, "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


def bench_single(args, wl):
    """One always-on expert: the dense projection (K = N = H) or the shared
    expert (H, I), at the workload's T.  Weights of several copies are
    cycled (more than the 256 MB Infinity Cache holds) inside one HIP graph."""
    import torch
    from nvfp4_weight_only_moe_amd import binding as B
    from nvfp4_weight_only_moe_amd import workloads as wls
    from oracle import moe as omoe
    import oracle

    dev = "cuda:0"
    torch.cuda.set_device(0)
    T, H, I, E = wl.T, wl.H, wl.I, wl.E
    decode = T <= 8
    if args.op == "router":
        # the BF16 router weight [E, H]; copies cycled past the Infinity Cache
        xb, x, wb, wr = wls.router_problem(7, T, H, E)
        w_bytes = E * H * 2
        copies = args.copies or (max(1, -(-(1 << 29) // w_bytes)) if decode else 1)
        base = torch.from_numpy(wb.view(np.int16)).to(dev)
        sets = [base] + [base.clone() for _ in range(copies - 1)]
        out = torch.empty((T, E), dtype=torch.float32, device=dev)
    else:
        _, ms, xb, x, _ = wls.random_problem(7, T, H, H if args.op == "linear" else I, 1, 1)
        if args.op == "linear":
            ms = ms[:1]                                       # [1, H, H]
            w_bytes = packed_bytes(H, H)
        else:
            w_bytes = 2 * packed_bytes(I, H) + packed_bytes(H, I)
        base = [B.moe_w4a16_quantize_pack(torch.from_numpy(m).to(dev)) for m in ms]
        copies = args.copies or (max(1, -(-(1 << 30) // w_bytes)) if decode else 1)
        sets = [base] + [[B.NVFP4Tensor(t.codes.clone(), t.scales.clone(), t.global_scale.clone()) for t in base]
                         for _ in range(copies - 1)]
        out = torch.empty((T, H), dtype=torch.int16, device=dev)
    x_d = torch.from_numpy(xb.view(np.int16)).to(dev)
    if args.op == "router":
        step = lambda i: B.moe_router_logits(x_d, sets[i % copies], out=out)
    elif args.op == "linear":
        ws = torch.empty((B.lib().moe_w4a16_linear_workspace_size(T, H, H),), dtype=torch.uint8, device=dev)
        step = lambda i: B.moe_w4a16_linear(x_d, sets[i % copies][0], out=out, ws=ws)
    else:
        ws = torch.empty((B.lib().moe_w4a16_shared_expert_workspace_size(T, H, I),), dtype=torch.uint8, device=dev)
        step = lambda i: B.moe_w4a16_shared_expert(x_d, *sets[i % copies], out=out, ws=ws)
    steps = args.steps or (400 if decode else 200)
    warmup = args.warmup if args.warmup is not None else (40 if decode else 20)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ref_out = out.clone()

    def timed(fn, n):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(n)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    eager_ms = timed(lambda n: [step(i) for i in range(n)], steps)
    graph_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step(0)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(copies):
                step(i)
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        if torch.equal(out, ref_out):
            reps = max(10, -(-steps // copies))
            graph_ms = timed(lambda n: [g.replay() for _ in range(n)], reps) / copies
            steps = reps * copies
            assert torch.equal(out, ref_out)
        else:
            log("graph replay output differs from eager: graph timing discarded")
    ms_per_step = graph_ms if graph_ms is not None else eager_ms

    B.moe_profile_begin(64 * max(steps, 1))
    for i in range(steps):
        step(i)
    prof = B.moe_profile_end()
    per_kernel_us = {k: round(v[1] / v[0] * 1e3, 3) for k, v in prof.items()}
    dominant = max(prof, key=lambda k: prof[k][1])
    dom_us = prof[dominant][1] / prof[dominant][0] * 1e3
    if args.op == "router":
        rb = w_bytes + T * H * 2 + T * E * 4
        work = {"router_gemv": (rb, None), "router_mfma": (rb, 2.0 * T * H * E)}
        alg_bytes, flops = rb, 2.0 * T * H * E
    elif args.op == "linear":
        work = {"dec_linear": (w_bytes + T * H * 2 * 2, None),
                "gemm_down": (w_bytes + T * H * 2 * 2, 2.0 * T * H * H)}
        alg_bytes, flops = w_bytes + T * H * 2 * 2, 2.0 * T * H * H
    else:
        w_gu, w_d = 2 * packed_bytes(I, H), packed_bytes(H, I)
        work = {"dec_gateup": (w_gu + T * H * 2, None), "dec_down": (w_d + T * H * 2, None),
                "gemm_gateup": (w_gu + T * H * 2, 4.0 * T * H * I), "gemm_down": (w_d + T * H * 2, 2.0 * T * H * I)}
        alg_bytes, flops = w_bytes + T * H * 2 * 2, 6.0 * T * H * I
    roofline = make_roofline(dominant, dom_us, *work.get(dominant, (alg_bytes, None)), traffic=None)
    cpu = None
    if not args.no_cpu:
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            threads = 1
        packed = [oracle.quantize_layer(m) for m in ms] if args.op != "router" else None
        n_tok = min(T, 64)
        t0 = time.perf_counter()
        if args.op == "router":
            for _ in range(200):
                oracle.router_logits(x[:n_tok], wr)
            n_tok *= 200
        elif args.op == "linear":
            omoe.linear(x[:n_tok], packed[0][0][0], packed[0][1][0], packed[0][2][0])
        else:
            layer = {nm: p for nm, p in zip(("gate", "up", "down"), packed)}
            omoe.shared_expert_forward(x[:n_tok], layer)
        dt = time.perf_counter() - t0
        cpu = {"value": round(n_tok / dt, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": (f"{n_tok} token-rows of fp64 logits (numpy matmul), {dt:.1f} s" if args.op == "router" else
                          f"{n_tok} token(s): dequantize + fp64 {'projection' if args.op == 'linear' else 'SwiGLU FFN'}"
                          f", 1 run, {dt:.1f} s; quantization excluded"),
               "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}
    rec = {
        "metric": METRIC, "value": round(T / (ms_per_step * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.op}-t{T}-h{H}" + (f"-e{E}" if args.op == "router" else
                                                          f"-n{H}" if args.op == "linear" else f"-i{I}"),
                   "T": T, "H": H, "I": H if args.op == "linear" else I, "E": E, "copies": copies,
                   "hip_graph": graph_ms is not None},
        "roofline": roofline, "cpu_baseline": cpu,
        "step_algorithmic_GBps": round(alg_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(alg_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "step_TFLOPs": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "eager_ms_per_step": round(eager_ms, 6), "per_kernel_us": per_kernel_us,
    }
    print(json.dumps(rec), flush=True)


def cpu_model():
    """The host CPU's model name (the oracle baseline depends on it)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def make_roofline(kernel, avg_us, work_bytes, work_flops, traffic):
    """The dominant kernel against the roofline that binds it at this
    workload: HBM when its algorithmic bytes take longer at 8 TB/s than its
    flops at the bf16 MFMA peak (decode kernels have no flop figure), MFMA
    otherwise; "other" gives the fraction of the other peak for context."""
    t_hbm = work_bytes / (HBM_PEAK_GBPS * 1e9)
    t_mfma = work_flops / (BF16_PEAK_TFLOPS * 1e12) if work_flops else 0.0
    gbps = work_bytes / (avg_us * 1e-6) / 1e9
    tflops = work_flops / (avg_us * 1e-6) / 1e12 if work_flops else None
    hbm = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
           "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    mfma = None if tflops is None else {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
                                        "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
    main, other = (hbm, mfma) if t_hbm >= t_mfma else (mfma, hbm)
    r = dict(main)
    r.update({"traffic": traffic, "kernel": kernel, "kernel_avg_us": round(avg_us, 3),
              "algorithmic_bytes_per_launch": int(work_bytes)})
    if work_flops:
        r["algorithmic_flops_per_launch"] = work_flops
    if other is not None:
        r["other"] = {"bound": other["bound"], "achieved": other["achieved"], "unit": other["unit"],
                      "frac": other["frac"]}
    return r


def gpu_clocks():
    """Current shader and memory clocks of cuda:0 right after the timed region,
    read from the amdgpu driver's DPM tables in sysfs (the entry marked '*'),
    matched to the device by PCI address; context only, None when unreadable.
    Reading files keeps the GPU process from starting any other program."""
    import glob
    import torch
    try:
        p = torch.cuda.get_device_properties(0)
        bdf = "%04x:%02x:%02x." % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
        for dev in glob.glob("/sys/class/drm/card*/device"):
            if not os.path.basename(os.path.realpath(dev)).startswith(bdf):
                continue
            def cur(name):
                with open(os.path.join(dev, name)) as f:
                    return next((ln.split(":", 1)[1].replace("*", "").strip() for ln in f if "*" in ln), None)
            return {"sclk": cur("pp_dpm_sclk"), "mclk": cur("pp_dpm_mclk")}
    except Exception:
        pass
    return None


if __name__ == "__main__":
    main()
