#!/usr/bin/env python3
"""Benchmark one routed-MoE layer over low-bit experts on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one whole layer (route -> permute -> expert FFNs + shared expert ->
combine, through ds4moe_forward) over one batch of synthetic tokens whose
inputs are already resident in HBM.  Layer weights rotate over several copies
at distinct addresses and the router logits over a pool of 64 draws, so that
the 256 MB Infinity Cache cannot serve a step from the previous one.

Prints one JSON line: MoE-layer tokens/s for the workload (default: batch-1
decode, 7168/2048, 256 experts top-8 + bf16 shared expert, Q2K experts), the
roofline of the dominant kernel (timed live with HIP events recorded by its own
launch), a per-stage breakdown, and the CPU oracle timed on a bounded sample.

The router_decode and router_prefill workloads time the router projection
(ds4moe_router_logits) on its own instead of the layer.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at batch 1 decode & 4096-tok prefill; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (the rate of E2M1 x E4M3 products), TFLOP/s
STAGES = ("route", "permute", "ffn_up", "ffn_down", "combine")
EVENT_EVERY = 16               # timed steps that carry the dominant kernel's events
WARM_S = 0.3                   # warm-up lasts at least this long (GPU clocks settle), and at least W steps


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "batched_decode", "prefill", "mxfp4_decode", "mxfp4_prefill",
                             "q4k_decode", "q4k_prefill", "verify6", "sessions16", "router_decode",
                             "router_prefill"])
    ap.add_argument("--headline-only", action="store_true",
                    help="decode: skip the prefill and small-batch sub-records of the default run")
    ap.add_argument("--algo", default="auto", choices=["auto", "gemv", "grouped"])
    ap.add_argument("--mma", default="bf16", choices=["bf16", "fp8"],
                    help="MXFP4 experts: bf16 operands, or MXFP8 x/h on the scaled matrix instructions")
    ap.add_argument("--copies", type=int, default=0, help="layer copies to rotate (0: by workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=20261202)
    return ap.parse_args()


def expert_bytes(spec, name):
    rows, K = spec.routed_shape(name)
    if spec.wfmt == "q2k":
        return rows * K // 256 * 84
    if spec.wfmt == "q4k":
        return rows * K // 2 + rows * K // 256 * 20
    return rows * K // 2 + rows * K // 32


def shared_bytes(spec):
    return 2 * spec.shared_ffn * spec.hidden * 2


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one MI355X: --gpus {args.gpus} (WORLD_SIZE={world}) is not supported; "
              "this library runs the layer on a single GPU with no sharding or collectives.",
              file=sys.stderr)
        sys.exit(2)

    if args.workload.startswith("router_"):
        return router_main(args)

    import torch
    from synth import WORKLOADS, make_layer

    wl = WORKLOADS[args.workload]
    spec, T = wl["spec"], wl["T"]
    if args.mma == "fp8" and spec.wfmt != "mxfp4":
        print("--mma fp8 applies to the MXFP4 workloads", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # The default run (batch-1 decode) also times the 4096-token prefill chunk
    # and the small batches on the same layer copies.
    extras = args.workload == "decode" and not args.headline_only and args.algo == "auto"
    copies = args.copies or (8 if T <= 64 else 2)

    t0 = time.time()
    base = make_layer(spec, seed=args.seed, device=dev)
    layers = [base] + [base.clone() for _ in range(copies - 1)]
    torch.cuda.synchronize()
    gen_s = time.time() - t0

    out = run_workload(args.workload, layers, args, args.steps, args.warmup)
    out["step"]["layer_gen_s"] = round(gen_s, 1)
    if extras:
        # prefill: 2 of the copies (3.8 GB each, beyond the 256 MB cache)
        pre = run_workload("prefill", layers[:2], args, min(args.steps, 50), min(args.warmup, 5))
        sub = {"workload": "prefill", **{k: pre[k] for k in ("value", "unit", "ms_per_step", "steps", "warmup",
                                                             "warmup_run", "dtype", "config", "roofline", "step")}}
        out["prefill"] = sub
        out["small_batches"] = []
        for name in ("verify6", "sessions16"):
            r = run_workload(name, layers, args, args.steps, args.warmup)
            out["small_batches"].append({"workload": name, **{k: r[k] for k in (
                "value", "unit", "ms_per_step", "config", "roofline", "step")}})
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = out.pop("_cpu")()
        if extras:
            out["prefill"]["cpu_baseline"] = pre["_cpu"]()
    for r in [out] + ([out["prefill"]] + out["small_batches"] if extras else []):
        r.pop("_cpu", None)
    print(json.dumps(out), flush=True)


def warm_up(step, warmup):
    """Untimed steps: at least `warmup` of them and at least WARM_S seconds
    of them (synchronizing every 64 steps, so the wall clock follows the
    GPU), so that the timed steps run at settled clocks.  Returns (steps
    run, seconds)."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < WARM_S:
        step(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i, time.perf_counter() - t0


def run_workload(name, layers, args, steps, warmup):
    """Time ds4moe_forward on one workload over the given layer copies.
    Returns the bench record (without cpu_baseline; "_cpu" is a callable that
    times the oracle on this workload's sample)."""
    import numpy as np
    import torch
    import bit_routed_moe_amd as ds4
    from synth import WORKLOADS, make_x, make_logits

    wl = WORKLOADS[name]
    spec, T, zipf = wl["spec"], wl["T"], wl["zipf"]
    fp8 = args.mma == "fp8" and spec.wfmt == "mxfp4"
    mma = "fp8" if fp8 else "bf16"
    dev = layers[0].device
    copies = len(layers)
    x = make_x(T, spec.hidden, seed=args.seed).to(dev)
    n_pool = 64
    logits = [make_logits(T, spec.n_experts, seed=args.seed, zipf_s=zipf, index=i).to(dev) for i in range(n_pool)]
    cfg = ds4.make_config(spec.hidden, spec.ffn, spec.n_experts, spec.top_k, spec.shared_ffn, spec.wfmt,
                          act="bf16", mma=mma, algo=args.algo)
    wts = [ds4.make_weights(L.gate, L.up, L.down, L.gate_scales, L.up_scales, L.down_scales,
                            L.sh_gate, L.sh_up, L.sh_down) for L in layers]
    ws = torch.empty(ds4.workspace_bytes(cfg, T), dtype=torch.uint8, device=dev)
    path = ds4.forward_path(cfg, T)
    y = torch.empty((T, spec.hidden), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        ds4.forward(cfg, wts[i % copies], T, x, logits[i % n_pool], y, ws, stream)

    # touched experts per logits draw (library route + permute; metadata only)
    P = T * spec.top_k
    idx = torch.empty((T, spec.top_k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, spec.top_k), dtype=torch.float32, device=dev)
    off = torch.empty(spec.n_experts + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(P, dtype=torch.int32, device=dev)
    pp = torch.empty(P, dtype=torch.int32, device=dev)
    act = torch.empty(spec.n_experts + 1, dtype=torch.int32, device=dev)
    n_active = []
    for i in range(n_pool):
        ds4.route(cfg, T, logits[i], idx, tw, stream)
        ds4.permute(cfg, T, idx, off, sp, pp, act, stream)
        torch.cuda.synchronize()
        n_active.append(int(act[0].item()))

    warm_steps, warm_s = warm_up(step, warmup)

    # dominant stage: gate/up projections (the largest weight stream / flop count)
    dom = "ffn_up"
    K = steps
    ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for e in ev_s + ev_e:                      # materialise the HIP event handles
        e.record(stream)
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    timed = set(range(0, K, EVENT_EVERY))     # the dominant kernel's own events on every 16th step
    for i in range(K):
        if i in timed:
            ds4.set_stage_events(dom, ev_s[i], ev_e[i])
        elif i - 1 in timed:
            ds4.set_stage_events(dom)
        step(warmup + i)
    t_stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ds4.set_stage_events(dom)
    total_ms = t_start.elapsed_time(t_stop)
    ms_per_step = total_ms / K
    dom_ms = [ev_s[i].elapsed_time(ev_e[i]) for i in sorted(timed)]
    dom_avg_ms = float(np.mean(dom_ms))

    # per-stage breakdown (separate short instrumented pass)
    nb = min(K, 50)
    stage_ms = {}
    evs = {s: ([torch.cuda.Event(enable_timing=True) for _ in range(nb)],
               [torch.cuda.Event(enable_timing=True) for _ in range(nb)]) for s in STAGES}
    for s in STAGES:
        for e in evs[s][0] + evs[s][1]:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(nb):
        for s in STAGES:
            ds4.set_stage_events(s, evs[s][0][i], evs[s][1][i])
        step(i)
    torch.cuda.synchronize()
    # batch 1 (path 1): route/permute/combine run inside the FFN launches
    fused = ("route", "permute", "combine") if path == 1 else ()
    for s in STAGES:
        ds4.set_stage_events(s)
        if s in fused:
            stage_ms[s] = None
            continue
        stage_ms[s] = round(float(np.mean([evs[s][0][i].elapsed_time(evs[s][1][i]) for i in range(nb)])) * 1e3, 2)

    # algorithmic work per step (touched experts only)
    used = [n_active[(warmup + i) % n_pool] for i in range(K)]
    D = float(np.mean(used))
    up_bytes = D * (expert_bytes(spec, "gate") + expert_bytes(spec, "up")) + shared_bytes(spec)
    step_bytes = D * (expert_bytes(spec, "gate") + expert_bytes(spec, "up") + expert_bytes(spec, "down")) \
        + 3 * spec.shared_ffn * spec.hidden * 2
    up_flops = 2.0 * P * spec.hidden * 2 * spec.ffn + 2.0 * T * spec.hidden * 2 * spec.shared_ffn
    step_flops = 6.0 * P * spec.hidden * spec.ffn + 6.0 * T * spec.hidden * spec.shared_ffn
    memory_bound = T <= 64
    if memory_bound:
        kbytes = up_bytes
        if path == 1:
            kname, ksrc = "t1_up_kernel (route + gate/up + SwiGLU, routed + shared; batch 1)", "decode_t1.hip"
        elif path == 2:
            kname, ksrc = ("gg_kernel (grouped GEMM, small-batch layout: gate/up + SwiGLU, routed + shared)"
                           if T <= 32 else "gg_kernel (grouped GEMM: gate/up + SwiGLU, routed + shared)"), "ffn_grouped.hip"
        else:
            kname, ksrc = "gemv_kernel (gate/up + SwiGLU, routed + shared)", "ffn_gemv.hip"
        achieved = kbytes / (dom_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": kname, "kernel_source": ksrc,
                "algorithmic_bytes_per_launch": int(kbytes), "avg_launch_us": round(dom_avg_ms * 1e3, 2)}
        step_frac = step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS
    elif fp8:
        # routed E2M1 x E4M3 products at the fp8 rate, the bf16 shared expert at
        # the bf16 rate; the weight stream is the binding roof (both reported)
        routed_up = 2.0 * P * spec.hidden * 2 * spec.ffn
        mfma_s = routed_up / (FP8_PEAK_TFLOPS * 1e12) + (up_flops - routed_up) / (BF16_PEAK_TFLOPS * 1e12)
        hbm_s = up_bytes / (HBM_PEAK_GBS * 1e9)
        t = dom_avg_ms * 1e-3
        achieved = up_bytes / t / 1e9
        roof = {"bound": "hbm" if hbm_s >= mfma_s else "mfma", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "grouped GEMM, MXFP4 x MXFP8 scaled MFMA (gate/up + SwiGLU + MXFP8 h; bf16 shared)",
                "kernel_source": "ffn_grouped.hip", "algorithmic_bytes_per_launch": int(up_bytes),
                "avg_launch_us": round(dom_avg_ms * 1e3, 2),
                "mfma": {"achieved_tflops": round(up_flops / t / 1e12, 1),
                         "peak_tflops": round(up_flops / mfma_s / 1e12, 1),
                         "frac": round(mfma_s / t, 4), "note": "fp8 rate for routed, bf16 rate for shared"},
                "roof_us": {"hbm": round(hbm_s * 1e6, 1), "mfma": round(mfma_s * 1e6, 1)}}
        step_frac = step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS
    else:
        achieved = up_flops / (dom_avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "grouped GEMM (gate/up + SwiGLU, routed + shared)", "kernel_source": "ffn_grouped.hip",
                "algorithmic_flops_per_launch": up_flops, "avg_launch_us": round(dom_avg_ms * 1e3, 2)}
        step_frac = step_flops / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS

    out = {
        "metric": METRIC,
        "value": round(T / (ms_per_step * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "warmup_run": {"steps": warm_steps, "s": round(warm_s, 3)},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": name, "forward_path": path, "tokens": T, "hidden": spec.hidden, "expert_ffn": spec.ffn,
                   "experts": spec.n_experts, "top_k": spec.top_k, "shared_ffn": spec.shared_ffn,
                   "routed_format": spec.wfmt, "routing": "zipf(1.1)" if zipf else "uniform",
                   "algo": args.algo, "mma": mma, "layer_copies": copies, "logit_draws": n_pool},
        "roofline": roof,
        "step": {"active_experts_avg": D, "algorithmic_bytes": int(step_bytes), "algorithmic_flops": step_flops,
                 "frac_of_roofline": round(step_frac, 4), "stage_us": stage_ms, "wall_s": round(wall, 3)},
    }
    roof["traffic"] = measured_traffic(name + ("_fp8" if fp8 else ""), roof["kernel_source"])
    host_x, host_logits = x.cpu(), [lg.cpu() for lg in logits]
    out["_cpu"] = lambda: cpu_baseline(layers[0], host_x, host_logits, T, mx8=fp8)
    return out


ROUTER_METRIC = "router projection tokens/s (logits = W_r x, bf16 W_r 256 x 7168); % HBM/MFMA peak"


def router_main(args):
    """The router projection alone (ds4moe_router_logits): 256 experts x 7168
    hidden, bf16 router matrix, fp32 logits; one token (router_decode) or a
    4096-token chunk (router_prefill).  A step is one call; batch 1 rotates
    96 router copies (352 MB, beyond the caches) so the weights stream from
    HBM."""
    import numpy as np
    import torch
    import bit_routed_moe_amd as ds4
    from synth import make_x, make_router_w

    H, E = 7168, 256
    T = 1 if args.workload == "router_decode" else 4096
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copies = args.copies or (96 if T == 1 else 2)
    w0 = make_router_w(E, H, seed=args.seed).to(dev)
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    x = make_x(T, H, seed=args.seed).to(dev)
    out = torch.empty((T, E), dtype=torch.float32, device=dev)
    cfg = ds4.make_config(H, 2048, E, 8, 2048, "q2k", act="bf16")
    stream = torch.cuda.current_stream()

    def step(i):
        ds4.router_logits(cfg, T, x, ws[i % copies], out, stream)

    warm_steps, warm_s = warm_up(step, args.warmup)
    K = args.steps
    ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for e in ev_s + ev_e:
        e.record(stream)
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    timed = set(range(0, K, EVENT_EVERY))
    for i in range(K):
        if i in timed:
            ds4.set_stage_events("router_proj", ev_s[i], ev_e[i])
        elif i - 1 in timed:
            ds4.set_stage_events("router_proj")
        step(args.warmup + i)
    t_stop.record(stream)
    torch.cuda.synchronize()
    ds4.set_stage_events("router_proj")
    ms_per_step = t_start.elapsed_time(t_stop) / K
    dom_ms = float(np.mean([ev_s[i].elapsed_time(ev_e[i]) for i in sorted(timed)]))

    nbytes = E * H * 2 + T * H * 2 + T * E * 4
    flops = 2.0 * T * E * H
    if T == 1:
        achieved = nbytes / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "router_gemv_kernel (bf16 router rows x 1 token)", "kernel_source": "router_proj.hip",
                "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": round(dom_ms * 1e3, 2)}
    else:
        achieved = flops / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "router_mfma_kernel (64 tokens x 64 experts per workgroup)",
                "kernel_source": "router_proj.hip", "algorithmic_flops_per_launch": flops,
                "avg_launch_us": round(dom_ms * 1e3, 2)}
    res = {
        "metric": ROUTER_METRIC, "value": round(T / (ms_per_step * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "warmup_run": {"steps": warm_steps, "s": round(warm_s, 3)},
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "hidden": H, "experts": E, "router_copies": copies},
        "roofline": roof,
    }
    roof["traffic"] = measured_traffic(args.workload, roof["kernel_source"])
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_limits
        xh = x.double().cpu().numpy()
        wh = w0.double().cpu().numpy()
        n = 0
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 10.0:
                oracle.router_logits(xh, wh)
                n += 1
            dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(n * T / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"the whole {T}-token workload, {n} times: fp64 product with the "
                                         f"router matrix, single thread; {dt:.1f} s",
                               "host_cores_available": len(os.sched_getaffinity(0))}
    print(json.dumps(res), flush=True)


DEVICE_HEADERS = ("common.hpp", "formats.hpp", "vecdot.hpp")


def kernel_source_digest(tu):
    """sha256 over a kernel's translation unit and the device-code headers."""
    import hashlib
    d = os.path.join(ROOT, "bit_routed_moe_amd", "csrc")
    h = hashlib.sha256()
    for name in (tu,) + DEVICE_HEADERS:
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload, tu):
    """HBM bytes per launch of the dominant kernel from the committed counter
    runs (FETCH_SIZE and WRITE_SIZE, each scaled by the copy-kernel factor), or
    None when there is none for this workload or the kernel's sources changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != kernel_source_digest(tu):
        return None
    return int(rec["bytes_per_launch"])


def _host_view(layer, experts):
    """The layer's bytes for the given experts (and the shared expert) copied
    to the host before timing: the oracle reads host memory."""
    host = {(n, e): layer.routed(n, e) for e in experts for n in ("gate", "up", "down")}
    sh = {n: layer.shared(n) for n in ("sh_gate", "sh_up", "sh_down")} if layer.spec.shared_ffn else {}

    class HostView:
        spec = layer.spec

        def routed(self, n, e):
            return host[(n, e)]

        def shared(self, n):
            return sh[n]

    return HostView()


def cpu_baseline(layer, x, logits_pool, T, mx8=False):
    """The fp64 oracle as it stands, timed on this host's cores over a bounded
    sample of the workload, at all the cores this process may use (the
    sample's independent expert evaluations spread over threads) and on one
    core.  Decode-sized batches use the per-token order (the definition);
    the 4096-token chunk uses the expert-outer order on a sample of experts,
    scaled to the chunk."""
    import numpy as np
    n_cores = len(os.sched_getaffinity(0))
    if T > 64:
        many = _cpu_prefill(layer, x, logits_pool[0], n_cores, mx8)
        one = _cpu_prefill(layer, x, logits_pool[0], 1, mx8)
    else:
        many = _cpu_per_token(layer, x, logits_pool, T, n_cores, mx8)
        one = _cpu_per_token(layer, x, logits_pool, T, 1, mx8)
    many["one_core"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
    many["host_cores_available"] = n_cores
    return many


def _cpu_per_token(layer, x, logits_pool, T, threads, mx8, n_tok=10):
    """n_tok tokens, each routed, its k experts decoded from their bytes and
    evaluated pair by pair, the shared expert, combine (oracle.forward's
    steps).  At batch 1 the sample is the one token under n_tok router draws,
    else the batch's first n_tok tokens.  With several threads, the pairs of
    disjoint expert sets run concurrently (numpy releases the GIL in its
    array loops); BLAS is held to one thread per worker."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    import oracle
    k = layer.spec.top_k
    if T == 1:
        batches = [(x[:1], logits_pool[i][:1]) for i in range(n_tok)]
    else:
        batches = [(x[:n_tok], logits_pool[0][:n_tok])]
    batches = [(xb.float().numpy().astype(np.float64), lb.numpy()) for xb, lb in batches]
    routes = [oracle.route(lb, k) for _, lb in batches]
    view = _host_view(layer, sorted({int(e) for idx, _ in routes for e in np.unique(idx)}))
    tasks = [(b, {int(e)}) for b, (idx, _) in enumerate(routes) for e in np.unique(idx)]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        routes = [oracle.route(lb, k) for _, lb in batches]
        run = lambda task: (task[0], oracle.expert_outputs(view, batches[task[0]][0], routes[task[0]][0],
                                                           mx8=mx8, experts=task[1])[0])
        if threads == 1:
            parts = [run(t) for t in tasks]
        else:
            with ThreadPoolExecutor(threads) as ex:
                parts = list(ex.map(run, tasks))
        o = [dict() for _ in batches]
        for b, ob in parts:
            o[b].update(ob)
        for b, (xb, _) in enumerate(batches):
            s = oracle.shared_outputs(view, xb)
            idx, w = routes[b]
            for t in range(xb.shape[0]):
                oracle.combine(w[t], np.stack([o[b][(t, j)] for j in range(k)]), None if s is None else s[t])
        dt = time.perf_counter() - t0
    what = (f"the 1-token batch under {n_tok} router draws" if T == 1
            else f"the first {n_tok} tokens of the {T}-token batch")
    return {"value": round(n_tok / dt, 5), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}: route, decode of each token's {k} experts' gate/up/down bytes to fp64 and "
                      f"per-pair SwiGLU FFNs{' (MXFP8 x and h)' if mx8 else ''} ({len(tasks)} expert evaluations"
                      f"{f' over {threads} threads' if threads > 1 else ''}), the bf16 shared expert, combine; "
                      f"{dt:.1f} s"}


def _cpu_prefill(layer, x, logits, threads, mx8, n_tok_shared=512):
    """The expert-outer oracle (oracle.forward_expert_outer) on the chunk,
    timed on a sample: routing of all tokens, the pairs of max(8, threads)
    experts (each decoded once, its tokens through fp64 matrix products), and
    the shared expert on the first n_tok_shared tokens; scaled to all active
    experts and all tokens."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    import oracle
    T = x.shape[0]
    k = layer.spec.top_k
    xh = x.float().numpy().astype(np.float64)
    lh = logits.numpy()
    idx, _ = oracle.route(lh, k)
    active = np.unique(idx)
    n_s = max(8, threads)
    sample = [int(e) for e in active[:n_s]]
    view = _host_view(layer, sample)
    groups = [set(sample[i::threads]) for i in range(threads)]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        routing = oracle.route(lh, k)
        t_route = time.perf_counter() - t0
        t0 = time.perf_counter()
        part = lambda g: oracle.forward_expert_outer(view, xh, lh, mx8=mx8, experts=g, shared=False,
                                                     routing=routing)
        if threads == 1:
            [part(g) for g in groups]
        else:
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(part, groups))
        t_exp = time.perf_counter() - t0
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        oracle.forward_expert_outer(view, xh[:n_tok_shared], lh[:n_tok_shared], mx8=mx8, experts=set())
        t_sh = time.perf_counter() - t0
    est = t_route + t_exp * len(active) / len(sample) + t_sh * T / n_tok_shared
    return {"value": round(T / est, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"expert-outer oracle on the {T}-token chunk: routing of every token ({t_route:.1f} s), "
                      f"the pairs of {len(sample)} of the {len(active)} active experts (decode to fp64, "
                      f"fp64 matrix products{', MXFP8 x and h' if mx8 else ''}; {t_exp:.1f} s"
                      f"{f' over {threads} threads' if threads > 1 else ''}), the shared expert on "
                      f"{n_tok_shared} tokens ({t_sh:.1f} s); scaled to the whole chunk: {est:.0f} s"}


if __name__ == "__main__":
    main()
