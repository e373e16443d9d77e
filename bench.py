"""Benchmark: sparse MoE FFN layer forward (moe_forward) on one MI355X.

One step = one moe_forward over one batch of seeded synthetic tokens (route,
dispatch, expert SwiGLU grouped GEMM, combine), inputs and weights resident in
HBM.  Prints one JSON line with tokens/s, the expert GEMM's roofline figures
and the CPU oracle timed on a bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec + expert-GEMM MFMA util %, Mixtral-shape E=8 top-2 bf16"
PEAK_MFMA_TFLOPS = 2516.6   # bf16 / fp16 dense matrix peak, MI355X
PEAK_HBM_GBS = 8000.0       # HBM3E
PEAK_F32_TFLOPS = 157.3     # fp32 vector ALU peak (the fp32 layer's GEMM runs on the VALU)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral",
                    choices=["tiny", "mixtral", "fine64", "skew", "decode"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fp8-weights", action="store_true",
                    help="expert weights as E4M3 codes with fp32 row scales (weight-streaming layers: "
                         "capacity <= 32 rows per expert)")
    ap.add_argument("--int8-weights", action="store_true",
                    help="expert weights as INT8 codes with fp32 row scales (weight-streaming layers: "
                         "capacity <= 32 rows per expert)")
    ap.add_argument("--int4-weights", action="store_true",
                    help="expert weights as INT4 codes, two per byte, with fp32 row scales (weight-streaming "
                         "layers only: capacity <= 32 rows per expert)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the step-time distribution, cold-cache steps and amd-smi sampling "
                         "(for runs under a profiler)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU work of the oracle sample")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the timing of moe_backward (the training pass) after the forward pass")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 1 GiB device copy (reference for byte counters)")
    return ap.parse_args()


CSRC = os.path.join(ROOT, "sparse_mixture_experts_gemm_amd", "csrc")
# the source file of each stage's kernels: a committed counter summary is used
# for a stage only while that file still has the hash recorded with it
STAGE_SOURCE = {"route": ("route.hip",), "dispatch": ("dispatch.hip",),
                "expert_ffn": ("expert_gemm.hip", "grouped_tiles.h"), "combine": ("combine.hip",)}
# the kernels moe_forward launches per stage (moe_dispatch's gather is not one)
STAGE_KERNELS = {"route": ("route_",), "dispatch": ("dispatch_hist", "dispatch_primary", "dispatch_finalize",
                                                    "dispatch_single"),
                 "expert_ffn": ("grouped_gemm",), "combine": ("combine_", "zero_fill")}


def counter_traffic(workload, qfmt=None):
    """HBM-side bytes (fetched + written) per forward pass of each stage's
    kernels, from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary of
    this workload, scaled by its copy calibration.  A stage is left out when
    its kernel source changed since the counters were taken."""
    import hashlib
    import re
    suffix = {None: "", "e4m3": "_fp8", "int8": "_int8", "int4": "_int4"}[qfmt]
    path = os.path.join(ROOT, "profiles", f"moe_forward_{workload}{suffix}_traffic.md")
    if not os.path.exists(path):
        return {}
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return {}
    blob = json.loads(m.group(1))
    out = {}
    for stage, srcs in STAGE_SOURCE.items():
        if any(blob.get("sources", {}).get(src) != hashlib.sha256(open(os.path.join(CSRC, src), "rb").read()).hexdigest()
               for src in srcs):
            continue
        ks = [v for k, v in blob["kernels"].items() if k.startswith(STAGE_KERNELS[stage])]
        if ks:
            out[stage] = sum(v["fetch_bytes"] + v["write_bytes"] for v in ks)
    return out


def stage_work(cfg, rows, active_experts, fp8=False, code_bits=8):
    """Algorithmic work per stage of one forward pass: what the method must
    touch (kept rows, active experts, one read of x, one write of y), not
    what this implementation moves.  fp8: expert weights as codes of
    code_bits bits (8 or 4) plus an fp32 scale per weight row."""
    T, d, E, dff, k = cfg.T, cfg.d, cfg.E, cfg.d_ff, cfg.k
    es = 2 if cfg.dtype == "bf16" else 4
    k1 = k + 1
    # route: x and the router weights read, logits and ranked candidates written
    route_bytes = T * d * es + E * d * es + T * E * 4 + T * k1 * 8
    # dispatch: candidates read, the slot arrays (eid, pos, row, flag, gate) and
    # token_of_row written (moe_forward gathers x inside the GEMM, so no copy)
    dispatch_bytes = T * k1 * 8 + T * k * 17 + rows * 4
    gemm_flops = rows * 6.0 * d * dff
    gemm_weight_bytes = active_experts * (3 * d * dff * code_bits // 8 + (2 * dff + d) * 4 if fp8
                                          else 3 * d * dff * es)
    # combine: each kept row's expert output (layer dtype) read once, y written,
    # the slot arrays read
    combine_bytes = rows * d * es + T * d * es + T * k * 8
    return dict(route_bytes=route_bytes, dispatch_bytes=dispatch_bytes, gemm_flops=gemm_flops,
                gemm_weight_bytes=gemm_weight_bytes, combine_bytes=combine_bytes,
                route_flops=2.0 * T * d * E)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the MoE layer runs on one GPU here (all experts resident in its HBM); "
              "multi-GPU runs are not implemented. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_synth
    import sparse_mixture_experts_gemm_amd as moe

    dev = "cuda:0"
    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
    cfg = moe_synth.CONFIGS[args.workload]
    print(f"[bench] workload {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    L = moe_synth.make_layer(cfg, dev)
    p = moe.Params(T=cfg.T, d=cfg.d, E=cfg.E, k=cfg.k, d_ff=cfg.d_ff, capacity_factor=cfg.cf,
                   reroute=cfg.reroute, lam=cfg.lam, aux_coef=cfg.aux_coef,
                   dtype=moe.MOE_BF16 if cfg.dtype == "bf16" else moe.MOE_F32, gate_temperature=cfg.tau,
                   top2_gap=cfg.gap)
    dt = p.torch_dtype
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    fp8 = None
    qfmt = "int4" if args.int4_weights else "int8" if args.int8_weights else "e4m3" if args.fp8_weights else None
    if qfmt:
        small = moe.capacity(p) <= 32
        if not (p.dtype == moe.MOE_BF16 and (not small or (d % 128 == 0 and cfg.d_ff % 128 == 0))):
            print(f"bench.py: quantised weights need a bf16 layer (with d, d_ff multiples of 128 when every expert "
                  f"holds at most 32 rows); {cfg.name} is {cfg.dtype}", file=sys.stderr)
            sys.exit(2)
        if qfmt == "int4" and not (small and d % 128 == 0 and cfg.d_ff % 128 == 0):
            print(f"bench.py: INT4 weights run on the weight-streaming kernel only (at most 32 rows per expert, "
                  f"d and d_ff multiples of 128); {cfg.name} has capacity {moe.capacity(p)}", file=sys.stderr)
            sys.exit(2)
        fp8 = {"fmt": qfmt}
        quant = {"int4": moe_synth.quantize_rows_int4, "int8": moe_synth.quantize_rows_int8,
                 "e4m3": moe_synth.quantize_rows_e4m3}[qfmt]
        for n in ("w1", "w3", "w2"):
            fp8["q" + n[1]], fp8["s" + n[1]] = quant(L[n])
            L[n] = None
        torch.cuda.empty_cache()
    R = moe.max_rows(p)

    load = None
    if cfg.load_from_prev:
        # previous batch's per-expert kept fraction, routed without a penalty on the GPU path
        pp = moe.Params(**{**p.__dict__, "lam": 0.0})
        rp = moe.Routing(pp, dev)
        lg = torch.empty((T, E), dtype=torch.float32, device=dev)
        moe.route(pp, L["x_prev"], L["w_router"], L["bias"], None, lg, rp)
        xp = torch.empty((R, d), dtype=dt, device=dev)
        moe.dispatch(pp, L["x_prev"], rp, xp, moe.alloc_workspace(pp, dev, dispatch_only=True))
        load = rp.kept.float() / float(T * k)
        del xp

    y = torch.empty((T, d), dtype=dt, device=dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    r = moe.Routing(p, dev)
    ws = moe.alloc_workspace(p, dev)

    def step(events=None):
        if fp8:
            {"int4": moe.forward_i4, "int8": moe.forward_i8, "e4m3": moe.forward_fp8}[fp8["fmt"]](
                p, L["x"], L["w_router"], L["bias"], load, fp8["q1"], fp8["s1"], fp8["q3"], fp8["s3"], fp8["q2"],
                fp8["s2"], y, logits, r, ws)
        elif events is not None:
            moe.forward_events(p, L["x"], L["w_router"], L["bias"], load, L["w1"], L["w3"], L["w2"], y, logits, r,
                               ws, events)
        else:
            moe.forward(p, L["x"], L["w_router"], L["bias"], load, L["w1"], L["w3"], L["w2"], y, logits, r, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # per-stage times of the forward pass itself: moe_forward_events enqueues
    # the same launches as moe_forward with six events between its stages (on
    # the launch stream); averaged over as many steps as were timed
    stage_names = ("route", "dispatch", "gate_up", "down", "combine")
    st_ms = None
    if not fp8:
        n_ev = args.steps
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(n_ev)]
        torch.cuda.synchronize()
        for e in evs:
            step(e)
        torch.cuda.synchronize()
        st = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(5)] for e in evs])  # ms
        st_ms = dict(zip(stage_names, (float(v) for v in st.mean(axis=0))))
        st_ms["events_step"] = float(np.mean([e[0].elapsed_time(e[5]) for e in evs]))

    # distribution of single-step times (events around each step, no sync in
    # between), then cold-cache steps: a 1 GiB fill before each one evicts
    # x, the weights and the workspace from L2 and the 256 MiB last-level cache
    step_ms = cold_ms = gpu_state = graph_ms = None
    if not args.no_extras:
        step_ms = step_times(step, max(20, args.steps), torch)
        graph_ms = graph_step_ms(step, args.steps, torch)
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cold_ms = step_times(step, 10, torch, before=lambda i: scratch.fill_(float(i)))
        del scratch
        gpu_state = smi_under_load(step, torch)

    totals = r.totals.cpu().tolist()
    kept = r.kept.cpu()
    rows = int(totals[0])
    active = int((kept > 0).sum())
    work = stage_work(cfg, rows, active, fp8=bool(fp8), code_bits=4 if fp8 and fp8["fmt"] == "int4" else 8)
    traffic = counter_traffic(args.workload, qfmt=fp8["fmt"] if fp8 else None)
    layer_flops = work["route_flops"] + work["gemm_flops"]

    def hbm(nbytes, ms, stage):
        gbs = nbytes / (ms * 1e-3) / 1e9
        out = {"us": ms * 1e3, "algorithmic_bytes": nbytes, "GB/s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}
        if stage in traffic:
            out["traffic_bytes"] = traffic[stage]
            out["traffic_over_algorithmic"] = traffic[stage] / nbytes
        return out

    stages = None
    if st_ms is not None:
        t_ffn = st_ms["gate_up"] + st_ms["down"]
        gemm_tflops = work["gemm_flops"] / (t_ffn * 1e-3) / 1e12
        stages = {
            "route": hbm(work["route_bytes"], st_ms["route"], "route"),
            "dispatch": hbm(work["dispatch_bytes"], st_ms["dispatch"], "dispatch"),
            "expert_ffn": {"us": t_ffn * 1e3, "gate_up_us": st_ms["gate_up"] * 1e3, "down_us": st_ms["down"] * 1e3,
                           "TFLOP/s": gemm_tflops, "mfma_frac": gemm_tflops / PEAK_MFMA_TFLOPS
                           if cfg.dtype == "bf16" else None,
                           "gate_up_TFLOP/s": work["gemm_flops"] * 2 / 3 / (st_ms["gate_up"] * 1e-3) / 1e12,
                           "down_TFLOP/s": work["gemm_flops"] / 3 / (st_ms["down"] * 1e-3) / 1e12,
                           "weight_bytes": work["gemm_weight_bytes"],
                           "weight_GB/s": work["gemm_weight_bytes"] / (t_ffn * 1e-3) / 1e9},
            "combine": hbm(work["combine_bytes"], st_ms["combine"], "combine"),
            "sum_of_stages_ms": sum(st_ms[n] for n in stage_names),
            "events_step_ms": st_ms["events_step"],
            "source": "moe_forward_events: HIP events between the forward's own launches on its stream, "
                      f"mean of {args.steps} steps",
        }
        if "expert_ffn" in traffic:
            stages["expert_ffn"]["traffic_bytes"] = traffic["expert_ffn"]
            stages["expert_ffn"]["traffic_over_weight_bytes"] = traffic["expert_ffn"] / work["gemm_weight_bytes"]
        achieved_ms = t_ffn
    else:
        achieved_ms = None

    if args.workload == "decode" or (fp8 and moe.capacity(p) <= 32):
        # weight streaming: the expert weights' bytes against HBM bandwidth.  With
        # one-byte weights there is no events variant; the whole step bounds it.
        t = achieved_ms if achieved_ms is not None else ms_per_step
        gbs = work["gemm_weight_bytes"] / (t * 1e-3) / 1e9
        roofline = {"kernel": "expert grouped GEMM, gate-up + down launches (weight streaming"
                              + (f", {fp8['fmt']} weights; timed over the whole step)" if fp8 else ")"),
                    "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                    "traffic": traffic.get("expert_ffn"),
                    "per_launch_work": f"{work['gemm_weight_bytes']} weight bytes ({active} active experts x 3 x d x d_ff)"}
    else:
        # one-byte weights on the matrix-core tile: no events variant, so the
        # whole step bounds the GEMM's time (an underestimate of its rate)
        t = achieved_ms if achieved_ms is not None else ms_per_step
        tf = work["gemm_flops"] / (t * 1e-3) / 1e12
        # bf16 layers multiply on the matrix cores; the fp32 layer's GEMM is a
        # vector-ALU kernel, priced against the fp32 vector peak
        bound, peak = ("mfma", PEAK_MFMA_TFLOPS) if cfg.dtype == "bf16" else ("alu", PEAK_F32_TFLOPS)
        roofline = {"kernel": "expert grouped GEMM, gate-up + down launches of moe_forward"
                              + (f" ({fp8['fmt']} weights; timed over the whole step)" if fp8 else ""),
                    "bound": bound, "achieved": tf, "peak": peak, "unit": "TFLOP/s",
                    "frac": tf / peak, "traffic": traffic.get("expert_ffn"),
                    "per_launch_work": f"{work['gemm_flops']:.4g} flop ({rows} kept rows x 6 x d x d_ff)"}

    backward = None
    if not args.no_backward and not fp8 and p.dtype == moe.MOE_BF16:
        backward = bench_backward(moe, moe_synth, torch, np, p, cfg, L, r, rows, dev, max(5, args.steps // 2))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, L, load, args.cpu_seconds, fp8)

    out = {
        "metric": METRIC, "value": T / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded SplitMix64/Box-Muller inputs and random-init weights of the workload's shape)",
        "config": {"workload": f"{cfg.name}: T={T} d={d} E={E} top-{k} d_ff={cfg.d_ff} cf={cfg.cf}"
                               + (f" bias={cfg.bias} lambda={cfg.lam}" if cfg.bias != "none" else ""),
                   "T": T, "d": d, "E": E, "k": k, "d_ff": cfg.d_ff, "capacity_factor": cfg.cf,
                   "rows": rows, "dropped": int(totals[1]), "rerouted": int(totals[2]),
                   "parallelism": "single GPU, all experts resident",
                   "expert_weights": f"{fp8['fmt']} codes + fp32 row scales" if fp8 else cfg.dtype},
        "layer_tflops": layer_flops / (ms_per_step * 1e-3) / 1e12,
        "mfma_util_pct": (100.0 * roofline["frac"]) if roofline["bound"] == "mfma" else None,
        "stages": stages,
        "roofline": roofline,
        "backward": backward,
        "cpu_baseline": cpu,
        "wall_s_timed": wall,
        "step_ms": step_ms,
        "graph_ms_per_step": graph_ms,
        "cold_step_ms": cold_ms,
        "gpu_state": gpu_state,
    }
    print(json.dumps(out))


def bench_backward(moe, moe_synth, torch, np, p, cfg, L, r, rows, dev, n):
    """moe_backward on the forward's routing with a seeded upstream gradient:
    mean time of n steps (events on the launch stream, after 2 warm-up steps).
    Algorithmic work: the three expert gradients (u = W2^T dy, dx_perm, dW1,
    dW3, dW2: 12 rows d d_ff flop); the recomputed gate-up products (4 rows
    d d_ff) are reported apart."""
    dy = moe_synth.upstream_grad(cfg, dev)
    gr = moe.Grads(p, dev)
    wsb = moe.alloc_backward_workspace(p, dev)

    def bstep():
        moe.backward(p, L["x"], L["w_router"], L["w1"], L["w3"], L["w2"], r, dy, gr, wsb)

    for _ in range(2):
        bstep()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        bstep()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n
    flops = 12.0 * rows * cfg.d * cfg.d_ff
    tf = flops / (ms * 1e-3) / 1e12
    out = {"ms_per_step": ms, "steps": n, "algorithmic_flop": flops, "TFLOP/s": tf, "mfma_frac": tf / PEAK_MFMA_TFLOPS,
           "recompute_flop": 4.0 * rows * cfg.d * cfg.d_ff,
           "tokens_per_s": cfg.T / (ms * 1e-3),
           "note": "moe_backward: fp32 gradients of x, router logits, W_r, bias, W1, W3, W2; routing held fixed"}
    del gr, wsb
    torch.cuda.empty_cache()
    return out


def graph_step_ms(step, n, torch):
    """The forward pass captured once in a HIP graph (torch.cuda.graph) and
    replayed n times on the current stream: mean ms per replay (the eager
    step's launch gaps removed), or None if the capture fails."""
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
        torch.cuda.synchronize()
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n
    except Exception as e:  # the eager measurement stands on its own
        print(f"[bench] graph capture failed: {e}", file=sys.stderr, flush=True)
        return None


def step_times(step, n, torch, before=None):
    """Median, p10 and p90 (ms) of n single steps, each bracketed by events
    on the launch stream; `before(i)` runs outside the bracket."""
    import numpy as np
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        if before is not None:
            before(i)
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"median": float(np.median(t)), "p10": float(np.percentile(t, 10)),
            "p90": float(np.percentile(t, 90)), "n": n}


def smi_under_load(step, torch, ramp_s=2.0, cap_s=30.0):
    """Socket power and per-XCD shader clocks from `amd-smi metric` under
    sustained load: steps run back to back for ramp_s first (power and clock
    settle within about a second; a sample taken at once reads the idle
    state), then the tool runs in a child process while the steps go on until
    it has exited.  None if unavailable or slower than cap_s."""
    import subprocess
    pending = []  # keep three batches queued so that the GPU never idles between them

    def batch():
        for _ in range(20):
            step()
        ev = torch.cuda.Event()
        ev.record()
        pending.append(ev)
        if len(pending) > 3:
            pending.pop(0).synchronize()

    t_ramp = time.perf_counter() + ramp_s
    while time.perf_counter() < t_ramp:
        batch()
    try:
        proc = subprocess.Popen(["amd-smi", "metric", "--clock", "--power", "--json"],
                                stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    except OSError:
        torch.cuda.synchronize()
        return None
    t_end = time.perf_counter() + cap_s
    while proc.poll() is None and time.perf_counter() < t_end:
        batch()
    torch.cuda.synchronize()
    if proc.poll() is None:
        proc.kill()
        proc.communicate()
        return None
    try:
        out, _ = proc.communicate()
        g = json.loads(out)["gpu_data"][0]
        clk = g["clock"]
        xcd = [clk[k]["clk"]["value"] for k in sorted(clk) if k.startswith("gfx_")]
        return {"socket_power_w": g["power"]["socket_power"]["value"], "gfx_clk_mhz": xcd,
                "source": f"amd-smi metric --clock --power, sampled after {ramp_s:.0f} s of back-to-back steps"}
    except Exception:
        return None


def cpu_baseline(cfg, L, load, target_s, fp8=None):
    """The oracle as it stands, on the host cores, on a bounded sample: router
    logits, ranking and dispatch for every token (the capacity couples them),
    expert FFN + combine for a sample of tokens; reported per token.  fp8: the
    expert FFN runs on the oracle's dequantised weights (double)."""
    import numpy as np
    import oracle

    oracle.lib()
    print("[bench] cpu baseline: copying inputs to host", file=sys.stderr, flush=True)
    c = {n: (oracle._np(v) if v is not None else None) for n, v in L.items()}
    xe = c["x"]
    if fp8:
        deq = {"int4": oracle.dequant_rows_i4, "int8": oracle.dequant_rows_i8,
               "e4m3": oracle.dequant_rows}[fp8["fmt"]]
        for j in ("1", "3", "2"):
            c["w" + j] = deq(fp8["q" + j].cpu().numpy(), fp8["s" + j].cpu().numpy())
        xe = L["x"].float().cpu().numpy().astype(np.float64)
    ld = None if load is None else load.cpu().numpy().astype(np.float32)
    T = cfg.T
    t0 = time.perf_counter()
    raw = oracle.router_logits(c["x"], c["w_router"], c["bias"])
    cand, cs = oracle.route(raw, cfg.k, ld, cfg.lam, cfg.gap)
    disp = oracle.dispatch(cand, cs, cfg.E, cfg.k, oracle.capacity(T, cfg.k, cfg.E, cfg.cf), cfg.reroute,
                           cfg.aux_coef, cfg.tau if cfg.tau > 0 else 1.0)
    t_route = time.perf_counter() - t0
    # calibrate on one token per oracle thread, then size the sample for about
    # target_s seconds of expert work
    n = max(2, oracle.num_threads())
    t1 = time.perf_counter()
    oracle.layer_tokens(np.arange(n, dtype=np.int32), xe, c["w1"], c["w3"], c["w2"], disp["eid"], disp["gate64"])
    per_tok = (time.perf_counter() - t1) / n
    n2 = int(max(2, min(T - n, target_s / max(per_tok, 1e-6))))
    toks = np.arange(n, n + n2, dtype=np.int32)
    t2 = time.perf_counter()
    oracle.layer_tokens(toks, xe, c["w1"], c["w3"], c["w2"], disp["eid"], disp["gate64"])
    t_ffn = time.perf_counter() - t2
    per_token_s = t_ffn / n2 + t_route / T
    cpu_model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    # the tiny fp32 layer in full on one thread: route, dispatch, expert FFN
    # and combine for all of its tokens
    tiny = tiny_single_thread(oracle)
    return {"value": 1.0 / per_token_s, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model,
            "sample": f"router logits + ranking + dispatch for all {T} tokens ({t_route:.2f} s), "
                      f"expert FFN + combine for {n2} tokens ({t_ffn:.2f} s); rate per token",
            "tiny_layer_single_thread": tiny}


def tiny_single_thread(oracle, reps=20):
    """The oracle's whole forward pass of the tiny fp32 layer (T 64, d 128,
    E 8, top-2, d_ff 256, capacity factor 1.0) on one thread, best of reps."""
    import moe_synth
    cfg = moe_synth.CONFIGS["tiny"]
    L = moe_synth.make_layer(cfg, "cpu")
    c = {n: (oracle._np(v) if v is not None else None) for n, v in L.items()}
    n0 = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        best = float("inf")
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.forward(c["x"], c["w_router"], c["bias"], c["w1"], c["w3"], c["w2"], E=cfg.E, k=cfg.k, cf=cfg.cf)
            best = min(best, time.perf_counter() - t0)
    finally:
        oracle.set_num_threads(n0)
    return {"value": cfg.T / best, "unit": "tokens/s", "cores": 1, "ms_per_layer": best * 1e3,
            "sample": f"tiny fp32 layer T={cfg.T} d={cfg.d} E={cfg.E} top-{cfg.k} d_ff={cfg.d_ff}, whole forward, "
                      f"best of {reps}"}


if __name__ == "__main__":
    main()
