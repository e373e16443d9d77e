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
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the step-time distribution, cold-cache steps and amd-smi sampling "
                         "(for runs under a profiler)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU work of the oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 1 GiB device copy (reference for byte counters)")
    return ap.parse_args()


def gemm_traffic(workload, fp8=False):
    """HBM-side bytes (fetched + written) of one moe_expert_ffn call (both
    grouped-GEMM launches), from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of this workload, scaled by its copy calibration.
    None when there is no summary or the GEMM source changed since."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"moe_forward_{workload}{'_fp8' if fp8 else ''}_traffic.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    blob = json.loads(m.group(1))
    src = os.path.join(ROOT, "sparse_mixture_experts_gemm_amd", "csrc", "expert_gemm.hip")
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != blob.get("expert_gemm_hip_sha256"):
        return None
    ks = [v for k, v in blob["kernels"].items() if k.startswith("grouped_gemm")]
    if not ks:
        return None
    return sum(v["fetch_bytes"] + v["write_bytes"] for v in ks)


def stage_bytes_flops(cfg, rows, active_experts, splits=1, fp8=False):
    """Algorithmic work per stage (what the method must touch).  fp8: expert
    weights of one byte plus an fp32 scale per weight row."""
    T, d, E, dff = cfg.T, cfg.d, cfg.E, cfg.d_ff
    es = 2 if cfg.dtype == "bf16" else 4
    k1 = cfg.k + 1
    route_bytes = T * d * es + E * d * es + T * E * 4 + T * k1 * 8
    # dispatch: candidates in, routing arrays out, x rows read once, x_perm written
    dispatch_bytes = T * k1 * 8 + T * cfg.k * 17 + T * d * es + rows * d * es
    gemm_flops = rows * 6.0 * d * dff
    gemm_weight_bytes = active_experts * (3 * d * dff + (2 * dff + d) * 4 if fp8 else 3 * d * dff * es)
    combine_bytes = rows * d * 4 * splits + T * d * es + T * cfg.k * 8
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
    if args.fp8_weights:
        if not (p.dtype == moe.MOE_BF16 and moe.capacity(p) <= 32 and d % 128 == 0 and cfg.d_ff % 128 == 0):
            print(f"bench.py: --fp8-weights needs a bf16 layer with capacity <= 32 and d, d_ff multiples of 128; "
                  f"{cfg.name} has capacity {moe.capacity(p)}", file=sys.stderr)
            sys.exit(2)
        fp8 = {}
        for n in ("w1", "w3", "w2"):
            fp8["q" + n[1]], fp8["s" + n[1]] = moe_synth.quantize_rows_e4m3(L[n])
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

    def step():
        if fp8:
            moe.forward_fp8(p, L["x"], L["w_router"], L["bias"], load, fp8["q1"], fp8["s1"], fp8["q3"], fp8["s3"],
                            fp8["q2"], fp8["s2"], y, logits, r, ws)
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

    # distribution of single-step times (events around each step, no sync in
    # between), then cold-cache steps: a 1 GiB fill before each one evicts
    # x, the weights and the workspace from L2 and the 256 MiB last-level cache
    step_ms = cold_ms = gpu_state = None
    if not args.no_extras:
        step_ms = step_times(step, max(20, args.steps), torch)
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cold_ms = step_times(step, 10, torch, before=lambda i: scratch.fill_(float(i)))
        del scratch
        gpu_state = smi_under_load(step, torch)

    totals = r.totals.cpu().tolist()
    kept = r.kept.cpu()
    rows = int(totals[0])
    active = int((kept > 0).sum())

    # per-stage times: each entry point bracketed by events on the launch stream
    x_perm = torch.empty((max(R, 1), d), dtype=dt, device=dev)
    h = torch.empty((max(R, 1), cfg.d_ff), dtype=torch.float16 if dt == torch.bfloat16 else dt, device=dev)
    y_perm = moe.alloc_y_perm(p, dev)
    wsd = moe.alloc_workspace(p, dev, dispatch_only=True)
    n_st = max(5, min(args.steps, 30))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_st)]
    for i in range(n_st + 3):
        e = ev[i - 3] if i >= 3 else None
        if e: e[0].record()
        moe.route(p, L["x"], L["w_router"], L["bias"], load, logits, r)
        if e: e[1].record()
        moe.dispatch(p, L["x"], r, x_perm, wsd)
        if e: e[2].record()
        if fp8:
            moe.expert_ffn_fp8(p, x_perm, r.offsets, fp8["q1"], fp8["s1"], fp8["q3"], fp8["s3"], fp8["q2"],
                               fp8["s2"], h, y_perm)
        else:
            moe.expert_ffn(p, x_perm, r.offsets, L["w1"], L["w3"], L["w2"], h, y_perm)
        if e: e[3].record()
        moe.combine(p, y_perm, r.row, r.gate, y)
        if e: e[4].record()
    torch.cuda.synchronize()
    st = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in ev])  # ms
    st_ms = st.mean(axis=0)
    work = stage_bytes_flops(cfg, rows, active, moe.ffn_splits(p), fp8=bool(fp8))
    t_route, t_disp, t_ffn, t_comb = (float(v) for v in st_ms)
    gemm_tflops = work["gemm_flops"] / (t_ffn * 1e-3) / 1e12
    stages = {
        "route": {"us": t_route * 1e3, "GB/s": work["route_bytes"] / (t_route * 1e-3) / 1e9,
                  "hbm_frac": work["route_bytes"] / (t_route * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "dispatch": {"us": t_disp * 1e3, "GB/s": work["dispatch_bytes"] / (t_disp * 1e-3) / 1e9,
                     "hbm_frac": work["dispatch_bytes"] / (t_disp * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "expert_ffn": {"us": t_ffn * 1e3, "TFLOP/s": gemm_tflops, "mfma_frac": gemm_tflops / PEAK_MFMA_TFLOPS,
                       "weight_GB/s": work["gemm_weight_bytes"] / (t_ffn * 1e-3) / 1e9},
        "combine": {"us": t_comb * 1e3, "GB/s": work["combine_bytes"] / (t_comb * 1e-3) / 1e9,
                    "hbm_frac": work["combine_bytes"] / (t_comb * 1e-3) / 1e9 / PEAK_HBM_GBS},
    }
    layer_flops = work["route_flops"] + work["gemm_flops"]

    roofline = {"kernel": "expert grouped GEMM (moe_expert_ffn: gate-up + down launches)",
                "bound": "mfma", "achieved": gemm_tflops, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": gemm_tflops / PEAK_MFMA_TFLOPS, "traffic": None}
    if args.workload == "decode":
        gbs = work["gemm_weight_bytes"] / (t_ffn * 1e-3) / 1e9
        roofline = {"kernel": "expert grouped GEMM (weight streaming" + (", E4M3 weights)" if fp8 else ")"),
                    "bound": "hbm", "achieved": gbs,
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "traffic": None}

    roofline["traffic"] = gemm_traffic(args.workload, fp8=bool(fp8))

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
                   "expert_weights": "fp8 e4m3 codes + fp32 row scales" if fp8 else cfg.dtype},
        "layer_tflops": layer_flops / (ms_per_step * 1e-3) / 1e12,
        "mfma_util_pct": 100.0 * gemm_tflops / PEAK_MFMA_TFLOPS,
        "stages": stages,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "wall_s_timed": wall,
        "step_ms": step_ms,
        "cold_step_ms": cold_ms,
        "gpu_state": gpu_state,
    }
    print(json.dumps(out))


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
        for j in ("1", "3", "2"):
            c["w" + j] = oracle.dequant_rows(fp8["q" + j].cpu().numpy(), fp8["s" + j].cpu().numpy())
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
    return {"value": 1.0 / per_token_s, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model,
            "sample": f"router logits + ranking + dispatch for all {T} tokens ({t_route:.2f} s), "
                      f"expert FFN + combine for {n2} tokens ({t_ffn:.2f} s); rate per token"}


if __name__ == "__main__":
    main()
