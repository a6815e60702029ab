#!/usr/bin/env python3
"""Benchmark of the MoE layer's hot path on one MI355X.

One step = one pass of the layer over one batch of synthetic tokens already
resident in HBM: moe_route -> moe_dispatch -> moe_expert_ffn_gate_up ->
moe_expert_ffn_down -> moe_combine (all libmoe HIP kernels). The default workload
is the T=4096, d=2048, E=64, k=6, F=1408 bf16 layer forward.

Prints ONE JSON line: tokens/s for the whole job, per-stage times with achieved
GB/s or TFLOP/s against MI355X peaks, the roofline of the dominant kernel (timed
live with HIP events on the stream the kernels run on), and the CPU oracle timed
on the host cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s fwd(+bwd) on 1 MI355X; dispatch/combine GB/s; GEMM MFMA %"
PEAK_HBM_GBS = 8000.0          # HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP32_VALU_TFLOPS = 78.6   # fp32 FMA without packed-FP32 ops: 256 CU * 4 SIMD * 16 lanes * 2 * 2.4 GHz


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mid_bf16",
                    choices=["mid_bf16", "large_bf16", "tiny_f32"])
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (for profiler runs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    return ap.parse_args()


def stage_work(wl):
    """Algorithmic bytes and flops per launch of every stage."""
    b = 2 if wl.dtype == "bf16" else 4
    T, d, E, k, F = wl.T, wl.d, wl.E, wl.k, wl.F
    P = T * k
    return {
        # x and the router weights read once; indices and gates written
        "route": dict(bytes=T * d * b + E * d * b + P * 8, flops=2 * T * d * E, unit="valu"),
        # each token read once and written k times (the plan's int traffic is < 1 %)
        "dispatch": dict(bytes=T * d * b + P * d * b, flops=0, unit="hbm"),
        # every expert weight read once, dispatched rows read, a = silu(h)*u written
        "gate_up": dict(bytes=E * 2 * F * d * b + P * d * b + P * F * b,
                        flops=2 * P * d * 2 * F, unit="mfma"),
        "down": dict(bytes=E * d * F * b + P * F * b + P * d * b, flops=2 * P * F * d, unit="mfma"),
        # k rows gathered per token, one row written, slots and gates read
        "combine": dict(bytes=P * d * b + T * d * b + P * 8, flops=0, unit="hbm"),
    }


def bound_of(work):
    """hbm or mfma/valu: whichever lower bound on the time is larger."""
    t_mem = work["bytes"] / (PEAK_HBM_GBS * 1e9)
    if work["flops"] == 0:
        return "hbm", t_mem
    peak = PEAK_BF16_TFLOPS if work["unit"] == "mfma" else PEAK_FP32_VALU_TFLOPS
    t_cmp = work["flops"] / (peak * 1e12)
    return (work["unit"] if t_cmp >= t_mem else "hbm"), max(t_cmp, t_mem)


def cpu_baseline(wl, inp, target_s):
    """The oracle as it is, on the host cores, over whole passes of the workload."""
    import threadpoolctl
    import oracle
    host = {n: t.cpu() for n, t in inp.items()}
    n, total = 0, 0.0
    while n < 3 and (total < target_s or n == 0):
        t0 = time.perf_counter()
        oracle.forward(host["x"], host["w_router"], host["w13"], host["w2"], wl.k)
        total += time.perf_counter() - t0
        n += 1
    threads = [oracle.num_threads()]
    threads += [p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()]
    return {"value": round(n * wl.T / total, 2), "unit": "tokens/s", "cores": int(max(threads)),
            "kind": "oracle",
            "sample": f"{n} full forward pass(es) of the {wl.T}-token workload "
                      f"({total:.1f} s; float64 numpy FFN, float32 C router)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the layer is one "
                                   "GPU's share; multi-GPU runs are not part of this build",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    import torch
    import moe_synth
    import token_routing_expert_router_amd as moe

    moe.load()
    wl = moe_synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = moe_synth.layer_inputs(wl, device=dev)
    x, wr, w13, w2 = inp["x"], inp["w_router"], inp["w13"], inp["w2"]
    T, k, E, F, d = wl.T, wl.k, wl.E, wl.F, wl.d
    dt = x.dtype

    # every output allocated once; the timed loop allocates nothing
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    plan = moe.moe_dispatch(x, moe.moe_route(x, wr, k)[0], E)
    act = torch.empty((T * k, F), dtype=dt, device=dev)
    y_disp = torch.empty((T * k, d), dtype=dt, device=dev)
    y = torch.empty((T, d), dtype=dt, device=dev)
    names = ["route", "dispatch", "gate_up", "down", "combine"]

    def step(ev):
        ev[0].record()
        moe.moe_route(x, wr, k, topk_idx=idx, topk_w=gates)
        ev[1].record()
        moe.moe_dispatch(x, idx, E, out=plan)
        ev[2].record()
        moe.moe_expert_ffn_gate_up(plan["x_disp"], plan["expert_off"], w13, act=act)
        ev[3].record()
        moe.moe_expert_ffn_down(act, plan["expert_off"], w2, y_disp=y_disp)
        ev[4].record()
        moe.moe_combine(y_disp, plan["pair_slot"], gates, y=y)
        ev[5].record()

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for _ in range(args.warmup):
        step(mk())
    events = [mk() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if moe.moe_dispatch_status(plan["ws"]) != 0:
        raise RuntimeError("dispatch raised its device flag")

    work = stage_work(wl)
    stages = {}
    for s, name in enumerate(names):
        ms = sum(ev[s].elapsed_time(ev[s + 1]) for ev in events) / args.steps
        w = work[name]
        bound, t_lb = bound_of(w)
        st = {"us": round(ms * 1e3, 2), "GB_s": round(w["bytes"] / (ms * 1e-3) / 1e9, 1),
              "bound": bound, "roofline_frac": round(t_lb / (ms * 1e-3), 3)}
        if w["flops"]:
            st["TFLOP_s"] = round(w["flops"] / (ms * 1e-3) / 1e12, 1)
        stages[name] = st
    dom = max(names, key=lambda n: stages[n]["us"])
    w = work[dom]
    bound = stages[dom]["bound"]
    t = stages[dom]["us"] * 1e-6
    if bound == "hbm":
        achieved, peak, unit, per = w["bytes"] / t / 1e9, PEAK_HBM_GBS, "GB/s", w["bytes"]
    else:
        peak = PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_FP32_VALU_TFLOPS
        achieved, unit, per = w["flops"] / t / 1e12, "TFLOP/s", w["flops"]
    roofline = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": None, "kernel": dom,
                "per_launch": per}

    ms_step = elapsed / args.steps * 1e3
    line = {
        "metric": METRIC,
        "value": round(T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: MoE layer forward T={T} d={d} E={E} k={k} F={F} "
                               f"{wl.dtype}, softmax top-{k} gating, SwiGLU experts",
                   "T": T, "d": d, "E": E, "k": k, "F": F, "parallelism": "none (1 GPU)"},
        "stages": stages,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
