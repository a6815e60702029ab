#!/usr/bin/env python3
"""Benchmark of the MoE layer's hot path on one MI355X.

Headline step = one forward pass of the layer over one batch of synthetic tokens
already resident in HBM: moe_route -> moe_dispatch -> moe_expert_ffn_gate_up ->
moe_expert_ffn_down -> moe_combine (all libmoe HIP kernels), on the largest layer that
fits one GPU: T=8192, d=7168, E=384, k=8, F=2048 bf16 (34 GB of expert weights
resident). The same JSON line also reports:
  mid          the T=4096, d=2048, E=64, k=6, F=1408 layer forward, with its own
               roofline line,
  train_step   forward + backward of that layer (combine_bwd, route_bwd,
               expert_ffn_bwd, dispatch_bwd) on the same shapes,
  ep_dispatch_combine  the rank-major dispatch and combine of 32 source ranks x 128
               tokens, d=7168, E=384, k=8, Zipf(1.2) routing (identity experts), and
               destination 0's receive path (reorder, 12-expert SwiGLU GEMM, scatter),
  overlap      the mid layer with a shared expert on a second stream, and with two
               micro-batches on two streams, each against its one-stream form,
  roofline     the dominant kernel of the headline step, timed live with HIP events,
  cpu_baseline the CPU oracle on the host cores over a bounded sample of the headline
               workload, scaled to the whole batch.

Prints ONE JSON line.
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
PEAK_FP32_MFMA_TFLOPS = 157.3  # dense fp32 MFMA
PEAKS = {"mfma": PEAK_BF16_TFLOPS, "mfma_f32": PEAK_FP32_MFMA_TFLOPS, "valu": PEAK_FP32_VALU_TFLOPS}


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large_bf16", choices=["large_bf16", "mid_bf16", "tiny_f32"],
                    help="workload of the headline forward step")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline only (no mid layer, train step, EP dispatch/combine or overlap)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--only-mid", action="store_true",
                    help="run only the T=4096 d=2048 E=64 layer forward (for profiler runs)")
    ap.add_argument("--only-overlap", action="store_true",
                    help="run only the two-stream shared-expert and micro-batch forms")
    ap.add_argument("--only-ep", action="store_true",
                    help="run only the rank-major dispatch/combine and receive path")
    ap.add_argument("--only-train", action="store_true",
                    help="run only the forward + backward step (for profiler runs)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def stage_work(wl):
    """Algorithmic bytes and flops per launch of every forward stage."""
    b = 2 if wl.dtype == "bf16" else 4
    T, d, E, k, F = wl.T, wl.d, wl.E, wl.k, wl.F
    P = T * k
    return {
        # x and the router weights read once; indices and gates written. bf16 logits run
        # as float32 matrix-core chains, float32 ones on the vector ALU
        "route": dict(bytes=T * d * b + E * d * b + P * 8, flops=2 * T * d * E,
                      unit="mfma_f32" if wl.dtype == "bf16" else "valu"),
        # each token read once and written k times (the plan's int traffic is < 1 %)
        "dispatch": dict(bytes=T * d * b + P * d * b, flops=0, unit="hbm"),
        # every expert weight read once, dispatched rows read, a = silu(h)*u written
        "gate_up": dict(bytes=E * 2 * F * d * b + P * d * b + P * F * b,
                        flops=2 * P * d * 2 * F, unit="mfma"),
        "down": dict(bytes=E * d * F * b + P * F * b + P * d * b, flops=2 * P * F * d, unit="mfma"),
        # k rows gathered per token, one row written, slots and gates read
        "combine": dict(bytes=P * d * b + T * d * b + P * 8, flops=0, unit="hbm"),
    }


def bwd_work(wl):
    b = 2
    T, d, E, k, F = wl.T, wl.d, wl.E, wl.k, wl.F
    P = T * k
    return {
        # dy read, y_disp read, dy_disp written, gate gradients written
        "combine_bwd": dict(bytes=T * d * b + 2 * P * d * b + P * 4, flops=0, unit="hbm"),
        # dA = dO W2 and dX = dHU W13 (weights read once each), dW2 = dO^T a and
        # dW13 = dHU^T X (fp32 weight gradients written once); 12 P d F flops in all
        "expert_ffn_bwd": dict(bytes=E * 3 * F * d * b + E * 3 * F * d * 4 + 2 * P * d * b
                               + 2 * P * 2 * F * b + P * 2 * F * b + P * d * b,
                               flops=12 * P * d * F, unit="mfma"),
        "route_bwd": dict(bytes=P * d * b + E * d * 4, flops=2 * P * d, unit="hbm"),
        "dispatch_bwd": dict(bytes=P * d * b + T * d * b, flops=0, unit="hbm"),
    }


def bound_of(work):
    """hbm or mfma/valu: whichever lower bound on the time is larger."""
    t_mem = work["bytes"] / (PEAK_HBM_GBS * 1e9)
    if work["flops"] == 0 or work["unit"] == "hbm":
        return "hbm", t_mem
    t_cmp = work["flops"] / (PEAKS[work["unit"]] * 1e12)
    return (work["unit"] if t_cmp >= t_mem else "hbm"), max(t_cmp, t_mem)


def summarize(names, events, steps, work):
    out = {}
    for s, name in enumerate(names):
        ms = sum(ev[s].elapsed_time(ev[s + 1]) for ev in events) / steps
        w = work[name]
        bound, t_lb = bound_of(w)
        st = {"us": round(ms * 1e3, 2), "GB_s": round(w["bytes"] / (ms * 1e-3) / 1e9, 1),
              "bound": bound, "roofline_frac": round(t_lb / (ms * 1e-3), 3)}
        if w["flops"]:
            st["TFLOP_s"] = round(w["flops"] / (ms * 1e-3) / 1e12, 1)
        out[name] = st
    return out


def timed(torch, step, nstages, steps, warmup):
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(nstages + 1)]
    for _ in range(warmup):
        step(mk())
    events = [mk() for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    return time.perf_counter() - t0, events


def forward_bench(torch, moe, wl, dev, steps, warmup):
    import moe_synth
    inp = moe_synth.layer_inputs(wl, device=dev)
    x, wr, w13, w2 = inp["x"], inp["w_router"], inp["w13"], inp["w2"]
    T, k, E, F, d = wl.T, wl.k, wl.E, wl.F, wl.d
    # every output allocated once; the timed loop allocates nothing
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    plan = moe.moe_dispatch(x, moe.moe_route(x, wr, k)[0], E)
    act = torch.empty((T * k, F), dtype=x.dtype, device=dev)
    y_disp = torch.empty((T * k, d), dtype=x.dtype, device=dev)
    y = torch.empty((T, d), dtype=x.dtype, device=dev)

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

    elapsed, events = timed(torch, step, 5, steps, warmup)
    if moe.moe_dispatch_status(plan["ws"]) != 0:
        raise RuntimeError("dispatch raised its device flag")
    stages = summarize(["route", "dispatch", "gate_up", "down", "combine"], events, steps,
                       stage_work(wl))
    return inp, elapsed, stages


def train_bench(torch, moe, wl, dev, steps, warmup):
    import moe_synth
    inp = moe_synth.layer_inputs(wl, device=dev)
    x, wr, w13, w2 = inp["x"], inp["w_router"], inp["w13"], inp["w2"]
    dy = moe_synth.upstream_grad(wl, device=dev)
    T, k, E, F, d = wl.T, wl.k, wl.E, wl.F, wl.d
    P = T * k
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    plan = moe.moe_dispatch(x, moe.moe_route(x, wr, k)[0], E)
    act = torch.empty((P, F), dtype=x.dtype, device=dev)
    hu = torch.empty((P, 2 * F), dtype=x.dtype, device=dev)
    y_disp = torch.empty((P, d), dtype=x.dtype, device=dev)
    y = torch.empty((T, d), dtype=x.dtype, device=dev)
    dy_disp = torch.empty((P, d), dtype=x.dtype, device=dev)
    dgates = torch.empty((T, k), dtype=torch.float32, device=dev)
    dx_disp = torch.empty((P, d), dtype=x.dtype, device=dev)
    dw13 = torch.empty((E, 2 * F, d), dtype=torch.float32, device=dev)
    dw2 = torch.empty((E, d, F), dtype=torch.float32, device=dev)
    ws = torch.empty(int(moe.load().moe_expert_ffn_bwd_workspace_size(E, P, d, F, 1)),
                     dtype=torch.uint8, device=dev)
    dl = torch.empty((T, k), dtype=torch.float32, device=dev)
    dwr = torch.empty((E, d), dtype=torch.float32, device=dev)
    dx = torch.empty((T, d), dtype=x.dtype, device=dev)

    def step(ev):
        ev[0].record()
        moe.moe_route(x, wr, k, topk_idx=idx, topk_w=gates)
        moe.moe_dispatch(x, idx, E, out=plan)
        moe.moe_expert_ffn_gate_up(plan["x_disp"], plan["expert_off"], w13, act=act, hu_save=hu)
        moe.moe_expert_ffn_down(act, plan["expert_off"], w2, y_disp=y_disp)
        moe.moe_combine(y_disp, plan["pair_slot"], gates, y=y)
        ev[1].record()
        moe.moe_combine_bwd(dy, y_disp, plan["pair_slot"], gates, dy_disp=dy_disp, dtopk_w=dgates)
        ev[2].record()
        # the router's backward needs only the gate gradients; running it before the
        # expert backward puts dx_disp's writer right before its reader
        moe.moe_route_bwd(x, idx, gates, dgates, plan["expert_off"], plan["row_pair"], E,
                          dlogits_sel=dl, dw_router=dwr)
        ev[3].record()
        moe.moe_expert_ffn_bwd(plan["x_disp"], dy_disp, hu, plan["expert_off"], w13, w2,
                               dx_disp=dx_disp, dw13=dw13, dw2=dw2, ws=ws)
        ev[4].record()
        moe.moe_dispatch_bwd(dx_disp, plan["pair_slot"], topk_idx=idx, dlogits_sel=dl,
                             w_router=wr, dx=dx)
        ev[5].record()

    elapsed, events = timed(torch, step, 5, steps, warmup)
    fwd_work = {"forward": dict(bytes=sum(w["bytes"] for w in stage_work(wl).values()),
                                flops=sum(w["flops"] for w in stage_work(wl).values()), unit="mfma")}
    fwd_work.update(bwd_work(wl))
    stages = summarize(["forward", "combine_bwd", "route_bwd", "expert_ffn_bwd", "dispatch_bwd"],
                       events, steps, fwd_work)
    del inp
    return {"workload": f"{wl.name}: forward + backward, T={T} d={d} E={E} k={k} F={F} bf16, "
                        "fp32 weight gradients",
            "value": round(T * steps / elapsed, 1), "unit": "tokens/s",
            "ms_per_step": round(elapsed / steps * 1e3, 4), "steps": steps, "stages": stages}


def ep_bench(torch, moe, wl, dev, steps, warmup):
    import moe_synth
    idx, w = moe_synth.zipf_routing(wl, device=dev)
    x = moe_synth.layer_inputs(wl, device=dev, with_experts=False)["x"]
    lay = moe.Layout(wl.n_src, wl.n_dst, wl.cap_rows_per_dst)
    plan = moe.moe_dispatch(x, idx, wl.E, layout=lay)
    y = torch.empty_like(x)

    def step(ev):
        ev[0].record()
        moe.moe_dispatch(x, idx, wl.E, layout=lay, out=plan)
        ev[1].record()
        moe.moe_combine(plan["x_disp"], plan["pair_slot"], w, y=y)   # identity experts
        ev[2].record()

    elapsed, events = timed(torch, step, 2, steps, warmup)
    b, P = 2, wl.T * wl.k
    work = {"dispatch": dict(bytes=wl.T * wl.d * b + P * wl.d * b, flops=0, unit="hbm"),
            "combine": dict(bytes=P * wl.d * b + wl.T * wl.d * b + P * 8, flops=0, unit="hbm")}
    stages = summarize(["dispatch", "combine"], events, steps, work)
    live = plan["chunk_off"][:, -1]
    out = {"workload": f"{wl.name}: rank-major dispatch + combine, {wl.n_src} sources x "
                       f"{wl.tokens_per_src} tokens, d={wl.d} E={wl.E} k={wl.k}, Zipf({wl.zipf_s}), "
                       f"{wl.cap_rows_per_dst} rows per destination",
           "max_rows_per_dst": int(live.max()), "stages": stages}
    out["receive_rank0"] = ep_receive_bench(torch, moe, wl, plan, steps, warmup)
    out["fp8"] = ep_fp8_bench(torch, moe, wl, x, idx, plan, lay, steps, warmup)
    out["partial_combine"] = ep_partial_bench(torch, moe, wl, plan, w, steps, warmup)
    del plan, x
    torch.cuda.empty_cache()
    return out


def ep_partial_bench(torch, moe, wl, plan, w, steps, warmup):
    """Combine with the destinations' partial sums: one row per (token, destination)
    returns instead of one per (token, expert) (identity experts)."""
    cap, d, T = wl.cap_rows_per_dst, wl.d, wl.T
    part = moe.moe_combine_partial(plan["x_disp"], plan["pair_slot"], w, wl.n_dst, cap)
    y = torch.empty((T, d), dtype=torch.bfloat16, device=part.device)

    def step(ev):
        ev[0].record()
        moe.moe_combine_partial(plan["x_disp"], plan["pair_slot"], w, wl.n_dst, cap, partial=part)
        ev[1].record()
        moe.moe_combine_partials(part, plan["pair_slot"], wl.n_dst, cap, y=y)
        ev[2].record()

    elapsed, events = timed(torch, step, 2, steps, warmup)
    dests = (plan["pair_slot"] // cap).sort(dim=1).values
    n_ret = int(T + (dests[:, 1:] != dests[:, :-1]).sum())
    P, b = T * wl.k, 2
    work = {"combine_partial": dict(bytes=P * d * b + n_ret * d * b + P * 8, flops=0, unit="hbm"),
            "combine_partials": dict(bytes=n_ret * d * b + T * d * b, flops=0, unit="hbm")}
    stages = summarize(["combine_partial", "combine_partials"], events, steps, work)
    res = {"return_rows": n_ret, "per_expert_rows": P, "stages": stages}
    del part, y
    return res


def ep_fp8_bench(torch, moe, wl, x, idx, plan, lay, steps, warmup, r=0):
    """The same dispatch with a block-scaled fp8 payload (E4M3 + one f32 scale per 128
    elements), and destination r's dequantizing reorder into its expert-major bf16
    input."""
    cap, d = wl.cap_rows_per_dst, wl.d
    q = moe.moe_dispatch_fp8(x, idx, wl.E, layout=lay)
    off, src = moe.moe_ep_recv_plan(q["counts"], q["chunk_off"], r, cap)
    x_local = torch.empty((cap, d), dtype=torch.bfloat16, device=x.device)

    def step(ev):
        ev[0].record()
        moe.moe_dispatch_fp8(x, idx, wl.E, layout=lay, out=q)
        ev[1].record()
        moe.moe_ep_recv_gather_fp8(q["q_disp"][r * cap:(r + 1) * cap],
                                   q["q_scale"][r * cap:(r + 1) * cap], src, x_local=x_local)
        ev[2].record()

    elapsed, events = timed(torch, step, 2, steps, warmup)
    if moe.moe_dispatch_status(q["ws"]) != 0:
        raise RuntimeError("fp8 dispatch raised its device flag")
    P, L = wl.T * wl.k, int(off[-1])
    row_q = d + d // 128 * 4
    work = {"dispatch_fp8": dict(bytes=wl.T * d * 2 + P * row_q, flops=0, unit="hbm"),
            "dequant_gather": dict(bytes=L * row_q + L * d * 2, flops=0, unit="hbm")}
    stages = summarize(["dispatch_fp8", "dequant_gather"], events, steps, work)
    res = {"payload_bytes_per_row": row_q, "bf16_bytes_per_row": 2 * d,
           "dequant_rows": L, "stages": stages}
    del q, x_local
    return res


def ep_receive_bench(torch, moe, wl, plan, steps, warmup, r=0, F=2048):
    """Destination r's receive path on the rank-major plan: its expert-major order,
    the gather, its grouped GEMM on the E/n_dst local experts (SwiGLU, F=2048, random
    weights), and the scatter back into its region."""
    cap, epr, d = wl.cap_rows_per_dst, wl.E // wl.n_dst, wl.d
    dev = plan["x_disp"].device
    region = plan["x_disp"][r * cap:(r + 1) * cap]
    g = torch.Generator(device=dev).manual_seed(7)
    w13 = (torch.randn((epr, 2 * F, d), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    w2 = (torch.randn((epr, d, F), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    off, src = moe.moe_ep_recv_plan(plan["counts"], plan["chunk_off"], r, cap)
    x_local = torch.empty_like(region)
    act = torch.empty((cap, F), dtype=torch.bfloat16, device=dev)
    y_local = torch.empty_like(region)
    y_region = torch.empty_like(region)

    def step(ev):
        ev[0].record()
        moe.moe_ep_recv_plan(plan["counts"], plan["chunk_off"], r, cap, local_off=off, row_src=src)
        ev[1].record()
        moe.moe_ep_recv_gather(region, src, x_local=x_local)
        ev[2].record()
        moe.moe_expert_ffn_gate_up(x_local, off, w13, act=act)
        ev[3].record()
        moe.moe_expert_ffn_down(act, off, w2, y_disp=y_local)
        ev[4].record()
        moe.moe_ep_recv_scatter(y_local, src, y_region)
        ev[5].record()

    elapsed, events = timed(torch, step, 5, steps, warmup)
    L = int(off[-1])
    b = 2
    work = {"recv_plan": dict(bytes=wl.n_src * epr * 4 + cap * 4, flops=0, unit="hbm"),
            "gather": dict(bytes=2 * L * d * b, flops=0, unit="hbm"),
            "gate_up": dict(bytes=epr * 2 * F * d * b + L * d * b + L * F * b,
                            flops=2 * L * d * 2 * F, unit="mfma"),
            "down": dict(bytes=epr * d * F * b + L * F * b + L * d * b, flops=2 * L * F * d,
                         unit="mfma"),
            "scatter": dict(bytes=2 * L * d * b, flops=0, unit="hbm")}
    stages = summarize(["recv_plan", "gather", "gate_up", "down", "scatter"], events, steps, work)
    res = {"workload": f"destination {r} of {wl.n_dst}: {L} rows over {epr} local experts, "
                       f"SwiGLU F={F} (random weights)",
           "rows": L, "ms": round(elapsed / steps * 1e3, 4), "stages": stages}
    del w13, w2, x_local, act, y_local, y_region
    return res


def overlap_bench(torch, moe, wl, dev, steps, warmup):
    """Two-stream forms of the headline layer: (a) plus a shared expert (SwiGLU, F as the
    routed experts) run on a second stream during the routed path, against the same
    calls on one stream; (b) two micro-batches on two streams against the whole batch."""
    import moe_synth
    inp = moe_synth.layer_inputs(wl, device=dev)
    x, wr, w13, w2 = inp["x"], inp["w_router"], inp["w13"], inp["w2"]
    g = torch.Generator(device=dev).manual_seed(99)
    w13s = (torch.randn((2 * wl.F, wl.d), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    w2s = (torch.randn((wl.d, wl.F), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    o_serial = moe.forward_shared(x, wr, w13, w2, w13s, w2s, wl.k)
    o_over = moe.forward_shared(x, wr, w13, w2, w13s, w2s, wl.k, side_stream=side)
    y_mb = torch.empty_like(x)

    def run(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) / steps * 1e3, 1)

    res = {"workload": f"{wl.name}: T={wl.T} d={wl.d} E={wl.E} k={wl.k} F={wl.F}, shared expert F={wl.F}"}
    res["shared_serial_us"] = run(lambda: moe.forward_shared(x, wr, w13, w2, w13s, w2s, wl.k,
                                                             out=o_serial))
    res["shared_two_streams_us"] = run(lambda: moe.forward_shared(x, wr, w13, w2, w13s, w2s, wl.k,
                                                                  side_stream=side, out=o_over))
    res["whole_batch_us"] = run(lambda: moe.forward(x, wr, w13, w2, wl.k))
    res["two_microbatches_two_streams_us"] = run(
        lambda: moe.forward_microbatched(x, wr, w13, w2, wl.k, 2, streams=[main, side], y=y_mb))
    # the rank-major path in its send and receive halves (8 destination regions of 8
    # experts): destinations' receive paths on one stream, then alternating on two
    # (micro-batches by expert group: every weight read once); and the same with the
    # shared expert on the side stream during the send half
    nd = 8
    o_ep = moe.forward_ep_split(x, wr, w13, w2, wl.k, nd)
    o_eps = moe.forward_ep_split(x, wr, w13, w2, wl.k, nd, streams=[main, side])
    o_epx = moe.forward_ep_split(x, wr, w13, w2, wl.k, nd, w13_shared=w13s, w2_shared=w2s)
    o_epxs = moe.forward_ep_split(x, wr, w13, w2, wl.k, nd, w13_shared=w13s, w2_shared=w2s,
                                  streams=[main, side])
    res["ep_split_destinations"] = nd
    res["ep_split_one_stream_us"] = run(lambda: moe.forward_ep_split(x, wr, w13, w2, wl.k, nd,
                                                                     out=o_ep))
    res["ep_split_two_streams_us"] = run(lambda: moe.forward_ep_split(
        x, wr, w13, w2, wl.k, nd, streams=[main, side], out=o_eps))
    res["ep_split_shared_one_stream_us"] = run(lambda: moe.forward_ep_split(
        x, wr, w13, w2, wl.k, nd, w13_shared=w13s, w2_shared=w2s, out=o_epx))
    res["ep_split_shared_two_streams_us"] = run(lambda: moe.forward_ep_split(
        x, wr, w13, w2, wl.k, nd, w13_shared=w13s, w2_shared=w2s, streams=[main, side],
        out=o_epxs))
    del o_ep, o_eps, o_epx, o_epxs
    del inp, o_serial, o_over
    return res


def _oracle_threads():
    import threadpoolctl
    import oracle
    threads = [oracle.num_threads()]
    threads += [p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()]
    return int(max(threads))


def cpu_baseline(wl, inp, target_s):
    """The oracle as it is, on the host cores, over whole passes of the workload (small
    layers), or over a bounded sample of one pass (the large layer, see below)."""
    import oracle
    if wl.T * wl.d * wl.E * max(wl.F, 1) > 4096 * 2048 * 64 * 1408:
        return cpu_baseline_sampled(wl, inp, target_s)
    host = {n: t.cpu() for n, t in inp.items()}
    n, total = 0, 0.0
    while n < 10 and (total < target_s or n == 0):
        t0 = time.perf_counter()
        oracle.forward(host["x"], host["w_router"], host["w13"], host["w2"], wl.k)
        total += time.perf_counter() - t0
        n += 1
    return {"value": round(n * wl.T / total, 2), "unit": "tokens/s", "cores": _oracle_threads(),
            "kind": "oracle",
            "sample": f"{n} full forward pass(es) of the {wl.T}-token workload "
                      f"({total:.1f} s; float64 numpy FFN, float32 C router)"}


def cpu_baseline_sampled(wl, inp, target_s):
    """One oracle forward of the large layer is minutes of host work (5.8 TFLOP of
    float64 expert GEMMs), so it is sampled: the oracle's own steps run in its order on
    the whole batch (route, plan, dispatch, combine), and its expert FFN on whole
    experts, evenly spaced over the expert ids, until about target_s seconds; the FFN
    time is scaled by E / experts sampled. Each sampled expert's weights are copied to
    the host when its turn comes (the oracle widens them to float64 itself)."""
    import numpy as np
    import oracle
    x_h, wr_h = inp["x"].cpu(), inp["w_router"].cpu()
    t = {}
    t0 = time.perf_counter()
    _, idx, gates = oracle.route(x_h, wr_h, wl.k)
    t["route"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    p = oracle.plan(idx, wl.E)
    t["plan"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    x_disp = oracle.dispatch(x_h, p["pair_slot"], wl.T * wl.k)
    t["dispatch"] = time.perf_counter() - t0
    off = p["expert_off"]
    y_disp = np.zeros((x_disp.shape[0], wl.d), dtype=np.float64)
    order = [int(e) for e in np.linspace(0, wl.E - 1, 64).round()]
    done, t_ffn, rows = 0, 0.0, 0
    for e in order:
        a, b = int(off[e]), int(off[e + 1])
        w13_e, w2_e = inp["w13"][e].cpu(), inp["w2"][e].cpu()
        t0 = time.perf_counter()
        if b > a:
            y_disp[a:b] = oracle.swiglu_expert(x_disp[a:b], w13_e, w2_e)
        t_ffn += time.perf_counter() - t0
        done += 1
        rows += b - a
        if done >= 2 and t_ffn + sum(t.values()) >= target_s:
            break
    t["expert_ffn"] = t_ffn * wl.E / done
    t0 = time.perf_counter()
    oracle.combine(y_disp, p["pair_slot"], gates)
    t["combine"] = time.perf_counter() - t0
    total = sum(t.values())
    return {"value": round(wl.T / total, 3), "unit": "tokens/s", "cores": _oracle_threads(),
            "kind": "oracle",
            "sample": f"one forward of the {wl.T}-token batch: route, plan, dispatch and combine "
                      f"on every token ({t['route'] + t['plan'] + t['dispatch'] + t['combine']:.1f} s), "
                      f"the expert FFN on {done} of {wl.E} experts ({rows} rows, {t_ffn:.1f} s) "
                      f"scaled by {wl.E}/{done} to {t['expert_ffn']:.0f} s; float64 numpy FFN, "
                      f"float32 C router"}


# Sources that define the grouped-GEMM kernels; a traffic record taken with other
# sources no longer describes the kernel and is not reported.
KERNEL_SOURCES = ("token_routing_expert_router_amd/csrc/ffn.hip",
                  "token_routing_expert_router_amd/csrc/gemm_common.h",
                  "token_routing_expert_router_amd/csrc/common.h")


def shape_tag(wl):
    return f"T{wl.T}_d{wl.d}_E{wl.E}_k{wl.k}_F{wl.F}"


def workload_desc(wl):
    return f"T={wl.T} d={wl.d} E={wl.E} k={wl.k} F={wl.F} {wl.dtype}"


def traffic_record_path(kernel, wl):
    """The committed FETCH_SIZE / WRITE_SIZE record of one kernel on one workload."""
    return os.path.join(ROOT, "profiles", f"{kernel}_{shape_tag(wl)}_hbm_traffic.json")


def kernel_source_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, wl):
    """HBM bytes per launch of `kernel` on workload `wl` from the committed FETCH_SIZE /
    WRITE_SIZE record, or None if there is none for this kernel AND workload, or the
    kernel sources changed since it was taken."""
    path = traffic_record_path(kernel, wl)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if (rec.get("stage") != kernel or rec.get("workload") != workload_desc(wl)
            or rec.get("source_sha256") != kernel_source_digest()):
        return None
    return int(rec["traffic_bytes_per_launch"])


def copy_probe(torch, mib):
    n = mib * 1024 * 1024 // 2
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": n * 2, "launches": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the layer is one "
                                   "GPU's share; runs across several GPUs are not supported",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    import torch
    if args.copy_probe_mib:
        copy_probe(torch, args.copy_probe_mib)
        return
    import moe_synth
    import token_routing_expert_router_amd as moe

    moe.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only_overlap:
        ov = overlap_bench(torch, moe, moe_synth.WORKLOADS["mid_bf16"], dev, args.steps,
                           args.warmup)
        print(json.dumps({"overlap": ov}), flush=True)
        return
    if args.only_ep:
        ep = ep_bench(torch, moe, moe_synth.WORKLOADS["ep32_zipf"], dev, args.steps, args.warmup)
        print(json.dumps({"ep_dispatch_combine": ep}), flush=True)
        return
    if args.only_train:
        ts = train_bench(torch, moe, moe_synth.WORKLOADS["mid_bf16_train"], dev, args.steps,
                         args.warmup)
        print(json.dumps({"train_step": ts}), flush=True)
        return
    wl = moe_synth.WORKLOADS[args.workload]
    if args.only_mid:
        wl = moe_synth.WORKLOADS["mid_bf16"]
    inp, elapsed, stages = forward_bench(torch, moe, wl, dev, args.steps, args.warmup)
    T, k, E, F, d = wl.T, wl.k, wl.E, wl.F, wl.d
    line = {
        "metric": METRIC,
        "value": round(T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: MoE layer forward {workload_desc(wl)}, softmax "
                               f"top-{k} gating, SwiGLU experts",
                   "T": T, "d": d, "E": E, "k": k, "F": F, "parallelism": "none (1 GPU)"},
        "stages": stages,
        "roofline": roofline_of(wl, stages),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
    del inp
    torch.cuda.empty_cache()
    if not args.no_extras and not args.only_mid and wl.dtype == "bf16":
        mwl = moe_synth.WORKLOADS["mid_bf16"]
        minp, mel, mst = forward_bench(torch, moe, mwl, dev, args.steps, args.warmup)
        del minp
        torch.cuda.empty_cache()
        line["mid"] = {"workload": f"{mwl.name}: MoE layer forward {workload_desc(mwl)}",
                       "value": round(mwl.T * args.steps / mel, 1), "unit": "tokens/s",
                       "ms_per_step": round(mel / args.steps * 1e3, 4), "steps": args.steps,
                       "stages": mst, "roofline": roofline_of(mwl, mst)}
        line["train_step"] = train_bench(torch, moe, moe_synth.WORKLOADS["mid_bf16_train"], dev,
                                         max(5, args.steps // 2), max(2, args.warmup // 2))
        torch.cuda.empty_cache()
        line["ep_dispatch_combine"] = ep_bench(torch, moe, moe_synth.WORKLOADS["ep32_zipf"], dev,
                                               max(5, args.steps // 2), max(2, args.warmup // 2))
        torch.cuda.empty_cache()
        line["overlap"] = overlap_bench(torch, moe, mwl, dev, max(5, args.steps // 2),
                                        max(2, args.warmup // 2))
    print(json.dumps(line), flush=True)


def roofline_of(wl, stages):
    """The dominant stage's kernel against its roofline: algorithmic bytes (or flops) per
    launch over its event-timed average duration."""
    work = stage_work(wl)
    dom = max(stages, key=lambda n: stages[n]["us"])
    w = work[dom]
    bound = stages[dom]["bound"]
    t = stages[dom]["us"] * 1e-6
    if bound == "hbm":
        achieved, peak, unit, per = w["bytes"] / t / 1e9, PEAK_HBM_GBS, "GB/s", w["bytes"]
    else:
        peak = PEAKS[bound]
        achieved, unit, per = w["flops"] / t / 1e12, "TFLOP/s", w["flops"]
    out = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
           "frac": round(achieved / peak, 4), "traffic": measured_traffic(dom, wl), "kernel": dom,
           "per_launch": per}
    if w["flops"]:
        out["mfma_frac"] = round(w["flops"] / t / 1e12 / PEAK_BF16_TFLOPS, 4)
        out["hbm_frac"] = round(w["bytes"] / t / 1e9 / PEAK_HBM_GBS, 4)
    return out


if __name__ == "__main__":
    main()
