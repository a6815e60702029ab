"""GPU checks of the two-stream paths: the shared expert computed on a second stream
while the routed path runs (forward_shared, combined by moe_combine_add), and two
micro-batches on two streams (forward_microbatched). Both reproduce their one-stream
forms bit for bit, and both match the oracle within the bf16 bar at the full T=4096
layer."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


def _say(msg):
    print(msg, flush=True)


def _np(t):
    return t.detach().float().cpu().numpy()


def _shared_weights(wl, device):
    g = torch.Generator(device=device).manual_seed(99)
    w13s = (torch.randn((2 * wl.F, wl.d), generator=g, device=device) * 0.02).to(torch.bfloat16)
    w2s = (torch.randn((wl.d, wl.F), generator=g, device=device) * 0.02).to(torch.bfloat16)
    return w13s, w2s


@pytest.mark.parametrize("T,d,E,k,F", [(300, 256, 16, 4, 192), (4096, 2048, 64, 6, 1408)])
def test_shared_expert_overlap(gpu_lib, T, d, E, k, F):
    moe = gpu_lib
    wl = moe_synth.small_workload(moe_synth.WORKLOADS["mid_bf16"], T=T, d=d, E=E, k=k, F=F)
    _say(f"shared expert overlap {wl}")
    inp = moe_synth.layer_inputs(wl, device="cuda")
    x, wr, w13, w2 = inp["x"], inp["w_router"], inp["w13"], inp["w2"]
    w13s, w2s = _shared_weights(wl, "cuda")
    side = torch.cuda.Stream()
    o2 = moe.forward_shared(x, wr, w13, w2, w13s, w2s, k, side_stream=side)
    o1 = moe.forward_shared(x, wr, w13, w2, w13s, w2s, k)
    torch.cuda.synchronize()
    assert torch.equal(o1["y"].view(torch.int16), o2["y"].view(torch.int16))
    host = {n: t.cpu() for n, t in inp.items()}
    ref = oracle.forward(host["x"], host["w_router"], host["w13"], host["w2"], k)
    assert np.array_equal(o2["topk_idx"].cpu().numpy(), ref["idx"])
    ref_y = ref["y"] + oracle.swiglu_expert(_np(x), w13s.cpu(), w2s.cpu())
    err = oracle.normwise_rel_err(_np(o2["y"]), ref_y)
    eerr = oracle.elementwise_rel_err(_np(o2["y"]), ref_y)
    _say(f"  err {err:.2e} (elementwise {eerr:.2e})")
    assert err <= BF16_TOL and eerr <= BF16_TOL


@pytest.mark.parametrize("n_micro", [2, 3])
def test_microbatched_equals_whole_batch(gpu_lib, n_micro):
    moe = gpu_lib
    wl = moe_synth.WORKLOADS["mid_bf16"]
    _say(f"micro-batches {n_micro} {wl}")
    inp = moe_synth.layer_inputs(wl, device="cuda")
    x, wr, w13, w2 = inp["x"], inp["w_router"], inp["w13"], inp["w2"]
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
    y_mb = moe.forward_microbatched(x, wr, w13, w2, wl.k, n_micro, streams=streams)
    y = moe.forward(x, wr, w13, w2, wl.k)["y"]
    torch.cuda.synchronize()
    assert torch.equal(y_mb.view(torch.int16), y.view(torch.int16))
    # and against the oracle's whole-batch layer
    host = {n: t.cpu() for n, t in inp.items()}
    ref = oracle.forward(host["x"], host["w_router"], host["w13"], host["w2"], wl.k)
    err = oracle.normwise_rel_err(_np(y_mb), ref["y"])
    eerr = oracle.elementwise_rel_err(_np(y_mb), ref["y"])
    _say(f"  err {err:.2e} (elementwise {eerr:.2e})")
    assert err <= BF16_TOL and eerr <= BF16_TOL


@pytest.mark.parametrize("T,d,E,k,F,n_dst", [(300, 256, 16, 4, 192, 4), (4096, 2048, 64, 6, 1408, 8)])
def test_ep_split_send_receive(gpu_lib, T, d, E, k, F, n_dst):
    """The send half (route + rank-major dispatch into n_dst regions) and the receive half
    (per destination: reorder, local grouped GEMM, scatter back), on one stream and with
    destinations alternating between two streams, with and without the shared expert on
    the side stream: equal to the expert-major forward bit for bit (one source), the plan
    equal to the oracle's, and y within the bf16 bar of the oracle's layer."""
    moe = gpu_lib
    wl = moe_synth.small_workload(moe_synth.WORKLOADS["mid_bf16"], T=T, d=d, E=E, k=k, F=F)
    _say(f"ep split {wl} n_dst={n_dst}")
    inp = moe_synth.layer_inputs(wl, device="cuda")
    x, wr, w13, w2 = inp["x"], inp["w_router"], inp["w13"], inp["w2"]
    w13s, w2s = _shared_weights(wl, "cuda")
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    o1 = moe.forward_ep_split(x, wr, w13, w2, k, n_dst)
    o2 = moe.forward_ep_split(x, wr, w13, w2, k, n_dst, streams=[main, side])
    o3 = moe.forward_ep_split(x, wr, w13, w2, k, n_dst, w13_shared=w13s, w2_shared=w2s,
                              streams=[main, side])
    y0 = moe.forward(x, wr, w13, w2, k)["y"]
    ys = moe.forward_shared(x, wr, w13, w2, w13s, w2s, k)["y"]
    torch.cuda.synchronize()
    assert torch.equal(o1["y"].view(torch.int16), y0.view(torch.int16))
    assert torch.equal(o2["y"].view(torch.int16), y0.view(torch.int16))
    assert torch.equal(o3["y"].view(torch.int16), ys.view(torch.int16))
    host = {n: t.cpu() for n, t in inp.items()}
    ref = oracle.forward(host["x"], host["w_router"], host["w13"], host["w2"], k)
    cap = T * max(k, E // n_dst)
    ref_plan = oracle.plan(ref["idx"], E, 1, n_dst, cap)
    for key in ("counts", "chunk_off", "pair_slot", "row_pair"):
        got = o2["plan"][key].cpu().numpy().reshape(ref_plan[key].shape)
        assert np.array_equal(got, ref_plan[key]), key
    err = oracle.normwise_rel_err(_np(o2["y"]), ref["y"])
    eerr = oracle.elementwise_rel_err(_np(o2["y"]), ref["y"])
    ref_s = ref["y"] + oracle.swiglu_expert(_np(x), w13s.cpu(), w2s.cpu())
    err_s = oracle.normwise_rel_err(_np(o3["y"]), ref_s)
    _say(f"  err {err:.2e} (elementwise {eerr:.2e}); with shared expert {err_s:.2e}")
    assert err <= BF16_TOL and eerr <= BF16_TOL and err_s <= BF16_TOL
