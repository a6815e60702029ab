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
