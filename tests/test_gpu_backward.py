"""GPU parity of the backward path (training step) against the CPU oracle.

combine_bwd -> route_bwd -> expert_ffn_bwd (dgrad + wgrad grouped GEMMs) ->
dispatch_bwd, driven through the C ABI, every gradient compared with
oracle.backward (float64) within the bf16 bar: normwise relative error <= 2e-2.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


def _np(t):
    return t.detach().float().cpu().numpy()


def _say(msg):
    print(msg, flush=True)


def _run(moe, wl, device="cuda", inputs=None):
    inp = inputs or moe_synth.layer_inputs(wl, device=device)
    dy = moe_synth.upstream_grad(wl, device=device)
    fwd = moe.forward(inp["x"], inp["w_router"], inp["w13"], inp["w2"], wl.k,
                      save_for_backward=True)
    bwd = moe.backward(inp["x"], inp["w_router"], inp["w13"], inp["w2"], fwd, dy)
    torch.cuda.synchronize()
    return inp, dy, fwd, bwd


def _compare(wl, inp, dy, fwd, bwd, tol=BF16_TOL):
    host = {n: t.cpu() for n, t in inp.items()}
    ref = oracle.backward(host["x"], host["w_router"], host["w13"], host["w2"], dy.cpu(), wl.k)
    assert np.array_equal(fwd["topk_idx"].cpu().numpy(), ref["idx"])
    assert np.array_equal(fwd["pair_slot"].cpu().numpy(), ref["pair_slot"])
    errs, eerrs = {}, {}
    for mine, theirs in (("dgates", "dgates"), ("dy_disp", "dy_disp"), ("dx_disp", "dx_disp"),
                         ("dw13", "dw13"), ("dw2", "dw2"), ("dlogits_sel", "dlogits_sel"),
                         ("dw_router", "dw_router"), ("dx", "dx")):
        errs[mine] = oracle.normwise_rel_err(_np(bwd[mine]), ref[theirs])
        eerrs[mine] = oracle.elementwise_rel_err(_np(bwd[mine]), ref[theirs])
    _say("  normwise    " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    _say("  elementwise " + "  ".join(f"{k} {v:.2e}" for k, v in eerrs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad
    return ref


BWD_CASES = [
    dict(T=300, d=256, E=8, k=2, F=192),
    dict(T=77, d=128, E=16, k=3, F=64),        # ragged rows, experts with no token
    dict(T=700, d=512, E=4, k=2, F=320),       # several 256-row tiles per expert
    dict(T=64, d=192, E=64, k=6, F=128),       # most experts empty or nearly so
    dict(T=150, d=128, E=16, k=10, F=64),      # k above 8: the multi-batch gathers
    # the 384-expert layer's widths: dA contracts over 7168 (112 stages), dX has 28
    # n-tiles, each expert's dW13 is 4096 x 7168
    dict(T=64, d=7168, E=4, k=2, F=2048),
]


@pytest.mark.parametrize("kw", BWD_CASES, ids=[str(c) for c in BWD_CASES])
def test_backward_parity(gpu_lib, kw):
    moe = gpu_lib
    wl = moe_synth.small_workload(moe_synth.WORKLOADS["mid_bf16_train"], **kw)
    _say(f"backward {wl}")
    inp, dy, fwd, bwd = _run(moe, wl)
    _compare(wl, inp, dy, fwd, bwd)


def test_backward_empty_experts_get_zero_weight_grads(gpu_lib):
    moe = gpu_lib
    wl = moe_synth.small_workload(moe_synth.WORKLOADS["mid_bf16_train"], T=5, d=64, E=32, k=2, F=64)
    inp, dy, fwd, bwd = _run(moe, wl)
    counts = fwd["counts"].cpu().numpy()[0]
    empty = np.nonzero(counts == 0)[0]
    assert len(empty) > 0
    for e in empty:
        assert torch.count_nonzero(bwd["dw13"][e]) == 0
        assert torch.count_nonzero(bwd["dw2"][e]) == 0
        assert torch.count_nonzero(bwd["dw_router"][e]) == 0


def test_mid_bf16_train_full(gpu_lib):
    """The full T=4096, d=2048, E=64, k=6, F=1408 forward + backward against the
    full oracle, and bitwise determinism of every gradient."""
    moe = gpu_lib
    wl = moe_synth.WORKLOADS["mid_bf16_train"]
    _say(f"train step {wl}")
    inp, dy, fwd, bwd = _run(moe, wl)
    _compare(wl, inp, dy, fwd, bwd)
    fwd2 = moe.forward(inp["x"], inp["w_router"], inp["w13"], inp["w2"], wl.k,
                       save_for_backward=True)
    bwd2 = moe.backward(inp["x"], inp["w_router"], inp["w13"], inp["w2"], fwd2, dy)
    torch.cuda.synchronize()
    for key in ("dx", "dw_router", "dw13", "dw2", "dgates"):
        assert torch.equal(bwd[key], bwd2[key]), key


@pytest.mark.parametrize("kw", [dict(T=300, d=256, E=8, k=2, F=192), dict(T=700, d=512, E=4, k=2, F=320)],
                         ids=["F192", "F320"])
def test_expert_bwd_writes_every_live_element(gpu_lib, kw):
    """Outputs pre-filled with NaN and with zeros give bit-identical results: every
    weight-gradient element and every live dx_disp row is written (tiles whose rows or
    columns run past the matrix included), none is read before it is written."""
    moe = gpu_lib
    wl = moe_synth.small_workload(moe_synth.WORKLOADS["mid_bf16_train"], **kw)
    inp, dy, fwd, bwd = _run(moe, wl)
    rows_live = int(fwd["expert_off"][-1])
    outs = []
    for fill in (float("nan"), 0.0):
        dxd = torch.full_like(bwd["dx_disp"], fill)
        dw13 = torch.full_like(bwd["dw13"], fill)
        dw2 = torch.full_like(bwd["dw2"], fill)
        moe.moe_expert_ffn_bwd(fwd["x_disp"], bwd["dy_disp"], fwd["hu_save"], fwd["expert_off"],
                               inp["w13"], inp["w2"], dx_disp=dxd, dw13=dw13, dw2=dw2)
        torch.cuda.synchronize()
        outs.append((dxd[:rows_live].clone(), dw13.clone(), dw2.clone()))
    for a, b in zip(*outs):
        assert torch.isfinite(a).all()
        assert torch.equal(a, b)
    assert torch.equal(outs[0][1], bwd["dw13"]) and torch.equal(outs[0][2], bwd["dw2"])
