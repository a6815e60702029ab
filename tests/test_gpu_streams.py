"""Two independent layers enqueued on two streams at once give, bit for bit, what each
gives alone on the default stream: no call shares device state with another, so
concurrent callers (each with its own buffers) cannot disturb each other. The forward
and the backward are both checked; the two layers differ in every size."""
import pytest
import torch

import moe_synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _inputs(wl):
    inp = moe_synth.layer_inputs(wl, device="cuda")
    return inp, moe_synth.upstream_grad(wl, device="cuda")


def _step(moe, wl, inp, dy):
    fwd = moe.forward(inp["x"], inp["w_router"], inp["w13"], inp["w2"], wl.k,
                      save_for_backward=True)
    bwd = moe.backward(inp["x"], inp["w_router"], inp["w13"], inp["w2"], fwd, dy)
    return fwd, bwd


KEYS_FWD = ("topk_idx", "topk_w", "pair_slot", "x_disp", "y_disp", "y")
KEYS_BWD = ("dx", "dw_router", "dw13", "dw2", "dgates")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def test_two_layers_on_two_streams_match_alone(gpu_lib):
    moe = gpu_lib
    base = moe_synth.WORKLOADS["mid_bf16_train"]
    wa = moe_synth.small_workload(base, T=1024, d=512, E=16, k=4, F=320)
    wb = moe_synth.small_workload(base, T=700, d=256, E=24, k=6, F=192)
    _say(f"two streams: {wa} | {wb}")
    ia, da = _inputs(wa)
    ib, db = _inputs(wb)
    torch.cuda.synchronize()
    alone_a = _step(moe, wa, ia, da)
    alone_b = _step(moe, wb, ib, db)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        with torch.cuda.stream(sa):
            got_a = _step(moe, wa, ia, da)
        with torch.cuda.stream(sb):
            got_b = _step(moe, wb, ib, db)
        torch.cuda.synchronize()
        for (alone, got, name) in ((alone_a, got_a, "a"), (alone_b, got_b, "b")):
            for key in KEYS_FWD:
                assert torch.equal(_bits(alone[0][key]), _bits(got[0][key])), (rep, name, key)
            for key in KEYS_BWD:
                assert torch.equal(_bits(alone[1][key]), _bits(got[1][key])), (rep, name, key)
