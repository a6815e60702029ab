"""GPU parity at the limits and degenerate routings of dispatch -> expert FFN -> combine.

The routing is given (not produced by the router), so these reach sizes and shapes the
router's own limits keep out of the whole-layer tests: the largest expert count the
plan and the grouped GEMM take (E = 1024), every token sent to the same k experts (a
few experts with several 256-row tiles each, every other expert empty), one expert
holding every row, and experts holding exactly one tile or one row past it. The plan
must match the oracle's bit for bit, the dispatched rows bitwise, the expert outputs
and the combined tokens within the bf16 bar.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


def _say(msg):
    print(msg, flush=True)


def _routing(kind, T, E, k, seed=0):
    """Expert ids [T, k] (distinct per token) and renormalised gates [T, k]."""
    g = torch.Generator().manual_seed(seed)
    if kind == "same":            # every token to experts 0..k-1, in that order
        idx = torch.arange(k, dtype=torch.int32).repeat(T, 1)
    elif kind == "reversed":      # every token to experts E-1, E-2, ..., E-k
        idx = (E - 1 - torch.arange(k, dtype=torch.int32)).repeat(T, 1)
    elif kind == "random":        # k distinct uniform experts per token
        idx = torch.argsort(torch.rand((T, E), generator=g), dim=1)[:, :k].to(torch.int32)
    elif kind == "blocks":        # token t to experts (t // 256 + j) mod E: 256-row runs
        base = torch.arange(T, dtype=torch.int64) // 256
        idx = ((base[:, None] + torch.arange(k)[None, :]) % E).to(torch.int32)
    else:
        raise ValueError(kind)
    gates = torch.softmax(torch.randn((T, k), generator=g), dim=1).to(torch.float32)
    return idx.contiguous(), gates.contiguous()


CASES = [
    # kind, T, d, E, k, F
    ("random", 600, 64, 1024, 8, 64),     # the largest E: most experts hold ~5 rows
    ("same", 700, 128, 8, 3, 64),         # three experts with 700 rows (3 tiles), five empty
    ("reversed", 520, 192, 16, 2, 128),   # the last experts hold everything
    ("same", 1000, 256, 1, 1, 128),       # one expert, every row: a dense FFN of 4 tiles
    ("blocks", 1024, 128, 4, 1, 64),      # experts of exactly 256 rows (one full tile)
    ("blocks", 1025, 128, 5, 1, 64),      # and one with 1 row
]


@pytest.mark.parametrize("kind,T,d,E,k,F", CASES, ids=[f"{c[0]}-T{c[1]}-d{c[2]}-E{c[3]}-k{c[4]}-F{c[5]}"
                                                      for c in CASES])
def test_given_routing_path(gpu_lib, kind, T, d, E, k, F):
    moe = gpu_lib
    wl = moe_synth.small_workload(moe_synth.WORKLOADS["mid_bf16"], T=T, d=d, E=E, k=k, F=F)
    _say(f"given routing {kind}: {wl}")
    inp = moe_synth.layer_inputs(wl)
    idx, gates = _routing(kind, T, E, k)
    x, w13, w2 = inp["x"].cuda(), inp["w13"].cuda(), inp["w2"].cuda()
    plan = moe.moe_dispatch(x, idx.cuda(), E)
    y_disp = moe.moe_expert_ffn(plan["x_disp"], plan["expert_off"], w13, w2)
    y = moe.moe_combine(y_disp, plan["pair_slot"], gates.cuda())
    torch.cuda.synchronize()
    assert moe.moe_dispatch_status(plan["ws"]) == 0

    ref = oracle.plan(idx.numpy(), E)
    for key in ("counts", "expert_off", "pair_slot"):
        assert np.array_equal(plan[key].cpu().numpy().reshape(ref[key].shape), ref[key]), key
    assert np.array_equal(plan["row_pair"].cpu().numpy(), ref["row_pair"]), "row_pair"
    ref_xd = oracle.dispatch(inp["x"], ref["pair_slot"], T * k)
    got_xd = plan["x_disp"].cpu()
    assert torch.equal(got_xd.view(torch.int16),
                       torch.from_numpy(ref_xd).to(torch.bfloat16).view(torch.int16)), "x_disp"
    ref_yd = oracle.expert_ffn(ref_xd, ref["expert_off"], inp["w13"], inp["w2"])
    ref_y = oracle.combine(ref_yd, ref["pair_slot"], gates.numpy())
    e_yd = oracle.normwise_rel_err(y_disp.float().cpu().numpy(), ref_yd)
    e_y = oracle.normwise_rel_err(y.float().cpu().numpy(), ref_y)
    _say(f"  rows per expert max {int(np.diff(ref['expert_off']).max())}, "
         f"empty experts {int((np.diff(ref['expert_off']) == 0).sum())}; "
         f"y_disp err {e_yd:.2e}  y err {e_y:.2e}")
    assert e_yd <= BF16_TOL and e_y <= BF16_TOL
