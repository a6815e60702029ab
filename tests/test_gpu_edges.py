"""GPU parity at the limits and degenerate routings of dispatch -> expert FFN -> combine,
and of their backward (combine_bwd -> expert_ffn_bwd -> dispatch_bwd).

The routing is given (not produced by the router), so these reach sizes and shapes the
router's own limits keep out of the whole-layer tests: the largest expert count the
plan and the grouped GEMM take (E = 1024), every token sent to the same k experts (a
few experts with several tiles each, every other expert empty), one expert holding
every row, experts holding exactly one tile of rows or one row past it, and widths of
exactly one n-tile or one n-tile plus 64 columns. The plan
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
    elif kind in ("blocks", "blocks224"):   # token t to experts (t // R + j) mod E: R-row runs
        base = torch.arange(T, dtype=torch.int64) // (256 if kind == "blocks" else 224)
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
    ("blocks", 1024, 128, 4, 1, 64),      # experts of exactly 256 rows
    ("blocks", 1025, 128, 5, 1, 64),      # and one with 1 row
    # the grouped GEMM's own tile edges (224 token rows; n-tiles of 192 gate/up and 384
    # down columns)
    ("blocks224", 896, 384, 4, 1, 192),   # experts of exactly 224 rows; one full n-tile each
    ("blocks224", 897, 448, 5, 1, 256),   # and one of 1 row; a full n-tile plus 64 columns
    ("same", 449, 768, 1, 1, 448),        # one expert of 449 rows (three m-tiles); two full down n-tiles
    # the headline layer's widths on one expert of 2048 rows: ten m-tiles, 11 gate/up
    # n-tiles (the last 128 columns wide) and 19 down n-tiles (the last 256 wide)
    ("same", 2048, 7168, 1, 1, 2048),
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


BWD_CASES = [
    # kind, T, d, E, k, F
    ("random", 300, 64, 1024, 8, 64),     # the largest E: experts of 0-8 rows, many empty
    ("same", 700, 128, 8, 3, 64),         # 700-row experts: long weight-gradient contractions
    ("blocks", 1025, 128, 5, 1, 64),      # experts of 256 rows and one of 1 row
    ("blocks224", 897, 448, 5, 1, 256),   # 224-row experts and one of 1 row; partial n-tiles
]


@pytest.mark.parametrize("kind,T,d,E,k,F", BWD_CASES,
                         ids=[f"{c[0]}-T{c[1]}-d{c[2]}-E{c[3]}-k{c[4]}-F{c[5]}" for c in BWD_CASES])
def test_given_routing_backward(gpu_lib, kind, T, d, E, k, F):
    """combine_bwd -> expert_ffn_bwd -> dispatch_bwd after a forward with the same given
    routing, against the oracle's transposes; experts without rows get zero weight
    gradients, bit for bit."""
    moe = gpu_lib
    wl = moe_synth.small_workload(moe_synth.WORKLOADS["mid_bf16_train"], T=T, d=d, E=E, k=k, F=F)
    _say(f"given routing backward {kind}: {wl}")
    inp = moe_synth.layer_inputs(wl)
    idx, gates = _routing(kind, T, E, k)
    x, w13, w2 = inp["x"].cuda(), inp["w13"].cuda(), inp["w2"].cuda()
    dy = moe_synth.upstream_grad(wl)
    P = T * k
    plan = moe.moe_dispatch(x, idx.cuda(), E)
    hu = torch.empty((P, 2 * F), dtype=torch.bfloat16, device="cuda")
    act = moe.moe_expert_ffn_gate_up(plan["x_disp"], plan["expert_off"], w13, hu_save=hu)
    y_disp = moe.moe_expert_ffn_down(act, plan["expert_off"], w2)
    dy_disp, dgates = moe.moe_combine_bwd(dy.cuda(), y_disp, plan["pair_slot"], gates.cuda())
    dx_disp, dw13, dw2 = moe.moe_expert_ffn_bwd(plan["x_disp"], dy_disp, hu, plan["expert_off"],
                                                w13, w2)
    dx = moe.moe_dispatch_bwd(dx_disp, plan["pair_slot"])
    torch.cuda.synchronize()

    ref = oracle.plan(idx.numpy(), E)
    assert np.array_equal(plan["pair_slot"].cpu().numpy(), ref["pair_slot"])
    xd = oracle.dispatch(inp["x"], ref["pair_slot"], P)
    yd = oracle.expert_ffn(xd, ref["expert_off"], inp["w13"], inp["w2"])
    r_dyd, r_dg = oracle.combine_bwd(dy, yd, ref["pair_slot"], gates.numpy(), P)
    r_dxd, r_dw13, r_dw2 = oracle.expert_ffn_bwd(xd, r_dyd, ref["expert_off"], inp["w13"],
                                                 inp["w2"])
    r_dx = oracle.dispatch_bwd(r_dxd, ref["pair_slot"])
    errs = {
        "dgates": oracle.normwise_rel_err(dgates.cpu().numpy(), r_dg),
        "dy_disp": oracle.normwise_rel_err(dy_disp.float().cpu().numpy(), r_dyd),
        "dx_disp": oracle.normwise_rel_err(dx_disp.float().cpu().numpy(), r_dxd),
        "dw13": oracle.normwise_rel_err(dw13.cpu().numpy(), r_dw13),
        "dw2": oracle.normwise_rel_err(dw2.cpu().numpy(), r_dw2),
        "dx": oracle.normwise_rel_err(dx.float().cpu().numpy(), r_dx),
    }
    _say("  " + "  ".join(f"{n} {v:.2e}" for n, v in errs.items()))
    bad = {n: v for n, v in errs.items() if not v <= BF16_TOL}
    assert not bad, bad
    empty = np.nonzero(np.diff(ref["expert_off"]) == 0)[0]
    if empty.size:
        assert torch.count_nonzero(dw13[torch.from_numpy(empty).cuda()]).item() == 0
        assert torch.count_nonzero(dw2[torch.from_numpy(empty).cuda()]).item() == 0


@pytest.mark.parametrize("layout", [None, (4, 4, 64)], ids=["expert-major", "rank-major"])
def test_empty_batch_writes_an_empty_plan(gpu_lib, layout):
    """T = 0: the plan outputs describe an empty batch whatever the buffers held before
    (zero counts and offsets, every row unused, the flag clear), and the router's
    backward gives a zero weight gradient without reading a plan."""
    moe = gpu_lib
    E, k, d = 16, 2, 64
    lay = moe.Layout(*layout) if layout else None
    n_src, n_dst, cap = layout if layout else (1, 1, 0)
    dev = "cuda"
    lib = moe.load()
    ws = torch.full((max(256, int(lib.moe_dispatch_workspace_size(0, E, k, None))),), 0x55,
                    dtype=torch.uint8, device=dev)
    counts = torch.full((n_src, E), 7, dtype=torch.int32, device=dev)
    expert_off = torch.full((E + 1,), 7, dtype=torch.int32, device=dev)
    chunk_off = torch.full((n_dst, n_src + 1), 7, dtype=torch.int32, device=dev)
    row_pair = torch.full((max(1, n_dst * cap),), 7, dtype=torch.int32, device=dev)
    import ctypes
    clay = lay._c() if lay else None
    st = lib.moe_dispatch(None, None, 0, d, E, k, 1, ctypes.byref(clay) if clay else None,
                          counts.data_ptr(), expert_off.data_ptr(), chunk_off.data_ptr(), None,
                          row_pair.data_ptr(), None, ws.data_ptr(), ws.numel(),
                          torch.cuda.current_stream().cuda_stream)
    assert st == 0
    assert moe.moe_dispatch_status(ws) == 0
    assert int(counts.abs().sum()) == 0 and int(expert_off.abs().sum()) == 0
    assert int(chunk_off.abs().sum()) == 0
    if cap:
        assert bool((row_pair == -1).all())
    dwr = torch.full((E, d), float("nan"), dtype=torch.float32, device=dev)
    st = lib.moe_route_bwd(None, None, None, None, None, None, 0, d, E, k, 1, None,
                           dwr.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(dwr)) == 0
