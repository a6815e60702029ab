"""GPU parity of the receive side of the rank-major (emulated expert-parallel) layout:
each destination's region reordered to expert-major order (moe_ep_recv_plan /
moe_ep_recv_gather), its local grouped GEMM, and the outputs moved back into the
region (moe_ep_recv_scatter) for combine at the sources. Indices and copies are
compared bit-exactly with the oracle; GEMM outputs within the bf16 bar."""
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


def test_ep_recv_plan_zipf_all_ranks(gpu_lib):
    """32 x 128 Zipf workload: every destination's order equals the oracle's."""
    moe = gpu_lib
    wl = moe_synth.WORKLOADS["ep32_zipf"]
    _say(f"ep recv plan {wl}")
    idx, _ = moe_synth.zipf_routing(wl)
    cap = wl.cap_rows_per_dst
    out = moe.moe_dispatch(None, idx.cuda(), wl.E, layout=moe.Layout(wl.n_src, wl.n_dst, cap),
                           d=wl.d, dtype=torch.bfloat16)
    ref = oracle.plan(idx.numpy(), wl.E, wl.n_src, wl.n_dst, cap)
    for r in range(wl.n_dst):
        off, src = moe.moe_ep_recv_plan(out["counts"], out["chunk_off"], r, cap)
        roff, rsrc = oracle.ep_recv_plan(ref["counts"], ref["chunk_off"], r, wl.n_dst, cap)
        torch.cuda.synchronize()
        assert off.cpu().numpy().tolist() == roff.tolist(), r
        assert np.array_equal(src.cpu().numpy(), rsrc), r


EP_CASES = [
    dict(n_src=4, n_dst=4, T=256, d=256, E=16, k=3, F=128),
    dict(n_src=2, n_dst=8, T=130, d=192, E=64, k=6, F=192),     # most local experts tiny
    dict(n_src=8, n_dst=2, T=512, d=128, E=8, k=2, F=320),      # several m-tiles per expert
]


@pytest.mark.parametrize("c", EP_CASES, ids=[str(c) for c in EP_CASES])
def test_ep_receive_path_equals_expert_major(gpu_lib, c):
    """Route, rank-major dispatch, per-destination reorder + grouped GEMM + scatter,
    combine at the sources: bit-identical to the expert-major forward (same rows
    per expert in the same order, so the same tiles), and within the bar of the
    oracle."""
    moe = gpu_lib
    wl = moe_synth.small_workload(moe_synth.WORKLOADS["mid_bf16"], T=c["T"], d=c["d"], E=c["E"],
                                  k=c["k"], F=c["F"])
    _say(f"ep receive path {c}")
    inp = moe_synth.layer_inputs(wl, device="cuda")
    x, wr, w13, w2 = inp["x"], inp["w_router"], inp["w13"], inp["w2"]
    n_src, n_dst, E, k, F, d = c["n_src"], c["n_dst"], c["E"], c["k"], c["F"], c["d"]
    epr = E // n_dst
    cap = n_src * (c["T"] // n_src) * max(k, epr)
    idx, gates, _ = moe.moe_route(x, wr, k)
    plan = moe.moe_dispatch(x, idx, E, layout=moe.Layout(n_src, n_dst, cap))
    assert moe.moe_dispatch_status(plan["ws"]) == 0
    y_disp = torch.zeros((n_dst * cap, d), dtype=x.dtype, device="cuda")
    for r in range(n_dst):
        region = plan["x_disp"][r * cap:(r + 1) * cap]
        off, src = moe.moe_ep_recv_plan(plan["counts"], plan["chunk_off"], r, cap)
        x_local = moe.moe_ep_recv_gather(region, src)
        y_local = moe.moe_expert_ffn(x_local, off, w13[r * epr:(r + 1) * epr].contiguous(),
                                     w2[r * epr:(r + 1) * epr].contiguous())
        moe.moe_ep_recv_scatter(y_local, src, y_disp[r * cap:(r + 1) * cap])
    y_ep = moe.moe_combine(y_disp, plan["pair_slot"], gates)
    fwd = moe.forward(x, wr, w13, w2, k)
    torch.cuda.synchronize()
    assert torch.equal(y_ep.view(torch.int16), fwd["y"].view(torch.int16))
    host = {n: t.cpu() for n, t in inp.items()}
    ref = oracle.forward(host["x"], host["w_router"], host["w13"], host["w2"], k)
    err = oracle.normwise_rel_err(_np(y_ep), ref["y"])
    _say(f"  err {err:.2e}")
    assert err <= BF16_TOL


@pytest.mark.parametrize("r", [0, 31])
def test_ep_receive_full_size_rank(gpu_lib, r):
    """The 32 x 128 Zipf workload at d=7168 with F=2048 experts: destination r's
    reordered input is bit-exact, its 12-expert grouped GEMM matches the oracle on
    sampled rows, and the scatter returns every sampled row to its region row."""
    moe = gpu_lib
    wl = moe_synth.WORKLOADS["ep32_zipf"]
    F = 2048
    _say(f"ep receive rank {r}: {wl}, F={F}")
    idx, _ = moe_synth.zipf_routing(wl)
    x = moe_synth.layer_inputs(wl, device="cuda", with_experts=False)["x"]
    cap, epr, d, k = wl.cap_rows_per_dst, wl.E // wl.n_dst, wl.d, wl.k
    plan = moe.moe_dispatch(x, idx.cuda(), wl.E, layout=moe.Layout(wl.n_src, wl.n_dst, cap))
    region = plan["x_disp"][r * cap:(r + 1) * cap]
    off, src = moe.moe_ep_recv_plan(plan["counts"], plan["chunk_off"], r, cap)
    x_local = moe.moe_ep_recv_gather(region, src)
    g = torch.Generator(device="cuda").manual_seed(1000 + r)
    w13 = (torch.randn((epr, 2 * F, d), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    w2 = (torch.randn((epr, d, F), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    y_local = moe.moe_expert_ffn(x_local, off, w13, w2)
    y_region = torch.zeros_like(region)
    moe.moe_ep_recv_scatter(y_local, src, y_region)
    torch.cuda.synchronize()
    off_h, src_h = off.cpu().numpy(), src.cpu().numpy()
    live = int(off_h[-1])
    _say(f"  live rows {live}, per expert {np.diff(off_h).tolist()}")
    assert live == int(plan["chunk_off"][r, -1])
    # the reordered rows hold their tokens bit-exactly
    rp = plan["row_pair"][r * cap:(r + 1) * cap]
    toks = (rp[src[:live].long()] // k).long()
    assert torch.equal(x_local[:live].view(torch.int16), x[toks].view(torch.int16))
    # sampled rows of every non-empty local expert against the oracle
    rng = np.random.default_rng(r)
    for le in range(epr):
        lo, hi = int(off_h[le]), int(off_h[le + 1])
        if hi == lo:
            continue
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, size=6)]))
        ref = oracle.swiglu_expert(_np(x_local[rows]), w13[le].cpu(), w2[le].cpu())
        err = oracle.normwise_rel_err(_np(y_local[rows]), ref)
        assert err <= BF16_TOL, (le, err)
        back = torch.from_numpy(src_h[rows]).long().cuda()
        assert torch.equal(y_region[back].view(torch.int16), y_local[rows].view(torch.int16))
    del plan, region, x_local, y_local, y_region, w13, w2
    torch.cuda.empty_cache()
