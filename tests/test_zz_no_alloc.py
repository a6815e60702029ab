"""moe_dispatch_noalloc (the dispatch whose workspace is the library's fixed per-GPU
array) against moe_dispatch with a caller workspace, through the C ABI: every plan
output and the dispatched buffer bit for bit, on two calls in a row with the second
smaller (the array keeps the first call's contents), in both layouts; and the
rejection of a plan whose workspace exceeds the array."""
import pytest
import torch

import moe_synth

pytestmark = pytest.mark.gpu

PLAN_KEYS = ("counts", "expert_off", "chunk_off", "pair_slot", "row_pair")


def _say(msg):
    print(msg, flush=True)


def _routing(T, E, k, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.argsort(torch.rand((T, E), generator=g), dim=1)[:, :k].to(torch.int32)


def _pair(moe, x, idx, E, lay):
    rows = (lay.n_dst * lay.cap) if lay else idx.numel()
    fill = lambda: torch.full((rows, x.shape[1]), -7.0, dtype=x.dtype, device=x.device)
    ref = moe.moe_dispatch(x, idx, E, layout=lay, out={"x_disp": fill()})
    got = moe.moe_dispatch_noalloc(x, idx, E, layout=lay, out={"x_disp": fill()})
    torch.cuda.synchronize()
    assert moe.moe_dispatch_status(ref["ws"]) == 0
    for key in PLAN_KEYS:
        assert torch.equal(got[key], ref[key]), key
    assert torch.equal(got["x_disp"].view(torch.int16), ref["x_disp"].view(torch.int16))


@pytest.mark.parametrize("layout", [None, (8, 8)], ids=["expert-major", "rank-major"])
def test_noalloc_dispatch_matches_dispatch_twice(gpu_lib, layout):
    moe = gpu_lib
    E, k, d = 384, 8, 512
    for T, seed in ((4096, 1), (1000, 2)):              # the second call is smaller
        lay = None
        if layout:
            n_src, n_dst = layout
            lay = moe.Layout(n_src, n_dst, n_src * (T // n_src) * max(k, E // n_dst))
        _say(f"noalloc dispatch T={T} E={E} k={k} d={d} layout={layout}")
        x = torch.randn((T, d), generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16).cuda()
        _pair(moe, x, _routing(T, E, k, seed).cuda(), E, lay)


def test_noalloc_dispatch_full_size_then_small(gpu_lib):
    """The 384-expert layer's plan (T=8192, d=7168, k=8) from the router, then a
    128-token batch, both against moe_dispatch."""
    moe = gpu_lib
    wl = moe_synth.WORKLOADS["large_bf16"]
    inp = moe_synth.layer_inputs(wl, device="cuda", with_experts=False)
    idx, _, _ = moe.moe_route(inp["x"], inp["w_router"], wl.k)
    _say(f"noalloc dispatch {wl.name}")
    _pair(moe, inp["x"], idx, wl.E, None)
    _pair(moe, inp["x"][:128].contiguous(), idx[:128].contiguous(), wl.E, None)


def test_noalloc_dispatch_rejects_plans_past_the_array(gpu_lib):
    moe = gpu_lib
    E, k, T = 1024, 8, 200_000                       # 782 plan blocks x 1024 experts
    assert moe.load().moe_dispatch_workspace_size(T, E, k, None) > 4 << 20
    x = torch.empty((T, 64), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoEError) as err:
        moe.moe_dispatch_noalloc(x, idx, E)
    assert err.value.status == 4                     # MOE_ERR_CAPACITY, nothing launched
