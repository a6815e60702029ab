"""GPU parity of the forward path: libmoe (through its C ABI) against the CPU oracle.

Bars: routing indices, counts, offsets, slots and dispatch buffers bit-exact; router
logits bit-exact (same float32 order on both sides); float outputs within normwise
relative error 2e-2 for bf16 and 1e-5 for float32 (max |got - ref| / max |ref|).
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-5


def _tol(wl):
    return F32_TOL if wl.dtype == "f32" else BF16_TOL


def _np(t):
    return t.detach().float().cpu().numpy() if t.is_floating_point() else t.cpu().numpy()


def _wl(name, **kw):
    return moe_synth.small_workload(moe_synth.WORKLOADS[name], **kw)


def _say(msg):
    print(msg, flush=True)


ROUTE_CASES = [
    ("tiny_f32", {}),
    ("mid_bf16", dict(T=1000)),                       # ragged: not a multiple of the tile
    ("mid_bf16", dict(T=1)),
    ("large_bf16", dict(T=333)),
    ("mid_bf16", dict(T=257, d=136, E=5, k=5)),       # k = E, d not a multiple of 32
    ("mid_bf16", dict(T=64, d=64, E=512, k=32)),      # largest E and k
    ("mid_bf16", dict(T=40, d=64, E=1, k=1)),
    ("mid_bf16", dict(T=100, d=8, E=16, k=2)),       # one 16-byte piece per row
    ("mid_bf16", dict(T=100, d=264, E=65, k=4)),     # just past one 64-expert group
    ("mid_bf16", dict(T=37, d=520, E=128, k=8)),     # d % 128 != 0, two expert groups
    ("mid_bf16", dict(T=70, d=1032, E=200, k=8)),    # four expert groups, ragged T and d
    ("mid_bf16", dict(T=50, d=256, E=449, k=8)),     # eight expert groups, 63 padded experts
    ("mid_bf16", dict(T=100, d=264, E=1024, k=8)),   # the 16-token form, 1024 experts
    ("mid_bf16", dict(T=33, d=128, E=600, k=32)),    # past 512 experts, largest k
    ("mid_bf16", {}),                                # the full T=4096 router, logits too
]


@pytest.mark.parametrize("name,kw", ROUTE_CASES, ids=[f"{n}-{kw}" for n, kw in ROUTE_CASES])
def test_route_parity(gpu_lib, name, kw):
    moe = gpu_lib
    wl = _wl(name, **kw)
    _say(f"route {wl}")
    inp = moe_synth.layer_inputs(wl, with_experts=False)
    x, w = inp["x"].cuda(), inp["w_router"].cuda()
    idx, gates, logits = moe.moe_route(x, w, wl.k, want_logits=True)
    torch.cuda.synchronize()
    ref_logits, ref_idx, ref_g = oracle.route(inp["x"], inp["w_router"], wl.k)
    got = logits.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref_logits.view(np.uint32)), "logits differ"
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    assert oracle.normwise_rel_err(_np(gates), ref_g) <= F32_TOL


@pytest.mark.parametrize("E,k", [(64, 6), (300, 8)])
def test_route_full_softmax_flag(gpu_lib, E, k):
    moe = gpu_lib
    wl = _wl("mid_bf16", T=300, E=E, k=k)
    inp = moe_synth.layer_inputs(wl, with_experts=False)
    idx, gates, _ = moe.moe_route(inp["x"].cuda(), inp["w_router"].cuda(), wl.k, flags=1)
    torch.cuda.synchronize()
    ref_idx, ref_g = oracle.topk_gating(oracle.router_logits(inp["x"], inp["w_router"]), wl.k,
                                        renorm=False)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    assert oracle.normwise_rel_err(_np(gates), ref_g) <= F32_TOL


def _check_plan(out, ref, rows_live_only=True):
    for key in ("counts", "expert_off", "chunk_off", "pair_slot"):
        got = out[key].cpu().numpy().reshape(ref[key].shape)
        assert np.array_equal(got, ref[key]), key
    assert np.array_equal(out["row_pair"].cpu().numpy(), ref["row_pair"]), "row_pair"


DISPATCH_CASES = [
    ("tiny_f32", {}),
    ("mid_bf16", dict(T=1000, d=256)),
    ("mid_bf16", dict(T=3, d=64, E=8, k=3)),
    ("large_bf16", dict(T=600, d=512)),
]


@pytest.mark.parametrize("name,kw", DISPATCH_CASES, ids=[f"{n}-{kw}" for n, kw in DISPATCH_CASES])
def test_dispatch_parity_expert_major(gpu_lib, name, kw):
    moe = gpu_lib
    wl = _wl(name, **kw)
    _say(f"dispatch {wl}")
    inp = moe_synth.layer_inputs(wl, with_experts=False)
    x = inp["x"].cuda()
    idx, gates, _ = moe.moe_route(x, inp["w_router"].cuda(), wl.k)
    out = moe.moe_dispatch(x, idx, wl.E)
    assert moe.moe_dispatch_status(out["ws"]) == 0
    _, ref_idx, ref_g = oracle.route(inp["x"], inp["w_router"], wl.k)
    ref = oracle.plan(ref_idx, wl.E)
    _check_plan(out, ref)
    xd = out["x_disp"].cpu()
    ref_xd = torch.from_numpy(oracle.dispatch(inp["x"], ref["pair_slot"], wl.pairs)).to(xd.dtype)
    assert torch.equal(xd.view(torch.int16) if xd.dtype == torch.bfloat16 else xd.view(torch.int32),
                       ref_xd.view(torch.int16) if xd.dtype == torch.bfloat16 else ref_xd.view(torch.int32))
    # identity experts: combine(dispatch(x)) == x, bit-exact after one rounding
    y = moe.moe_combine(out["x_disp"], out["pair_slot"], gates)
    torch.cuda.synchronize()
    if wl.dtype == "bf16":
        assert torch.equal(y.cpu(), inp["x"])
    else:
        assert oracle.normwise_rel_err(_np(y), inp["x"].numpy()) <= F32_TOL


def test_dispatch_workspace_reused_across_sizes(gpu_lib):
    """One plan workspace, sized by the first (largest) call, reused by smaller and then
    larger batches again: every plan and every dispatched row still matches the oracle,
    so nothing a call reads is left over from the one before."""
    moe = gpu_lib
    ws = None
    for T in (4096, 1000, 37, 2500):
        wl = _wl("mid_bf16", T=T, d=128)
        _say(f"dispatch with a reused workspace {wl}")
        inp = moe_synth.layer_inputs(wl, with_experts=False)
        x = inp["x"].cuda()
        idx, _, _ = moe.moe_route(x, inp["w_router"].cuda(), wl.k)
        out = moe.moe_dispatch(x, idx, wl.E, out=None if ws is None else {"ws": ws})
        ws = out["ws"]
        assert moe.moe_dispatch_status(ws) == 0
        ref = oracle.plan(idx.cpu().numpy(), wl.E)
        _check_plan(out, ref)
        ref_xd = torch.from_numpy(oracle.dispatch(inp["x"], ref["pair_slot"], wl.pairs)).to(torch.bfloat16)
        assert torch.equal(out["x_disp"].cpu().view(torch.int16), ref_xd.view(torch.int16))


@pytest.mark.parametrize("name,kw", [("mid_bf16", dict(T=700, d=384, E=16, k=4, F=448)),
                                     ("tiny_f32", {})])
def test_forward_outputs_written_whatever_they_held(gpu_lib, name, kw):
    """Every output of route, dispatch, the two GEMMs and combine pre-filled with NaN,
    then with zeros: bit-identical results, so every element the layer returns is
    written by the call and nothing reads an output before writing it."""
    moe = gpu_lib
    wl = _wl(name, **kw)
    _say(f"pre-filled outputs {wl}")
    inp = moe_synth.layer_inputs(wl, device="cuda")
    x, wr, w13, w2 = inp["x"], inp["w_router"], inp["w13"], inp["w2"]
    T, k, E, F, d = wl.T, wl.k, wl.E, wl.F, wl.d
    P = T * k
    res = []
    for fill in (float("nan"), 0.0):
        f32 = dict(dtype=torch.float32, device="cuda")
        idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
        gates = torch.full((T, k), fill, **f32)
        lg = torch.full((T, E), fill, **f32)
        moe.moe_route(x, wr, k, topk_idx=idx, topk_w=gates, logits=lg)
        plan = moe.moe_dispatch(x, idx, E, out={
            "x_disp": torch.full((P, d), fill, dtype=x.dtype, device="cuda"),
            "counts": torch.full((1, E), -7, dtype=torch.int32, device="cuda"),
            "expert_off": torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
            "chunk_off": torch.full((1, 2), -7, dtype=torch.int32, device="cuda"),
            "pair_slot": torch.full((T, k), -7, dtype=torch.int32, device="cuda"),
            "row_pair": torch.full((P,), -7, dtype=torch.int32, device="cuda")})
        act = torch.full((P, F), fill, dtype=x.dtype, device="cuda")
        hu = torch.full((P, 2 * F), fill, dtype=x.dtype, device="cuda") if wl.dtype == "bf16" else None
        moe.moe_expert_ffn_gate_up(plan["x_disp"], plan["expert_off"], w13, act=act, hu_save=hu)
        y_disp = torch.full((P, d), fill, dtype=x.dtype, device="cuda")
        moe.moe_expert_ffn_down(act, plan["expert_off"], w2, y_disp=y_disp)
        y = torch.full((T, d), fill, dtype=x.dtype, device="cuda")
        moe.moe_combine(y_disp, plan["pair_slot"], gates, y=y)
        torch.cuda.synchronize()
        outs = [idx, gates, lg, plan["x_disp"], plan["counts"], plan["expert_off"],
                plan["chunk_off"], plan["pair_slot"], plan["row_pair"], act, y_disp, y]
        if hu is not None:
            outs.append(hu)
        res.append([o.clone() for o in outs])
    for a, b in zip(*res):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else
                           (a.view(torch.int32) if a.dtype == torch.float32 else a),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else
                           (b.view(torch.int32) if b.dtype == torch.float32 else b))
        if a.is_floating_point():
            assert bool(torch.isfinite(a).all())


def test_dispatch_ep_layout_zipf_full(gpu_lib):
    """32 source ranks x 128 tokens, d=7168, E=384, R=8, Zipf(1.2), buffers sized to
    N*T*max(R,E/N) = 49152 rows per destination."""
    moe = gpu_lib
    wl = moe_synth.WORKLOADS["ep32_zipf"]
    _say(f"ep dispatch {wl}")
    idx, w = moe_synth.zipf_routing(wl)
    x = moe_synth.layer_inputs(wl, device="cuda", with_experts=False)["x"]
    lay = moe.Layout(wl.n_src, wl.n_dst, wl.cap_rows_per_dst)
    out = moe.moe_dispatch(x, idx.cuda(), wl.E, layout=lay)
    assert moe.moe_dispatch_status(out["ws"]) == 0
    ref = oracle.plan(idx.numpy(), wl.E, wl.n_src, wl.n_dst, wl.cap_rows_per_dst)
    _check_plan(out, ref)
    # the article's bound, and its tight form, per destination
    live = out["chunk_off"][:, -1].cpu().numpy()
    assert live.max() <= wl.n_src * wl.tokens_per_src * min(wl.k, wl.E // wl.n_dst)
    assert live.max() <= wl.cap_rows_per_dst
    # every live row holds its token bit-exactly
    rp = out["row_pair"]
    live_rows = torch.nonzero(rp >= 0).squeeze(1)
    toks = (rp[live_rows] // wl.k).long()
    assert torch.equal(out["x_disp"][live_rows].view(torch.int16), x[toks].view(torch.int16))
    # identity experts, and random expert outputs against the oracle's combine
    y = moe.moe_combine(out["x_disp"], out["pair_slot"], w.cuda())
    torch.cuda.synchronize()
    assert torch.equal(y, x)
    rows = wl.n_dst * wl.cap_rows_per_dst
    y_disp = torch.zeros((rows, wl.d), dtype=torch.bfloat16, device="cuda")
    y_disp[live_rows] = moe_synth.random_rows(wl, live_rows.numel(), device="cuda")
    y2 = moe.moe_combine(y_disp, out["pair_slot"], w.cuda())
    torch.cuda.synchronize()
    # every token against the oracle, on the live rows only (pair slots renumbered into
    # a compact copy; the receive buffers hold 22.5 GB, mostly unused capacity)
    live_np = live_rows.cpu().numpy()
    compact = np.searchsorted(live_np, ref["pair_slot"])
    assert np.array_equal(live_np[compact], ref["pair_slot"])
    ref_y = oracle.combine(y_disp[live_rows].cpu(), compact, w.numpy())
    err = oracle.normwise_rel_err(_np(y2), ref_y)
    eerr = oracle.elementwise_rel_err(_np(y2), ref_y)
    _say(f"  combine on all {wl.T} tokens: normwise {err:.3e}, elementwise {eerr:.3e}")
    assert err <= BF16_TOL and eerr <= BF16_TOL
    del y_disp, out
    torch.cuda.empty_cache()


def test_dispatch_device_flags(gpu_lib):
    moe = gpu_lib
    idx = torch.tensor([[0, 1], [2, 8], [3, 3], [1, 2]], dtype=torch.int32, device="cuda")
    x = torch.randn((4, 64), device="cuda").to(torch.bfloat16)
    out = moe.moe_dispatch(x, idx, 8)
    assert moe.moe_dispatch_status(out["ws"]) == 5             # MOE_ERR_BAD_INDEX
    ps = out["pair_slot"].cpu().numpy()
    assert ps[1, 1] == -1                                        # the out-of-range pair
    ok = torch.tensor([[0, 1], [2, 7], [3, 4], [1, 2]], dtype=torch.int32, device="cuda")
    out = moe.moe_dispatch(x, ok, 8, out={"ws": out["ws"]})     # the flag is overwritten
    assert moe.moe_dispatch_status(out["ws"]) == 0
    # experts that receive no token leave empty segments
    assert out["counts"].cpu().numpy().tolist() == [[1, 2, 2, 1, 1, 0, 0, 1]]
    assert out["expert_off"].cpu().numpy().tolist() == [0, 1, 3, 5, 6, 7, 7, 7, 8]


FFN_CASES = [
    ("tiny_f32", {}),
    ("mid_bf16", dict(T=700)),
    ("mid_bf16", dict(T=96, d=128, E=4, k=2, F=64)),
    ("large_bf16", dict(T=96, d=7168, E=24, k=8, F=2048)),
]


@pytest.mark.parametrize("name,kw", FFN_CASES, ids=[f"{n}-{kw}" for n, kw in FFN_CASES])
def test_layer_forward_parity(gpu_lib, name, kw):
    moe = gpu_lib
    wl = _wl(name, **kw)
    _say(f"forward {wl}")
    inp = moe_synth.layer_inputs(wl)
    dev = {n: t.cuda() for n, t in inp.items()}
    out = moe.forward(dev["x"], dev["w_router"], dev["w13"], dev["w2"], wl.k)
    torch.cuda.synchronize()
    ref = oracle.forward(inp["x"], inp["w_router"], inp["w13"], inp["w2"], wl.k)
    assert np.array_equal(out["topk_idx"].cpu().numpy(), ref["idx"])
    assert np.array_equal(out["pair_slot"].cpu().numpy(), ref["pair_slot"])
    e_ffn = oracle.normwise_rel_err(_np(out["y_disp"]), ref["y_disp"])
    e_y = oracle.normwise_rel_err(_np(out["y"]), ref["y"])
    ee_ffn = oracle.elementwise_rel_err(_np(out["y_disp"]), ref["y_disp"])
    ee_y = oracle.elementwise_rel_err(_np(out["y"]), ref["y"])
    _say(f"  y_disp err {e_ffn:.3e} (elementwise {ee_ffn:.3e})  y err {e_y:.3e} "
         f"(elementwise {ee_y:.3e})")
    assert e_ffn <= _tol(wl) and e_y <= _tol(wl)
    assert ee_ffn <= _tol(wl) and ee_y <= _tol(wl)


def test_mid_bf16_full_forward(gpu_lib):
    """The full T=4096, d=2048, E=64, k=6, F=1408 layer, in the configuration the
    benchmark times, against the full oracle."""
    moe = gpu_lib
    wl = moe_synth.WORKLOADS["mid_bf16"]
    _say(f"full forward {wl}")
    inp = moe_synth.layer_inputs(wl, device="cuda")
    out = moe.forward(inp["x"], inp["w_router"], inp["w13"], inp["w2"], wl.k)
    torch.cuda.synchronize()
    host = {n: t.cpu() for n, t in inp.items()}
    ref = oracle.forward(host["x"], host["w_router"], host["w13"], host["w2"], wl.k)
    got_idx = out["topk_idx"].cpu().numpy()
    # near-tie audit: tokens whose k-th and (k+1)-th logits are closer than a
    # reordered sum's rounding error keep their oracle selection too
    gap = oracle.topk_gap(oracle.router_logits(host["x"], host["w_router"]), wl.k)
    near = np.nonzero(gap < 1e-4)[0]
    _say(f"  near-tie audit: {near.size} tokens with gap < 1e-4 (min gap {gap.min():.3g})")
    assert np.array_equal(got_idx[near], ref["idx"][near])
    assert np.array_equal(got_idx, ref["idx"])
    for key in ("counts", "expert_off", "pair_slot", "row_pair"):
        assert np.array_equal(out[key].cpu().numpy().reshape(ref[key].shape), ref[key]), key
    e_y = oracle.normwise_rel_err(_np(out["y"]), ref["y"])
    e_ffn = oracle.normwise_rel_err(_np(out["y_disp"]), ref["y_disp"])
    ee_y = oracle.elementwise_rel_err(_np(out["y"]), ref["y"])
    ee_ffn = oracle.elementwise_rel_err(_np(out["y_disp"]), ref["y_disp"])
    _say(f"  y_disp err {e_ffn:.3e} (elementwise {ee_ffn:.3e})  y err {e_y:.3e} "
         f"(elementwise {ee_y:.3e})")
    assert e_y <= BF16_TOL and e_ffn <= BF16_TOL
    assert ee_y <= BF16_TOL and ee_ffn <= BF16_TOL
    # bitwise determinism
    out2 = moe.forward(inp["x"], inp["w_router"], inp["w13"], inp["w2"], wl.k)
    torch.cuda.synchronize()
    assert torch.equal(out["y"], out2["y"]) and torch.equal(out["y_disp"], out2["y_disp"])


def _mtile_rows(a, b, n_extra=4):
    """Rows of expert segment [a, b) to check: the first and last row of every m-tile
    (the grouped GEMM splits a segment into ceil(M/256) equal tiles of ceil(M/tiles)
    rows) plus a few evenly spaced ones, at least 8 in all when the segment has them."""
    M = b - a
    if M <= 0:
        return []
    tiles = -(-M // 256)
    rp = -(-M // tiles)
    rows = set()
    for t in range(tiles):
        lo = a + t * rp
        hi = min(b, lo + rp)
        rows.update((lo, hi - 1))
    rows.update(int(r) for r in np.linspace(a, b - 1, n_extra + 2).round())
    extra = a + 1
    while len(rows) < min(8, M):
        rows.add(extra)
        extra += 1
    return sorted(rows)


@pytest.mark.timeout(1200)
def test_large_bf16_full_forward_every_expert(gpu_lib):
    """T=8192, d=7168, E=384, k=8, F=2048 with all 34 GB of expert weights resident, in
    the configuration the benchmark times: routing and plan checked for every token;
    y_disp on at least 8 rows of EVERY expert (the first and last row of each of its
    m-tiles among them) and y on 512 tokens, against the oracle's SwiGLU with each
    expert's weights streamed to the host one expert at a time."""
    moe = gpu_lib
    wl = moe_synth.WORKLOADS["large_bf16"]
    _say(f"large forward {wl}")
    inp = moe_synth.layer_inputs(wl, device="cuda")
    out = moe.forward(inp["x"], inp["w_router"], inp["w13"], inp["w2"], wl.k)
    torch.cuda.synchronize()
    x_h, wr_h = inp["x"].cpu(), inp["w_router"].cpu()
    _, ref_idx, ref_g = oracle.route(x_h, wr_h, wl.k)
    assert np.array_equal(out["topk_idx"].cpu().numpy(), ref_idx)
    ref = oracle.plan(ref_idx, wl.E)
    for key in ("counts", "expert_off", "pair_slot", "row_pair"):
        assert np.array_equal(out[key].cpu().numpy().reshape(ref[key].shape), ref[key]), key
    # rows to check: the m-tile edges of every expert, and the rows of 512 sampled tokens
    sample_t = np.arange(0, wl.T, wl.T // 512)
    assert sample_t.size == 512
    off = ref["expert_off"]
    want = set()
    for e in range(wl.E):
        rows_e = _mtile_rows(int(off[e]), int(off[e + 1]))
        assert len(rows_e) >= min(8, int(off[e + 1] - off[e]))
        want.update(rows_e)
    want.update(int(r) for r in ref["pair_slot"][sample_t].ravel())
    rows = np.array(sorted(want))
    toks = ref["row_pair"][rows] // wl.k                      # the token each row holds
    xr = oracle._f64(x_h)[toks]
    y_ref_rows = np.zeros((rows.size, wl.d))
    e_of_row = np.searchsorted(off, rows, side="right") - 1
    for e in range(wl.E):
        sel = np.nonzero(e_of_row == e)[0]
        if sel.size:
            y_ref_rows[sel] = oracle.swiglu_expert(xr[sel], inp["w13"][e], inp["w2"][e])
        if e % 64 == 63:
            _say(f"  oracle: experts 0..{e} done")
    got_rows = _np(out["y_disp"][torch.from_numpy(rows).cuda()])
    e_rows = oracle.normwise_rel_err(got_rows, y_ref_rows)
    ee_rows = oracle.elementwise_rel_err(got_rows, y_ref_rows)
    _say(f"  y_disp on {rows.size} rows of all {wl.E} experts: normwise {e_rows:.3e}, "
         f"elementwise {ee_rows:.3e}")
    for e in range(wl.E):                                   # no expert hides behind the rest
        sel = np.nonzero(e_of_row == e)[0]
        if sel.size:
            err_e = oracle.normwise_rel_err(got_rows[sel], y_ref_rows[sel])
            assert err_e <= BF16_TOL, (e, err_e)
    assert e_rows <= BF16_TOL and ee_rows <= BF16_TOL
    # y of the sampled tokens: the gate-weighted sum of the oracle's expert outputs
    pos = {int(r): i for i, r in enumerate(rows)}
    y_ref = np.zeros((sample_t.size, wl.d))
    for n, t in enumerate(sample_t):
        for j in range(wl.k):
            y_ref[n] += ref_g[t, j] * y_ref_rows[pos[int(ref["pair_slot"][t, j])]]
    got_y = _np(out["y"][torch.from_numpy(sample_t).cuda()])
    err = oracle.normwise_rel_err(got_y, y_ref)
    eerr = oracle.elementwise_rel_err(got_y, y_ref)
    _say(f"  y on {sample_t.size} tokens: normwise {err:.3e}, elementwise {eerr:.3e}")
    assert err <= BF16_TOL and eerr <= BF16_TOL
    del inp, out
    torch.cuda.empty_cache()


def test_empty_and_tiny_inputs(gpu_lib):
    moe = gpu_lib
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.randn((8, 64), device="cuda").to(torch.bfloat16)
    idx, g, _ = moe.moe_route(x, w, 2)
    assert idx.shape == (0, 2)
    out = moe.moe_dispatch(x, idx, 8)
    y = moe.moe_combine(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), idx, g)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)


def test_split_ffn_calls_match_composite(gpu_lib):
    """moe_expert_ffn_gate_up + moe_expert_ffn_down == moe_expert_ffn bit for bit,
    and hu_save holds h and u (a = silu(h) * u recomputed from them agrees)."""
    moe = gpu_lib
    wl = _wl("mid_bf16", T=500, d=256, E=16, k=4, F=192)
    inp = moe_synth.layer_inputs(wl, device="cuda")
    idx, gates, _ = moe.moe_route(inp["x"], inp["w_router"], wl.k)
    plan = moe.moe_dispatch(inp["x"], idx, wl.E)
    hu = torch.empty((wl.pairs, 2 * wl.F), dtype=torch.bfloat16, device="cuda")
    y1 = moe.moe_expert_ffn(plan["x_disp"], plan["expert_off"], inp["w13"], inp["w2"], hu_save=hu)
    act = moe.moe_expert_ffn_gate_up(plan["x_disp"], plan["expert_off"], inp["w13"])
    y2 = moe.moe_expert_ffn_down(act, plan["expert_off"], inp["w2"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    h, u = hu[:, :wl.F].float(), hu[:, wl.F:].float()
    a_ref = torch.nn.functional.silu(h) * u
    assert oracle.normwise_rel_err(_np(act), a_ref.cpu().numpy()) <= BF16_TOL
    ref = oracle.forward(inp["x"].cpu(), inp["w_router"].cpu(), inp["w13"].cpu(), inp["w2"].cpu(), wl.k)
    F = wl.F
    x_disp = ref["x_disp"].astype(np.float64)
    w13 = inp["w13"].double().cpu().numpy()
    for e in (0, 7, 15):
        a, b = ref["expert_off"][e], ref["expert_off"][e + 1]
        h_ref = x_disp[a:b] @ w13[e, :F].T
        assert oracle.normwise_rel_err(_np(hu[a:b, :F]), h_ref) <= BF16_TOL


@pytest.mark.parametrize("n_src,n_dst,Ts,E,k", [(4, 8, 600, 64, 6), (3, 1, 1000, 16, 4),
                                                (1, 4, 2000, 384, 8), (64, 16, 16, 64, 2)])
def test_dispatch_ep_layout_multiblock(gpu_lib, n_src, n_dst, Ts, E, k):
    """Rank-major layouts with several 256-token plan blocks per source."""
    moe = gpu_lib
    T = n_src * Ts
    g = torch.Generator().manual_seed(T + E)
    idx = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    cap = n_src * Ts * max(k, E // n_dst)
    _say(f"ep multiblock n_src={n_src} n_dst={n_dst} Ts={Ts} E={E} k={k}")
    x = torch.randn((T, 64), generator=g).to(torch.bfloat16).cuda()
    out = moe.moe_dispatch(x, idx.cuda(), E, layout=moe.Layout(n_src, n_dst, cap))
    assert moe.moe_dispatch_status(out["ws"]) == 0
    ref = oracle.plan(idx.numpy(), E, n_src, n_dst, cap)
    _check_plan(out, ref)
    rp = out["row_pair"]
    live = torch.nonzero(rp >= 0).squeeze(1)
    assert torch.equal(out["x_disp"][live].view(torch.int16), x[(rp[live] // k).long()].view(torch.int16))


@pytest.mark.parametrize("k", [1, 6, 9, 32])
def test_combine_gather_edges(gpu_lib, k):
    """Combine on its own: k across the eight-row load batches, pairs whose slot is
    negative or past rows_total (they contribute nothing, by the ABI), a ragged row
    width; against the oracle's weighted sum over the valid pairs."""
    moe = gpu_lib
    T, d, rows = 300, 264, 700
    _say(f"combine edges k={k}")
    g = torch.Generator().manual_seed(100 + k)
    y_disp = torch.randn(rows, d, generator=g).to(torch.bfloat16)
    slot = torch.randint(0, rows, (T, k), generator=g, dtype=torch.int32)
    slot[::7, 0] = -1
    slot[::11, k - 1] = rows + 5
    w = torch.rand(T, k, generator=g)
    y = moe.moe_combine(y_disp.cuda(), slot.cuda(), w.cuda())
    torch.cuda.synchronize()
    valid = ((slot >= 0) & (slot < rows)).numpy()
    ref = oracle.combine(y_disp, np.where(valid, slot.numpy(), 0), w.numpy() * valid)
    err = oracle.normwise_rel_err(_np(y), ref)
    _say(f"  err {err:.2e}")
    assert err <= BF16_TOL
