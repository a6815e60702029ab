"""GPU parity of the block-scaled fp8 dispatch payload (moe_dispatch_fp8) and the
receiver's dequantization (moe_ep_recv_gather_fp8) against the oracle: codes and
scales bit-exact, dequantized rows bit-exact after the same float32 product and bf16
rounding, and the whole forward on the dequantized inputs within the bf16 bar."""
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


def _check_payload(x, plan, k):
    """Every live row's codes and scales equal the oracle's for its token."""
    rp = plan["row_pair"]
    live = torch.nonzero(rp >= 0).squeeze(1)
    toks = (rp[live] // k).long()
    codes, scales = oracle.quantize_blocks_fp8(x.cpu())
    qd = plan["q_disp"][live].cpu().numpy()
    qs = plan["q_scale"][live].cpu().numpy()
    t = toks.cpu().numpy()
    bad = np.nonzero(qd != codes[t])
    assert bad[0].size == 0, (bad[0][:4], bad[1][:4], qd[bad][:8], codes[t][bad][:8])
    assert np.array_equal(qs.view(np.uint32), scales[t].view(np.uint32))
    return live, toks


def _crafted_rows():
    """Rows whose block maximum is 448 (so the reciprocal is exactly 1 and the codes
    see the values as they are): every finite E4M3 value, every midpoint between
    neighbours (round half to even), values past 448 in the other blocks' scale,
    zeros of both signs, an all-zero block, and a block with one non-zero value."""
    vals = oracle.e4m3_decode(np.arange(0, 0x7F)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    body = np.concatenate([vals, -vals, mids, -mids, [0.0, -0.0]])
    n = 128 * int(np.ceil((len(body) + 1) / 127))
    rows = []
    for start in range(0, len(body), 127):
        blk = np.zeros(128)
        chunk = body[start:start + 127]
        blk[:len(chunk)] = chunk
        blk[127] = 448.0
        rows.append(blk)
    row = np.concatenate(rows)
    width = ((len(row) + 128 * 3 + 1023) // 1024) * 1024
    full = np.zeros(width)
    full[:len(row)] = row
    tail = np.zeros(width - len(row))
    if len(tail) >= 256:
        tail[5] = -3.5                       # a block with one non-zero value
        tail[128:256] = np.linspace(-1000, 1000, 128)   # a large block
    full[len(row):] = tail
    x = np.stack([full, -full, full * 2.0 ** -20, full * 0.37])
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)


def test_fp8_payload_crafted_rows(gpu_lib):
    moe = gpu_lib
    x = _crafted_rows().cuda()
    T, d = x.shape
    _say(f"fp8 crafted rows {T} x {d}")
    idx = torch.tensor([[0], [1], [2], [3]], dtype=torch.int32, device="cuda")
    plan = moe.moe_dispatch_fp8(x, idx, 4)
    assert moe.moe_dispatch_status(plan["ws"]) == 0
    torch.cuda.synchronize()
    _check_payload(x, plan, 1)


@pytest.mark.parametrize("d", [128, 1024, 8192, 8320, 16512])
def test_fp8_payload_row_widths(gpu_lib, d):
    """Rows of one block, of exactly one and of just over one 8192-element batch of
    the quantizing copy, and of two batches plus a block."""
    moe = gpu_lib
    wl = moe_synth.small_workload(moe_synth.WORKLOADS["mid_bf16"], T=40, d=d, E=8, k=3)
    _say(f"fp8 payload width {wl}")
    inp = moe_synth.layer_inputs(wl, device="cuda", with_experts=False)
    idx, _, _ = moe.moe_route(inp["x"], inp["w_router"], wl.k)
    plan = moe.moe_dispatch_fp8(inp["x"], idx, wl.E)
    assert moe.moe_dispatch_status(plan["ws"]) == 0
    torch.cuda.synchronize()
    live, _ = _check_payload(inp["x"], plan, wl.k)
    assert live.numel() == wl.T * wl.k


@pytest.mark.parametrize("name", ["mid_bf16", "ep32_zipf"])
def test_fp8_payload_and_dequant(gpu_lib, name):
    moe = gpu_lib
    wl = moe_synth.WORKLOADS[name]
    _say(f"fp8 payload {wl}")
    x = moe_synth.layer_inputs(wl, device="cuda", with_experts=False)["x"]
    if name == "ep32_zipf":
        idx, _ = moe_synth.zipf_routing(wl)
        idx = idx.cuda()
        lay = moe.Layout(wl.n_src, wl.n_dst, wl.cap_rows_per_dst)
    else:
        wr = moe_synth.layer_inputs(wl, device="cuda", with_experts=False)["w_router"]
        idx, _, _ = moe.moe_route(x, wr, wl.k)
        lay = None
    plan = moe.moe_dispatch_fp8(x, idx, wl.E, layout=lay)
    assert moe.moe_dispatch_status(plan["ws"]) == 0
    torch.cuda.synchronize()
    live, toks = _check_payload(x, plan, wl.k)
    # the receiver's dequantization, on the whole buffer (rows in place)
    deq = moe.moe_ep_recv_gather_fp8(plan["q_disp"], plan["q_scale"])
    torch.cuda.synchronize()
    codes, scales = oracle.quantize_blocks_fp8(x.cpu())
    ref = torch.from_numpy(oracle.dequantize_blocks_fp8(codes, scales)).to(torch.bfloat16)
    sample = live[:: max(1, live.numel() // 4096)]
    st = (plan["row_pair"][sample] // wl.k).long().cpu()
    assert torch.equal(deq[sample].cpu().view(torch.int16), ref[st].view(torch.int16))
    del plan, deq
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layout", ["expert_major", "rank_major"])
def test_fp8_forward_against_oracle(gpu_lib, layout):
    """Route -> fp8 dispatch -> receiver dequantization (-> reorder per destination) ->
    expert FFN -> combine, against the oracle's forward on the dequantized tokens."""
    moe = gpu_lib
    wl = moe_synth.small_workload(moe_synth.WORKLOADS["mid_bf16"], T=256, d=256, E=16, k=3, F=192)
    _say(f"fp8 forward {layout}")
    inp = moe_synth.layer_inputs(wl, device="cuda")
    x, wr, w13, w2 = inp["x"], inp["w_router"], inp["w13"], inp["w2"]
    idx, gates, _ = moe.moe_route(x, wr, wl.k)
    if layout == "expert_major":
        plan = moe.moe_dispatch_fp8(x, idx, wl.E)
        x_disp = moe.moe_ep_recv_gather_fp8(plan["q_disp"], plan["q_scale"])
        y_disp = moe.moe_expert_ffn(x_disp, plan["expert_off"], w13, w2)
    else:
        n_src, n_dst = 4, 4
        cap = n_src * (wl.T // n_src) * max(wl.k, wl.E // n_dst)
        epr = wl.E // n_dst
        plan = moe.moe_dispatch_fp8(x, idx, wl.E, layout=moe.Layout(n_src, n_dst, cap))
        y_disp = torch.zeros((n_dst * cap, wl.d), dtype=torch.bfloat16, device="cuda")
        for r in range(n_dst):
            off, src = moe.moe_ep_recv_plan(plan["counts"], plan["chunk_off"], r, cap)
            x_local = moe.moe_ep_recv_gather_fp8(plan["q_disp"][r * cap:(r + 1) * cap],
                                                 plan["q_scale"][r * cap:(r + 1) * cap], src)
            y_local = moe.moe_expert_ffn(x_local, off, w13[r * epr:(r + 1) * epr].contiguous(),
                                         w2[r * epr:(r + 1) * epr].contiguous())
            moe.moe_ep_recv_scatter(y_local, src, y_disp[r * cap:(r + 1) * cap])
    y = moe.moe_combine(y_disp, plan["pair_slot"], gates)
    torch.cuda.synchronize()
    codes, scales = oracle.quantize_blocks_fp8(x.cpu())
    xq = torch.from_numpy(oracle.dequantize_blocks_fp8(codes, scales)).to(torch.bfloat16)
    host = {n: t.cpu() for n, t in inp.items()}
    # routing on the unquantized tokens, experts on their dequantized fp8 copies
    _, ref_idx, ref_g = oracle.route(host["x"], host["w_router"], wl.k)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    p = oracle.plan(ref_idx, wl.E)
    xd = oracle.dispatch(xq, p["pair_slot"], wl.T * wl.k)
    yd = oracle.expert_ffn(xd, p["expert_off"], host["w13"], host["w2"])
    ref_y = oracle.combine(yd, p["pair_slot"], ref_g)
    err = oracle.normwise_rel_err(_np(y), ref_y)
    _say(f"  err {err:.2e}")
    assert err <= BF16_TOL
