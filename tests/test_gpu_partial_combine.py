"""GPU parity of the partial combine of the rank-major layout (moe_combine_partial at
the destinations, moe_combine_partials at the sources) against the oracle."""
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


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def test_partial_combine_one_destination_is_combine(gpu_lib):
    """With one destination the partial is the combine itself (same fma order, same
    rounding), so both paths agree bit for bit."""
    moe = gpu_lib
    wl = moe_synth.small_workload(moe_synth.WORKLOADS["mid_bf16"], T=300, d=256, E=16, k=4, F=64)
    idx, w = moe_synth.zipf_routing(moe_synth.small_workload(moe_synth.WORKLOADS["ep32_zipf"],
                                                             T=300, E=16, k=4, n_src=1, n_dst=1))
    x = moe_synth.layer_inputs(wl, device="cuda", with_experts=False)["x"]
    plan = moe.moe_dispatch(x, idx.cuda(), 16)
    rows = 300 * 4
    y_disp = moe_synth.random_rows(wl, rows, device="cuda")
    y = moe.moe_combine(y_disp, plan["pair_slot"], w.cuda())
    part = moe.moe_combine_partial(y_disp, plan["pair_slot"], w.cuda(), 1, rows)
    y2 = moe.moe_combine_partials(part, plan["pair_slot"], 1, rows)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_partial_combine_zipf_full(gpu_lib):
    """32 x 128 Zipf workload, d=7168, random expert outputs: partial rows and the final
    sums against the oracle (bf16 payload), and the precision cost against the direct
    combine."""
    moe = gpu_lib
    wl = moe_synth.WORKLOADS["ep32_zipf"]
    _say(f"partial combine {wl}")
    idx, w = moe_synth.zipf_routing(wl)
    cap = wl.cap_rows_per_dst
    plan = moe.moe_dispatch(None, idx.cuda(), wl.E, layout=moe.Layout(wl.n_src, wl.n_dst, cap),
                            d=wl.d, dtype=torch.bfloat16)
    rows = wl.n_dst * cap
    rp = plan["row_pair"]
    live = torch.nonzero(rp >= 0).squeeze(1)
    y_disp = torch.zeros((rows, wl.d), dtype=torch.bfloat16, device="cuda")
    y_disp[live] = moe_synth.random_rows(wl, live.numel(), device="cuda")
    part = moe.moe_combine_partial(y_disp, plan["pair_slot"], w.cuda(), wl.n_dst, cap)
    y = moe.moe_combine_partials(part, plan["pair_slot"], wl.n_dst, cap)
    y_direct = moe.moe_combine(y_disp, plan["pair_slot"], w.cuda())
    torch.cuda.synchronize()
    ps = plan["pair_slot"].cpu().numpy()
    dests = ps // cap
    n_pairs = sum(len(set(dests[t].tolist())) for t in range(wl.T))
    _say(f"  return rows: {n_pairs} partial vs {wl.T * wl.k} per-expert")
    # every token against the oracle, in chunks of C tokens: a chunk's rows go to a
    # compact region layout whose regions each hold, packed in (token, j) order, the
    # chunk's rows of that destination (cap' = the fullest region's count), so the
    # oracle sees the same destinations and gates per token
    yd_live = _np(y_disp[live].cpu())
    live_np = live.cpu().numpy()
    compact = np.searchsorted(live_np, ps)
    assert np.array_equal(live_np[compact], ps)
    got_all = part.view(wl.n_dst, wl.T, wl.d)
    ref_rows, got_rows, ref_y = [], [], np.zeros((wl.T, wl.d))
    C = 64
    for t0 in range(0, wl.T, C):
        t1 = min(wl.T, t0 + C)
        dc = dests[t0:t1]
        cap_c = int(np.bincount(dc.ravel(), minlength=wl.n_dst).max())
        small = np.zeros((wl.n_dst * cap_c, wl.d), dtype=np.float32)
        slot = np.zeros((t1 - t0, wl.k), dtype=np.int64)
        fill = np.zeros(wl.n_dst, dtype=np.int64)
        for t in range(t0, t1):
            for j in range(wl.k):
                r = dc[t - t0, j]
                slot[t - t0, j] = r * cap_c + fill[r]
                fill[r] += 1
                small[slot[t - t0, j]] = yd_live[compact[t, j]]
        p1, pr1 = oracle.combine_partial(small, slot, w.numpy()[t0:t1], wl.n_dst, cap_c)
        ref_y[t0:t1] = oracle.combine_from_partials(_bf16(p1), pr1)
        ref_rows.append(p1[pr1])
        got_rows.append(_np(got_all[:, t0:t1][torch.from_numpy(pr1).cuda()]))
    err_p = oracle.normwise_rel_err(np.concatenate(got_rows), np.concatenate(ref_rows))
    err_y = oracle.normwise_rel_err(_np(y), ref_y)
    cost = oracle.normwise_rel_err(_np(y), _np(y_direct))
    _say(f"  partial err {err_p:.2e}, sum err {err_y:.2e}, vs direct combine {cost:.2e}")
    assert err_p <= BF16_TOL and err_y <= BF16_TOL and cost <= BF16_TOL
    del plan, y_disp, part
    torch.cuda.empty_cache()
