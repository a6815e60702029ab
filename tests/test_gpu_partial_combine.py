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
    sample = np.arange(0, wl.T, 29)
    # the oracle per sampled token, on a compact copy of its k rows that keeps each
    # row's destination: row dest*k + j of a region layout with cap' = k
    yd_all = y_disp.cpu()
    ref_part = np.zeros((wl.n_dst, len(sample), wl.d))
    present = np.zeros((wl.n_dst, len(sample)), dtype=bool)
    for i, t in enumerate(sample):
        small = np.zeros((wl.n_dst * wl.k, wl.d), dtype=np.float32)
        slot = np.zeros((1, wl.k), dtype=np.int64)
        for j in range(wl.k):
            slot[0, j] = dests[t, j] * wl.k + j
            small[slot[0, j]] = _np(yd_all[ps[t, j]])
        p1, pr1 = oracle.combine_partial(small, slot, w.numpy()[t:t + 1], wl.n_dst, wl.k)
        ref_part[:, i], present[:, i] = p1[:, 0], pr1[:, 0]
    ref_y = oracle.combine_from_partials(_bf16(ref_part), present)
    got_part = part.view(wl.n_dst, wl.T, wl.d)[:, torch.from_numpy(sample).cuda()]
    mask = torch.from_numpy(present).cuda()
    err_p = oracle.normwise_rel_err(_np(got_part[mask]), ref_part[present])
    err_y = oracle.normwise_rel_err(_np(y[torch.from_numpy(sample).cuda()]), ref_y)
    cost = oracle.normwise_rel_err(_np(y), _np(y_direct))
    _say(f"  partial err {err_p:.2e}, sum err {err_y:.2e}, vs direct combine {cost:.2e}")
    assert err_p <= BF16_TOL and err_y <= BF16_TOL and cost <= BF16_TOL
    del plan, y_disp, part
    torch.cuda.empty_cache()
