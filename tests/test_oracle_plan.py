"""Pins for the oracle's dispatch plan (counts, offsets, slots) and dispatch copy.

Pinned by hand-worked examples (tests/golden/plan_examples.json), by the invariants
the EFA article's buffer design implies (counts sum to T*k; each sender's rows are
one contiguous chunk; a destination never receives more than N*T*max(R, E/N)
rows), and by an independent brute force (sorting the pairs) on small inputs.
"""
import json
import os

import numpy as np
import pytest

import oracle
import moe_synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "plan_examples.json")))["cases"],
                         ids=lambda c: c["name"])
def test_plan_golden(case):
    p = oracle.plan(np.array(case["idx"]), case["E"], case["n_src"], case["n_dst"], case["cap"])
    for key in ("counts", "expert_off", "chunk_off", "pair_slot", "row_pair"):
        assert p[key].tolist() == case[key], key


def _random_idx(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


def _brute_force_expert_major(idx, E):
    """Sort the (expert, token) keys of all pairs: row = position in the sorted list."""
    T, k = idx.shape
    keys = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k))
    slot = np.zeros((T, k), dtype=np.int64)
    for row, (_, t, j) in enumerate(keys):
        slot[t, j] = row
    return slot


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 3, 2), (50, 8, 2), (129, 16, 5), (300, 64, 6)])
def test_plan_expert_major_brute_force(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    idx = _random_idx(rng, T, E, k)
    p = oracle.plan(idx, E)
    assert np.array_equal(p["pair_slot"], _brute_force_expert_major(idx, E))
    counts = np.bincount(idx.ravel(), minlength=E)
    assert np.array_equal(p["counts"][0], counts)
    assert p["expert_off"][-1] == T * k and np.all(np.diff(p["expert_off"]) == counts)
    assert np.array_equal(np.sort(p["pair_slot"].ravel()), np.arange(T * k))
    assert np.array_equal(p["row_pair"][p["pair_slot"].ravel()], np.arange(T * k))


def _check_ep_invariants(p, idx, E, n_src, n_dst, cap):
    T, k = idx.shape
    Ts, epr = T // n_src, E // n_dst
    counts = p["counts"]
    assert counts.sum() == T * k
    for s in range(n_src):
        assert np.array_equal(counts[s], np.bincount(idx[s * Ts:(s + 1) * Ts].ravel(), minlength=E))
    # tight receive bound: a token sends at most min(k, E/N) rows to one destination
    tight = n_src * Ts * min(k, epr)
    slots = p["pair_slot"]
    rows_used = p["row_pair"] >= 0
    assert rows_used.sum() == T * k
    assert len(np.unique(slots)) == T * k
    for r in range(n_dst):
        live = p["chunk_off"][r, n_src]
        assert live <= tight <= cap
        region = rows_used[r * cap:(r + 1) * cap]
        assert region[:live].all() and not region[live:].any()   # packed, no gaps
    for t in range(T):
        s = t // Ts
        for j in range(k):
            e = int(idx[t, j])
            r = e // epr
            row = int(slots[t, j]) - r * cap
            lo, hi = p["chunk_off"][r, s], p["chunk_off"][r, s + 1]
            assert lo <= row < hi                       # inside sender s's one chunk
    # inside a chunk: expert-major, then ascending token
    for r in range(n_dst):
        for s in range(n_src):
            lo, hi = p["chunk_off"][r, s], p["chunk_off"][r, s + 1]
            keys = []
            for row in range(r * cap + lo, r * cap + hi):
                pr = int(p["row_pair"][row])
                keys.append((int(idx[pr // k, pr % k]), pr // k))
            assert keys == sorted(keys)


@pytest.mark.parametrize("n_src,n_dst,Ts,E,k", [(2, 2, 3, 4, 2), (4, 2, 16, 8, 3), (8, 4, 10, 32, 8),
                                                (3, 3, 5, 9, 1)])
def test_plan_ep_layout_invariants(n_src, n_dst, Ts, E, k):
    rng = np.random.default_rng(n_src * 7 + E)
    T = n_src * Ts
    idx = _random_idx(rng, T, E, k)
    cap = n_src * Ts * max(k, E // n_dst)
    p = oracle.plan(idx, E, n_src, n_dst, cap)
    _check_ep_invariants(p, idx, E, n_src, n_dst, cap)
    # the global expert offsets do not depend on the layout
    assert np.array_equal(p["expert_off"], oracle.plan(idx, E)["expert_off"])


def test_plan_ep_zipf_workload_invariants():
    wl = moe_synth.WORKLOADS["ep32_zipf"]
    idx, w = moe_synth.zipf_routing(wl)
    idx = idx.numpy()
    p = oracle.plan(idx, wl.E, wl.n_src, wl.n_dst, wl.cap_rows_per_dst)
    assert wl.cap_rows_per_dst == 49152
    _check_ep_invariants(p, idx, wl.E, wl.n_src, wl.n_dst, wl.cap_rows_per_dst)
    # Zipf: the destination holding the most popular experts receives the most rows
    live = p["chunk_off"][:, -1]
    assert live[0] == live.max() and live[0] > 4 * live.mean()


def test_plan_rejects_bad_indices():
    with pytest.raises(AssertionError):
        oracle.plan(np.array([[0, 4]]), 4)
    with pytest.raises(AssertionError):
        oracle.plan(np.array([[1, 1]]), 4)


def test_dispatch_copies_rows_bitwise():
    rng = np.random.default_rng(9)
    T, E, k, d = 40, 6, 3, 24
    idx = _random_idx(rng, T, E, k)
    x = rng.standard_normal((T, d)).astype(np.float32)
    p = oracle.plan(idx, E)
    xd = oracle.dispatch(x, p["pair_slot"], T * k)
    for t in range(T):
        for j in range(k):
            assert np.array_equal(xd[p["pair_slot"][t, j]].view(np.uint32), x[t].view(np.uint32))
    # every row is filled by exactly the token row_pair names
    assert np.array_equal(xd, x[p["row_pair"] // k])


# ------------------------------------------------------------ receive side (EP)
def test_ep_recv_plan_golden():
    """The hand-worked receive order of the 2-sender, 2-destination example."""
    case = json.load(open(os.path.join(GOLDEN, "plan_examples.json")))["cases"][1]
    p = oracle.plan(np.array(case["idx"]), case["E"], case["n_src"], case["n_dst"], case["cap"])
    for r in range(case["n_dst"]):
        off, src = oracle.ep_recv_plan(p["counts"], p["chunk_off"], r, case["n_dst"], case["cap"])
        assert off.tolist() == case["ep_recv"]["local_off"][r]
        assert src.tolist() == case["ep_recv"]["row_src"][r]


@pytest.mark.parametrize("T,E,k", [(40, 8, 2), (257, 16, 5)])
def test_ep_recv_plan_single_rank_is_identity(T, E, k):
    """One sender, one destination: the region already is expert-major."""
    rng = np.random.default_rng(T)
    idx = _random_idx(rng, T, E, k)
    p = oracle.plan(idx, E)
    off, src = oracle.ep_recv_plan(p["counts"], p["chunk_off"], 0, 1, p["cap"])
    assert np.array_equal(off, p["expert_off"])
    assert np.array_equal(src, np.arange(T * k))


def test_ep_recv_plan_matches_expert_major_layout():
    """At the 32 x 128 Zipf workload, every destination's reordered region holds
    exactly the pairs of its experts in the order of the plain expert-major layout
    (which plan() builds independently), and its live rows are a permutation of
    the region's live rows."""
    wl = moe_synth.WORKLOADS["ep32_zipf"]
    idx, _ = moe_synth.zipf_routing(wl)
    idx = np.asarray(idx)
    p_ep = oracle.plan(idx, wl.E, wl.n_src, wl.n_dst, wl.cap_rows_per_dst)
    p_em = oracle.plan(idx, wl.E)
    cap, epr = p_ep["cap"], wl.E // wl.n_dst
    em_pair_of_row = p_em["row_pair"]
    for r in range(wl.n_dst):
        off, src = oracle.ep_recv_plan(p_ep["counts"], p_ep["chunk_off"], r, wl.n_dst, cap)
        live = int(p_ep["chunk_off"][r, wl.n_src])
        assert off[-1] == live
        assert np.array_equal(np.sort(src[:live]), np.arange(live))
        assert np.all(src[live:] == -1)
        lo, hi = p_em["expert_off"][r * epr], p_em["expert_off"][(r + 1) * epr]
        assert np.array_equal(off, p_em["expert_off"][r * epr:(r + 1) * epr + 1] - lo)
        pairs_local = p_ep["row_pair"][r * cap + src[:live]]
        assert np.array_equal(pairs_local, em_pair_of_row[lo:hi])


# ------------------------------------------------------------ partial combine
def _bf16_round(a):
    import torch
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def test_combine_partial_golden():
    """The 2-sender, 2-destination example with y_disp row i = (i + 1) * ones(2) and
    gates 0.5 / 0.25 / ...: worked by hand from its pair_slot."""
    case = json.load(open(os.path.join(GOLDEN, "plan_examples.json")))["cases"][1]
    ps = np.array(case["pair_slot"])
    y_disp = np.repeat(np.arange(1, 25, dtype=np.float64)[:, None], 2, axis=1)
    g = np.tile([0.75, 0.25], (6, 1))
    partial, present = oracle.combine_partial(y_disp, ps, g, 2, case["cap"])
    # token 0: slots (2, 12) -> r=0 gets 0.75*3, r=1 gets 0.25*13
    assert partial[0, 0, 0] == 0.75 * 3 and partial[1, 0, 0] == 0.25 * 13
    # token 1: slots (0, 3) both at r=0: 0.75*1 + 0.25*4
    assert partial[0, 1, 0] == 0.75 * 1 + 0.25 * 4 and not present[1, 1]
    assert present.sum() == 10     # tokens 0, 2, 4, 5 split (2 each); 1 at r=0; 3 at r=1


@pytest.mark.parametrize("n_src,n_dst", [(1, 1), (4, 2), (2, 8)])
def test_combine_partial_unrounded_equals_combine(n_src, n_dst):
    """Without the payload rounding, summing partials is combine() reordered."""
    rng = np.random.default_rng(n_dst)
    T, E, k, d = 64, 16, 4, 8
    idx = _random_idx(rng, T, E, k)
    cap = n_src * (T // n_src) * max(k, E // n_dst)
    p = oracle.plan(idx, E, n_src, n_dst, cap)
    y_disp = rng.normal(size=(n_dst * cap, d))
    g = rng.uniform(0.1, 1, (T, k))
    partial, present = oracle.combine_partial(y_disp, p["pair_slot"], g, n_dst, cap)
    got = oracle.combine_from_partials(partial, present)
    ref = oracle.combine(y_disp, p["pair_slot"], g)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    dests = p["pair_slot"] // cap
    for t in range(T):
        assert set(np.nonzero(present[:, t])[0]) == set(dests[t].tolist())


def test_combine_partial_rounding_bound():
    """With bf16 payloads the sum moves by at most half an ulp per partial."""
    rng = np.random.default_rng(5)
    T, E, k, d, n_src, n_dst = 32, 8, 3, 16, 2, 4
    idx = _random_idx(rng, T, E, k)
    cap = n_src * (T // n_src) * max(k, E // n_dst)
    p = oracle.plan(idx, E, n_src, n_dst, cap)
    y_disp = rng.normal(size=(n_dst * cap, d))
    g = rng.uniform(0.1, 1, (T, k))
    exact, present = oracle.combine_partial(y_disp, p["pair_slot"], g, n_dst, cap)
    rounded, _ = oracle.combine_partial(y_disp, p["pair_slot"], g, n_dst, cap, _bf16_round)
    diff = np.abs(oracle.combine_from_partials(rounded, present)
                  - oracle.combine_from_partials(exact, present))
    bound = (np.abs(exact) * 2.0 ** -8).sum(axis=0)
    assert np.all(diff <= bound + 1e-300)
