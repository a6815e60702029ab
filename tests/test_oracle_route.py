"""Pins for the oracle's router logits and top-k gating (CPU only).

Each pin is fixed by something other than the oracle itself: hand-derived float32
cases, exact integer arithmetic, a float64 error bound, exhaustive subset search,
and the k=2 closed form of the gates.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hex_arr(rows):
    return np.array([[float.fromhex(v) for v in r] for r in rows], dtype=np.float32)


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "router_order.json")))["cases"],
                         ids=lambda c: c["name"])
def test_router_golden_order(case):
    x, w, want = _hex_arr(case["x"]), _hex_arr(case["w"]), _hex_arr(case["logits"])
    got = oracle.router_logits(x, w)
    assert got.dtype == np.float32
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (got, want)


def test_router_one_hot_rows_select_columns():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((17, 40)).astype(np.float32)
    cols = np.array([3, 0, 39, 17, 3])
    w = np.zeros((5, 40), dtype=np.float32)
    w[np.arange(5), cols] = 1.0
    got = oracle.router_logits(x, w)
    assert np.array_equal(got, x[:, cols])


def test_router_integer_inputs_exact():
    rng = np.random.default_rng(2)
    x = rng.integers(-8, 9, size=(33, 64))
    w = rng.integers(-8, 9, size=(12, 64))
    got = oracle.router_logits(x.astype(np.float32), w.astype(np.float32))
    assert np.array_equal(got.astype(np.int64), x @ w.T)


def test_router_within_float64_error_bound():
    rng = np.random.default_rng(3)
    d = 2048
    x = rng.standard_normal((64, d)).astype(np.float32)
    w = (0.02 * rng.standard_normal((16, d))).astype(np.float32)
    got = oracle.router_logits(x, w).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    # sequential float32 summation: |err| <= d * 2^-24 * sum_i |x_i w_i| (first order)
    bound = d * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T)
    assert np.all(np.abs(got - ref) <= bound)


def _brute_force_topk(row, k):
    """The unique k-subset whose every member beats every non-member under the
    order (higher logit first, then lower id)."""
    E = len(row)
    beats = lambda a, b: (row[a] > row[b]) or (row[a] == row[b] and a < b)
    found = []
    for S in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in S]
        if all(beats(a, b) for a in S for b in rest):
            found.append(S)
    assert len(found) == 1
    return set(found[0])


def test_topk_exhaustive_small():
    rng = np.random.default_rng(4)
    for E in range(1, 7):
        for k in range(1, E + 1):
            logits = rng.integers(-2, 3, size=(4, E)).astype(np.float32)  # many ties
            idx, gates = oracle.topk_gating(logits, k)
            for t in range(4):
                assert set(idx[t].tolist()) == _brute_force_topk(logits[t], k)
                sel = logits[t, idx[t]]
                # descending logits, ties by ascending id
                for a in range(k - 1):
                    assert sel[a] > sel[a + 1] or (sel[a] == sel[a + 1] and idx[t, a] < idx[t, a + 1])
                assert math.isclose(gates[t].sum(), 1.0, rel_tol=0, abs_tol=1e-15)


def test_topk_ties_lower_id_first():
    logits = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]], dtype=np.float32)
    idx, gates = oracle.topk_gating(logits, 3)
    assert idx.tolist() == [[1, 2, 4]]
    assert np.allclose(gates, 1.0 / 3.0, rtol=0, atol=1e-15)
    # signed zeros compare equal: the lower id wins
    idx0, _ = oracle.topk_gating(np.array([[-0.0, 0.0, -1.0]], dtype=np.float32), 1)
    assert idx0.tolist() == [[0]]


def test_gates_k2_closed_form():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((50, 7)).astype(np.float32)
    idx, gates = oracle.topk_gating(logits, 2)
    l0 = logits[np.arange(50), idx[:, 0]].astype(np.float64)
    l1 = logits[np.arange(50), idx[:, 1]].astype(np.float64)
    g0 = 1.0 / (1.0 + np.exp(l1 - l0))
    assert np.allclose(gates[:, 0], g0, rtol=1e-14, atol=0)
    assert np.allclose(gates[:, 1], 1.0 - g0, rtol=1e-13, atol=1e-16)


def test_gates_are_renormalised_full_softmax():
    rng = np.random.default_rng(6)
    logits = (3 * rng.standard_normal((40, 11))).astype(np.float32)
    idx, g_renorm = oracle.topk_gating(logits, 4, renorm=True)
    idx2, g_full = oracle.topk_gating(logits, 4, renorm=False)
    assert np.array_equal(idx, idx2)
    full = np.exp(logits.astype(np.float64))
    full /= full.sum(axis=1, keepdims=True)
    assert np.allclose(g_full, np.take_along_axis(full, idx, 1), rtol=1e-13, atol=0)
    assert np.allclose(g_renorm, g_full / g_full.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)


def test_topk_gap_brute_force():
    """The k/(k+1) gap against an explicit enumeration of every logit's rank."""
    rng = np.random.default_rng(7)
    lg = rng.normal(0, 1, (50, 9)).astype(np.float32)
    lg[3, 2] = lg[3, 5]                      # an exact tie straddling the cut for some k
    for k in (1, 3, 8, 9):
        gap = oracle.topk_gap(lg, k)
        for t in range(lg.shape[0]):
            vals = sorted((float(v) for v in lg[t]), reverse=True)
            want = np.inf if k == lg.shape[1] else vals[k - 1] - vals[k]
            assert gap[t] == want, (t, k)
    assert np.all(oracle.topk_gap(lg, 3) >= 0)
