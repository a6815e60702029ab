"""Pins for the oracle's expert FFN, combine, whole forward and backward (CPU only).

* E=1, k=1 reduces the layer to a dense SwiGLU FFN: checked against torch's CPU
  matmul and silu (library routines).
* identity experts with gates summing to one: combine(dispatch(x)) == x
  (the invariant the EFA article's dispatch/combine duality implies).
* the composed forward equals the per-token definition y[t] = sum_j g_j FFN_e(x[t]).
* backward: torch.autograd on a float64 re-expression of the layer, central finite
  differences of the expert FFN, and the zero row sums of the softmax Jacobian.
"""
import numpy as np
import pytest
import torch

import oracle
import moe_synth


def _small(name, **kw):
    return moe_synth.small_workload(moe_synth.WORKLOADS[name], **kw)


def test_dense_ffn_special_case_matches_torch():
    wl = _small("mid_bf16", T=37, d=64, E=1, k=1, F=48)
    inp = moe_synth.layer_inputs(wl)
    f = oracle.forward(inp["x"], inp["w_router"], inp["w13"], inp["w2"], 1)
    x, w13, w2 = (inp[n].double() for n in ("x", "w13", "w2"))
    ref = torch.nn.functional.silu(x @ w13[0, :48].T) * (x @ w13[0, 48:].T) @ w2[0].T
    assert np.allclose(f["gates"], 1.0)
    assert oracle.normwise_rel_err(f["y"], ref.numpy()) < 1e-13


def test_identity_experts_combine_dispatch_is_identity():
    wl = _small("mid_bf16", T=300, d=96, E=16, k=4)
    inp = moe_synth.layer_inputs(wl, with_experts=False)
    logits, idx, gates = oracle.route(inp["x"], inp["w_router"], wl.k)
    p = oracle.plan(idx, wl.E)
    xd = oracle.dispatch(inp["x"], p["pair_slot"], wl.pairs)
    y = oracle.combine(xd, p["pair_slot"], gates)
    x = inp["x"].double().numpy()
    assert np.max(np.abs(y - x)) <= 4 * 2.0 ** -52 * np.max(np.abs(x))
    # rounded to the storage dtype it is bit-exact
    assert torch.equal(torch.from_numpy(y).to(torch.bfloat16), inp["x"])


@pytest.mark.parametrize("name,kw", [("tiny_f32", {}), ("mid_bf16", dict(T=64, d=96, E=8, k=3, F=40))])
def test_forward_equals_per_token_definition(name, kw):
    wl = _small(name, **kw)
    inp = moe_synth.layer_inputs(wl)
    f = oracle.forward(inp["x"], inp["w_router"], inp["w13"], inp["w2"], wl.k)
    idx, gates, y = oracle.forward_tokens(inp["x"], inp["w_router"], wl.k,
                                          lambda e: (inp["w13"][e], inp["w2"][e]))
    assert np.array_equal(idx, f["idx"])
    assert np.array_equal(gates, f["gates"])
    assert oracle.normwise_rel_err(f["y"], y) < 1e-13
    # every expert's segment holds only its tokens
    for e in range(wl.E):
        a, b = f["expert_off"][e], f["expert_off"][e + 1]
        toks = f["row_pair"][a:b] // wl.k
        assert all(e in f["idx"][t] for t in toks)


def _torch_layer(x, wr, w13, w2, idx, F):
    """Float64 re-expression with torch ops (routing choice fixed by idx)."""
    logits = x @ wr.T
    g = torch.softmax(torch.gather(logits, 1, idx), dim=1)
    y = torch.zeros_like(x)
    for t in range(x.shape[0]):
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            h = x[t] @ w13[e, :F].T
            u = x[t] @ w13[e, F:].T
            y[t] = y[t] + g[t, j] * ((torch.nn.functional.silu(h) * u) @ w2[e].T)
    return y


def test_backward_matches_autograd():
    wl = _small("mid_bf16", T=12, d=16, E=5, k=2, F=10, dtype="f32")
    inp = moe_synth.layer_inputs(wl)
    dy = moe_synth.upstream_grad(wl)
    b = oracle.backward(inp["x"], inp["w_router"], inp["w13"], inp["w2"], dy, wl.k)
    leaves = {n: inp[n].double().requires_grad_(True) for n in ("x", "w_router", "w13", "w2")}
    y = _torch_layer(leaves["x"], leaves["w_router"], leaves["w13"], leaves["w2"],
                     torch.from_numpy(b["idx"].astype(np.int64)), wl.F)
    # the oracle's gates come from float32 logits, autograd's from float64 logits:
    # they differ by float32 rounding (~1e-7 relative); a wrong term would be O(1)
    assert oracle.normwise_rel_err(b["y"], y.detach().numpy()) < 1e-6
    (y * dy.double()).sum().backward()
    for mine, name in (("dx", "x"), ("dw_router", "w_router"), ("dw13", "w13"), ("dw2", "w2")):
        err = oracle.normwise_rel_err(b[mine], leaves[name].grad.numpy())
        assert err < 1e-6, (mine, err)


def test_route_bwd_jacobian_rows_sum_to_zero():
    rng = np.random.default_rng(11)
    g = rng.random((20, 6)) + 0.1
    g /= g.sum(axis=1, keepdims=True)
    dg = rng.standard_normal((20, 6))
    x = rng.standard_normal((20, 8))
    w = rng.standard_normal((10, 8))
    idx = np.stack([rng.permutation(10)[:6] for _ in range(20)])
    dl, dwr, dxr = oracle.route_bwd(x, w, idx, g, dg)
    assert np.allclose(dl.sum(axis=1), 0.0, atol=1e-15)
    # adding a constant to the upstream gate gradient changes nothing (sum g = 1)
    dl2, _, _ = oracle.route_bwd(x, w, idx, g, dg + 3.0)
    assert np.allclose(dl, dl2, atol=1e-14)


def test_expert_bwd_finite_differences():
    rng = np.random.default_rng(12)
    M, d, F = 5, 7, 4
    x = rng.standard_normal((M, d))
    w13 = 0.5 * rng.standard_normal((2 * F, d))
    w2 = 0.5 * rng.standard_normal((d, F))
    do = rng.standard_normal((M, d))
    dx, dw13, dw2 = oracle.swiglu_expert_bwd(x, do, w13, w2)
    loss = lambda x_, a_, b_: float(np.sum(do * oracle.swiglu_expert(x_, a_, b_)))
    h = 1e-6
    for arr, grad, pos in ((x, dx, (2, 3)), (w13, dw13, (1, 5)), (w13, dw13, (F + 2, 0)),
                           (w2, dw2, (6, 3))):
        plus, minus = arr.copy(), arr.copy()
        plus[pos] += h
        minus[pos] -= h
        args_p = [x, w13, w2]
        args_m = [x, w13, w2]
        which = 0 if arr is x else (1 if arr is w13 else 2)
        args_p[which], args_m[which] = plus, minus
        fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert abs(fd - grad[pos]) < 1e-7 * max(1.0, abs(fd)), (pos, fd, grad[pos])
