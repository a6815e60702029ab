"""GPU parity of the router on exactly equal logits, where the tie-break decides the
selection: equal float32 logits go to the lower expert id first, and the selection is
listed in descending logit order. Three constructions make ties on purpose:

* an all-zero router: every logit is +0, so every token takes experts 0..k-1 with
  gates 1/k;
* duplicated router rows: w[2i+1] = w[2i], so every logit value occurs twice and an odd
  k splits a pair at the k-th place;
* integer-valued x in {-1, 0, 1} and w in {-1, 0, 1}: integer logits in [-d, d], many
  equal within each token.

Every router kernel is covered: the 4x4x1 matrix-core chains (E <= 64), the 16x16x1
chains (E > 64, and the 16-token form above 512 experts) and the float32 vector-ALU
kernel. Indices and logits are compared bit for bit with the oracle, gates within 1e-5."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5


def _say(msg):
    print(msg, flush=True)


def _x(T, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((T, d), generator=g).to(dtype)


def _check(moe, x, w, k, label):
    _say(f"ties {label}: T={x.shape[0]} d={x.shape[1]} E={w.shape[0]} k={k} {x.dtype}")
    idx, gates, logits = moe.moe_route(x.cuda(), w.cuda(), k, want_logits=True)
    torch.cuda.synchronize()
    ref_logits, ref_idx, ref_g = oracle.route(x, w, k)
    got = logits.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref_logits.view(np.uint32)), "logits differ"
    # the construction really has ties at the selection boundary somewhere
    gap = oracle.topk_gap(ref_logits, k) if k < w.shape[0] else np.ones(1)
    _say(f"  tokens with a tie at the k-th place: {int((gap == 0).sum())}")
    assert np.array_equal(idx.cpu().numpy(), ref_idx), "indices differ"
    assert oracle.normwise_rel_err(gates.cpu().numpy(), ref_g) <= F32_TOL
    return ref_idx, ref_g, gap


CASES = [(1000, 256, 64, 6, torch.bfloat16), (333, 512, 384, 8, torch.bfloat16),
         (70, 128, 1024, 8, torch.bfloat16), (129, 64, 8, 2, torch.float32),
         (100, 128, 300, 7, torch.float32)]


@pytest.mark.parametrize("T,d,E,k,dt", CASES, ids=[f"{c[0]}x{c[1]}-E{c[2]}-k{c[3]}-{c[4]}" for c in CASES])
def test_all_zero_router(gpu_lib, T, d, E, k, dt):
    x = _x(T, d, dt, 1)
    w = torch.zeros((E, d), dtype=dt)
    ref_idx, ref_g, _ = _check(gpu_lib, x, w, k, "zero router")
    assert (ref_idx == np.arange(k)[None, :]).all()
    assert np.allclose(ref_g, 1.0 / k)


@pytest.mark.parametrize("T,d,E,k,dt", CASES, ids=[f"{c[0]}x{c[1]}-E{c[2]}-k{c[3]}-{c[4]}" for c in CASES])
@pytest.mark.parametrize("odd", [False, True])
def test_duplicated_router_rows(gpu_lib, T, d, E, k, dt, odd):
    if odd:
        k = k - 1 if k % 2 == 0 else k
    g = torch.Generator().manual_seed(E + k)
    half = (torch.randn((E // 2 + 1, d), generator=g) * 0.02).to(dt)
    w = half.repeat_interleave(2, dim=0)[:E].contiguous()
    x = _x(T, d, dt, 2)
    ref_idx, _, gap = _check(gpu_lib, x, w, max(k, 1), f"duplicated rows, k {'odd' if odd else 'even'}")
    # every pair of equal logits is listed lower id first
    sel = ref_idx
    if k % 2 == 1:
        assert (gap == 0).sum() == T                          # every token splits a pair
        assert (sel[:, -1] % 2 == 0).all()                   # ... and keeps its lower id


@pytest.mark.parametrize("T,d,E,k,dt", CASES, ids=[f"{c[0]}x{c[1]}-E{c[2]}-k{c[3]}-{c[4]}" for c in CASES])
def test_integer_logits(gpu_lib, T, d, E, k, dt):
    g = torch.Generator().manual_seed(T + d)
    x = torch.randint(-1, 2, (T, d), generator=g).to(dt)
    w = torch.randint(-1, 2, (E, d), generator=g).to(dt)
    _, _, gap = _check(gpu_lib, x, w, k, "integer logits")
    assert (gap == 0).sum() > 0
    # a row of x that is all zero gives +0 for every expert: experts 0..k-1
    x[0] = 0
    ref_idx, _, _ = _check(gpu_lib, x, w, k, "integer logits, zero token")
    assert (ref_idx[0] == np.arange(k)).all()
