"""Oracle: a plain, slow, obviously correct CPU implementation of the MoE layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
package; only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` do. It shares no code with the GPU library (no kernels, headers,
helpers or tables); both sides only share the seeded input generators.

What is computed, and where it is defined. [EFA] below is Perplexity, "Enabling
trillion-parameter models on AWS EFA" (N. Licker, K. Hu, V. Zaytsev, L. Chen,
2025-11-04); section names are those of its table of contents.

* router logits   a small linear layer scores each token against each expert
                  ([EFA] Introduction). fp32, canonical order (see router_logits.c).
* top-k gating    every token goes to R (= k) of the E experts ([EFA] Send and receive
                  buffers); the model hands dispatch the tokens and their per-token
                  experts ([EFA] MoE all-to-all over EFA). The gating function is not
                  on the pages; reading used: softmax over the k selected logits
                  (equivalently the full softmax renormalised over the selection).
                  Ties: equal logits -> lower expert id first; output in descending
                  logit order.
* plan            per-expert token counts, their cumulative sum as offsets into
                  contiguous per-destination send buffers ([EFA] Dispatch and
                  combine). Order inside one expert's segment: ascending token id
                  (the article's atomics leave it open; a stable order is the reading).
* dispatch        copy each token into the slot of each of its experts, so that the
                  grouped GEMM sees expert-contiguous rows ([EFA] Dispatch and combine,
                  receiver side).
* expert FFN      grouped GEMM of each expert's rows with that expert's weights
                  ([EFA] MoE all-to-all over EFA). Expert form (not on the pages):
                  SwiGLU, o = (silu(x W1^T) * (x W3^T)) W2^T, no biases.
* combine         each token's expert outputs return to it and are averaged with the
                  gate weights: y[t] = sum_j g[t,j] o[slot(t,j)], accumulated at the
                  receiver ([EFA] Introduction; Dispatch and combine; Dispatch/combine
                  latency).
* receive order   a destination's region (one chunk per sender) reordered so that each
                  local expert's rows are contiguous before its grouped GEMM ([EFA]
                  Dispatch and combine, receiver side); senders ascending inside an
                  expert (a stable reading: the pages leave the order open).
* partial combine destinations sum each token's gate-weighted outputs before the
                  return; one row per (token, destination) travels back.
* backward        the transposes of the above, and the softmax-over-top-k Jacobian.

Precision: everything is float64 except the router logits, which decide integers and
are therefore computed in the same float32 canonical order as the GPU library.
Inputs arrive as float32 arrays holding the stored values (bf16 widens exactly).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "_liboracle.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(path)
        lib.oracle_router_logits_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_router_logits_f32.restype = None
        lib.oracle_num_threads.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def num_threads() -> int:
    """Host threads the oracle's C routine runs on (OpenMP)."""
    return int(_lib().oracle_num_threads())


def _f32(a) -> np.ndarray:
    if hasattr(a, "detach"):          # a torch tensor: widen to float32 exactly
        a = a.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        return a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- route
def router_logits(x, w_router) -> np.ndarray:
    """logit[t,e] = sum_i x[t,i] w[e,i], float32, fused multiply-add in index order."""
    x = _f32(x)
    w = _f32(w_router)
    T, d = x.shape
    E, d2 = w.shape
    assert d == d2
    out = np.empty((T, E), dtype=np.float32)
    _lib().oracle_router_logits_f32(x.ctypes.data, w.ctypes.data, T, d, E, out.ctypes.data)
    return out


def topk_gating(logits: np.ndarray, k: int, renorm: bool = True):
    """Select the k largest logits of each token and their gate weights.

    Returns (idx int32 [T,k], gates float64 [T,k]). idx is in descending logit order
    with ties going to the lower expert id. Gates: softmax over the k selected
    logits (renorm=True), else the full softmax's probabilities of the selected.
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    assert 1 <= k <= E
    # stable sort of the negated logits: descending logit, lower id first on ties
    order = np.argsort(-logits, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, idx, axis=1).astype(np.float64)
    if renorm:
        z = np.exp(sel - sel[:, :1])          # sel[:, 0] is the largest
        gates = z / z.sum(axis=1, keepdims=True)
    else:
        full = logits.astype(np.float64)
        zf = np.exp(full - full.max(axis=1, keepdims=True))
        p = zf / zf.sum(axis=1, keepdims=True)
        gates = np.take_along_axis(p, idx, axis=1)
    return idx, gates


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the gap between its k-th and (k+1)-th largest logit (float64; +inf
    when k == E). A token whose gap is below the rounding error of a reordered sum
    could change its selection if the logits were summed in another order, which is
    why the router fixes one order (the near-tie audit counts such tokens)."""
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    assert 1 <= k <= E
    if k == E:
        return np.full(T, np.inf)
    srt = -np.sort(-logits, axis=1)
    return srt[:, k - 1] - srt[:, k]


def route(x, w_router, k: int, renorm: bool = True):
    logits = router_logits(x, w_router)
    idx, gates = topk_gating(logits, k, renorm)
    return logits, idx, gates


# --------------------------------------------------------------------------- plan
def plan(idx, E: int, n_src: int = 1, n_dst: int = 1, cap_rows_per_dst: int | None = None):
    """Where each (token, expert) pair goes.

    Tokens are split into n_src equal consecutive groups (source ranks); experts into
    n_dst equal consecutive groups (destination ranks, expert e on rank e // (E/n_dst)).
    Destination r owns rows [r*cap, (r+1)*cap). Inside it, each sender's rows form one
    contiguous chunk (one write per peer), chunks in sender order; inside a chunk, the
    sender's pairs are grouped by expert (cumulative sum of its per-expert counts), and
    inside an expert by ascending token id. With n_src = n_dst = 1 and cap = T*k this
    is the plain expert-major layout whose expert e occupies rows
    [expert_off[e], expert_off[e+1]).

    Returns a dict of int64 arrays:
      counts     [n_src, E]       pairs of sender s routed to expert e
      expert_off [E+1]            exclusive cumulative sum of the per-expert totals
      chunk_off  [n_dst, n_src+1] offset of sender s's chunk inside destination r
      pair_slot  [T, k]           row of pair (t, j)
      row_pair   [n_dst*cap]      t*k + j of the pair in each row, -1 if unused
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    assert T % n_src == 0 and E % n_dst == 0
    Ts = T // n_src
    epr = E // n_dst
    if cap_rows_per_dst is None:
        cap_rows_per_dst = T * k if (n_src == 1 and n_dst == 1) else n_src * Ts * max(k, epr)
    cap = int(cap_rows_per_dst)
    for t in range(T):
        row = [int(e) for e in idx[t]]
        assert all(0 <= e < E for e in row), f"expert id out of range at token {t}"
        assert len(set(row)) == k, f"token {t} lists an expert twice"

    counts = np.zeros((n_src, E), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            counts[t // Ts, idx[t, j]] += 1
    totals = counts.sum(axis=0)
    expert_off = np.zeros(E + 1, dtype=np.int64)
    expert_off[1:] = np.cumsum(totals)

    chunk = np.zeros((n_src, n_dst), dtype=np.int64)       # rows sender s sends to r
    for s in range(n_src):
        for e in range(E):
            chunk[s, e // epr] += counts[s, e]
    chunk_off = np.zeros((n_dst, n_src + 1), dtype=np.int64)
    for r in range(n_dst):
        for s in range(n_src):
            chunk_off[r, s + 1] = chunk_off[r, s] + chunk[s, r]
        assert chunk_off[r, n_src] <= cap, "destination region over capacity"

    # first row of (sender s, expert e) inside its chunk: experts of the same
    # destination with a lower id come first
    within = np.zeros((n_src, E), dtype=np.int64)
    for s in range(n_src):
        for e in range(E):
            first = (e // epr) * epr
            within[s, e] = counts[s, first:e].sum()

    pair_slot = np.zeros((T, k), dtype=np.int64)
    row_pair = np.full(n_dst * cap, -1, dtype=np.int64)
    seen = np.zeros((n_src, E), dtype=np.int64)            # running rank, token order
    for t in range(T):
        s = t // Ts
        for j in range(k):
            e = int(idx[t, j])
            r = e // epr
            row = r * cap + chunk_off[r, s] + within[s, e] + seen[s, e]
            seen[s, e] += 1
            pair_slot[t, j] = row
            row_pair[row] = t * k + j
    return {"counts": counts, "expert_off": expert_off, "chunk_off": chunk_off,
            "pair_slot": pair_slot, "row_pair": row_pair, "cap": cap}


# ------------------------------------------------- block-scaled fp8 dispatch payload
# [EFA] evaluation: dispatch carries block-scaled fp8, combine stays bf16. The pages do
# not fix the format; reading used: OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7,
# 3 mantissa bits; largest finite value 448, no infinities, S.1111.111 is NaN), blocks
# of 128 consecutive hidden elements of a row, one float32 scale per block equal to the
# block's largest magnitude over 448, codes = E4M3(x * (448 / largest magnitude)) (the
# reciprocal rounded to float32 once per block, the product once per element) rounded
# to nearest even and saturated at +-448; an all-zero block has scale 0 and zero codes.
E4M3_MAX = 448.0
FP8_BLOCK = 128


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code, straight from the field definitions (float32)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return (sign * val).astype(np.float32)


def e4m3_encode(v) -> np.ndarray:
    """float32 values -> E4M3 codes, round to nearest even, saturating at +-448.
    Exact: for float32 inputs every step below is exact in float64."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    sgn = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    a = np.abs(v)
    # subnormal range [0, 2^-6): steps of 2^-9; a rounded 8 is the first normal code
    sub = np.rint(a * 2.0 ** 9).astype(np.int64)
    # normal range: a = f * 2^ex with f in [0.5, 1), so a = (2f) * 2^(ex-1), 2f in [1, 2)
    f, ex = np.frexp(a)
    e = ex.astype(np.int64) - 1
    q = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 0, q)
    nrm = np.minimum(((e + 7) << 3) | q, 0x7E)
    code = np.where(a < 2.0 ** -6, sub, nrm)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    return (sgn | code).astype(np.uint8)


def quantize_blocks_fp8(x, block: int = FP8_BLOCK):
    """Per row, per block of `block` elements with m = max|x|: scale = m / 448 and
    codes = E4M3(x * (448 / m)), every operation in float32 with one rounding.
    Returns (codes uint8 [T,d], scales f32 [T,d/block])."""
    x = _f32(x)
    T, d = x.shape
    assert d % block == 0
    xb = x.reshape(T, d // block, block)
    amax = np.abs(xb).max(axis=2).astype(np.float32)
    scales = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    inv = (np.float32(E4M3_MAX) / safe).astype(np.float32)
    ratio = (xb * inv[:, :, None]).astype(np.float32)
    codes = e4m3_encode(ratio)
    codes[amax == 0] = 0
    return codes.reshape(T, d), scales


def dequantize_blocks_fp8(codes, scales, block: int = FP8_BLOCK) -> np.ndarray:
    """value = decode(code) * scale, in float32 (one rounding)."""
    codes = np.asarray(codes, dtype=np.uint8)
    T, d = codes.shape
    vals = e4m3_decode(codes).reshape(T, d // block, block)
    return (vals * np.asarray(scales, dtype=np.float32)[:, :, None]).astype(np.float32).reshape(T, d)


# ------------------------------------------------------ receive side (emulated EP)
def ep_recv_plan(counts, chunk_off, r: int, n_dst: int, cap: int):
    """Destination r's receive region in expert-major order.

    [EFA] Dispatch and combine: the receiver moves the tokens it got into the tensor
    the grouped GEMM consumes; [EFA] Send and receive buffers: each sender's rows sit
    in one contiguous chunk of the destination's region. Inside sender s's chunk
    (at chunk_off[r, s]) the rows of the destination's experts follow each other in
    ascending expert id, each block in the sender's own (ascending token) order, as
    written by plan(). The local order lists local expert le = e - r*epr ascending,
    inside it the senders ascending, inside those the sender's order.

    Returns local_off [epr+1] (exclusive cumulative sum of the local experts' row
    totals) and row_src [cap]: for local row j < local_off[epr], the row of the
    region (0-based inside destination r) it comes from; -1 for the rest.
    """
    counts = np.asarray(counts, dtype=np.int64)
    chunk_off = np.asarray(chunk_off, dtype=np.int64)
    n_src, E = counts.shape
    epr = E // n_dst
    local_off = np.zeros(epr + 1, dtype=np.int64)
    row_src = []
    for le in range(epr):
        e = r * epr + le
        for s in range(n_src):
            # rows of sender s for expert e: after its rows for the lower local experts
            start = chunk_off[r, s] + counts[s, r * epr:e].sum()
            for i in range(counts[s, e]):
                row_src.append(int(start + i))
        local_off[le + 1] = len(row_src)
    assert len(row_src) <= cap
    out = np.full(cap, -1, dtype=np.int64)
    out[:len(row_src)] = row_src
    return local_off, out


# ------------------------------------------------- partial combine (rank-major layout)
def combine_partial(y_disp, pair_slot, gates, n_dst: int, cap: int, round_to=None):
    """Partial sums at the destinations: for token t and destination r holding rows of t
    (rows [r*cap, (r+1)*cap)), partial[r, t] = sum over those j of g[t,j] y_disp[slot],
    float64 in j order, then rounded by round_to (the return payload's precision; None
    keeps float64). The article accumulates at the combine's receiver only ([EFA]
    Dispatch/combine latency); summing at the destinations first is the variant that
    sends one row per (token, destination). Returns (partial [n_dst, T, d], present
    [n_dst, T] bool)."""
    y_disp = _f64(y_disp)
    pair_slot = np.asarray(pair_slot, dtype=np.int64)
    gates = np.asarray(gates, dtype=np.float64)
    T, k = pair_slot.shape
    d = y_disp.shape[1]
    partial = np.zeros((n_dst, T, d), dtype=np.float64)
    present = np.zeros((n_dst, T), dtype=bool)
    for t in range(T):
        for j in range(k):
            s = int(pair_slot[t, j])
            if s < 0 or s >= n_dst * cap:
                continue
            r = s // cap
            partial[r, t] += gates[t, j] * y_disp[s]
            present[r, t] = True
    if round_to is not None:
        partial = round_to(partial)
    return partial, present


def combine_from_partials(partial, present) -> np.ndarray:
    """y[t] = sum over the destinations r with rows of t, r ascending, of partial[r, t]."""
    partial = np.asarray(partial, dtype=np.float64)
    n_dst, T, d = partial.shape
    y = np.zeros((T, d), dtype=np.float64)
    for r in range(n_dst):
        y += np.where(np.asarray(present)[r][:, None], partial[r], 0.0)
    return y


# ----------------------------------------------------------------------- dispatch
def dispatch(x, pair_slot, rows_total: int) -> np.ndarray:
    """x_disp[pair_slot[t,j]] = x[t] (a copy of the stored values); unused rows 0."""
    x = _f32(x)
    pair_slot = np.asarray(pair_slot, dtype=np.int64)
    T, k = pair_slot.shape
    out = np.zeros((rows_total, x.shape[1]), dtype=np.float32)
    for j in range(k):
        out[pair_slot[:, j]] = x
    return out


# --------------------------------------------------------------------- expert FFN
def silu(z):
    return z / (1.0 + np.exp(-z))


def swiglu_expert(xr, w13_e, w2_e):
    """One expert on rows xr [M,d]: (silu(xr W1^T) * (xr W3^T)) W2^T, float64.
    w13_e [2F,d] (rows 0..F-1 = W1, F..2F-1 = W3), w2_e [d,F]."""
    xr = np.asarray(xr, dtype=np.float64)
    w13_e = _f64(w13_e)
    w2_e = _f64(w2_e)
    F = w13_e.shape[0] // 2
    h = xr @ w13_e[:F].T
    u = xr @ w13_e[F:].T
    return (silu(h) * u) @ w2_e.T


def expert_ffn(x_disp, expert_off, w13, w2) -> np.ndarray:
    """Grouped GEMM: rows [expert_off[e], expert_off[e+1]) through expert e."""
    x_disp = _f64(x_disp)
    expert_off = np.asarray(expert_off, dtype=np.int64)
    E = len(expert_off) - 1
    d = w2.shape[1]
    out = np.zeros((x_disp.shape[0], d), dtype=np.float64)
    for e in range(E):
        a, b = int(expert_off[e]), int(expert_off[e + 1])
        if b > a:
            out[a:b] = swiglu_expert(x_disp[a:b], w13[e], w2[e])
    return out


# ------------------------------------------------------------------------ combine
def combine(y_disp, pair_slot, gates) -> np.ndarray:
    """y[t] = sum_j gates[t,j] * y_disp[pair_slot[t,j]], float64, j in order."""
    y_disp = _f64(y_disp)
    pair_slot = np.asarray(pair_slot, dtype=np.int64)
    gates = np.asarray(gates, dtype=np.float64)
    T, k = pair_slot.shape
    y = np.zeros((T, y_disp.shape[1]), dtype=np.float64)
    for j in range(k):
        y += gates[:, j:j + 1] * y_disp[pair_slot[:, j]]
    return y


# ------------------------------------------------------------------------ forward
def forward(x, w_router, w13, w2, k: int, renorm: bool = True) -> dict:
    """The whole layer: route -> plan -> dispatch -> expert FFN -> combine."""
    E = w_router.shape[0]
    logits, idx, gates = route(x, w_router, k, renorm)
    p = plan(idx, E)
    x_disp = dispatch(x, p["pair_slot"], x.shape[0] * k)
    y_disp = expert_ffn(x_disp, p["expert_off"], w13, w2)
    y = combine(y_disp, p["pair_slot"], gates)
    return dict(logits=logits, idx=idx, gates=gates, x_disp=x_disp, y_disp=y_disp, y=y, **p)


def forward_tokens(x_rows, w_router, k: int, expert_weights, renorm: bool = True):
    """The layer for a few tokens, one at a time, straight from its definition:
    y[t] = sum_j g[t,j] * FFN_{idx[t,j]}(x[t]). ``expert_weights(e)`` returns
    (w13_e, w2_e). Returns (idx, gates, y float64 [n,d])."""
    _, idx, gates = route(x_rows, w_router, k, renorm)
    xr = _f64(x_rows)
    cache = {}
    y = np.zeros_like(xr)
    for n in range(xr.shape[0]):
        for j in range(k):
            e = int(idx[n, j])
            if e not in cache:
                cache[e] = expert_weights(e)
            w13_e, w2_e = cache[e]
            y[n] += gates[n, j] * swiglu_expert(xr[n:n + 1], w13_e, w2_e)[0]
    return idx, gates, y


# ----------------------------------------------------------------------- backward
def combine_bwd(dy, y_disp, pair_slot, gates, rows_total: int):
    """Transpose of combine: dy_disp[slot(t,j)] = g[t,j] dy[t];
    dgates[t,j] = <dy[t], y_disp[slot(t,j)]>."""
    dy = _f64(dy)
    y_disp = _f64(y_disp)
    pair_slot = np.asarray(pair_slot, dtype=np.int64)
    gates = np.asarray(gates, dtype=np.float64)
    T, k = pair_slot.shape
    dy_disp = np.zeros((rows_total, dy.shape[1]), dtype=np.float64)
    dgates = np.zeros((T, k), dtype=np.float64)
    for j in range(k):
        dy_disp[pair_slot[:, j]] = gates[:, j:j + 1] * dy
        dgates[:, j] = np.sum(dy * y_disp[pair_slot[:, j]], axis=1)
    return dy_disp, dgates


def swiglu_expert_bwd(xr, do, w13_e, w2_e):
    """Gradients of one SwiGLU expert. Returns (dx [M,d], dw13 [2F,d], dw2 [d,F])."""
    xr = np.asarray(xr, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    w13_e = _f64(w13_e)
    w2_e = _f64(w2_e)
    F = w13_e.shape[0] // 2
    w1, w3 = w13_e[:F], w13_e[F:]
    h = xr @ w1.T
    u = xr @ w3.T
    sig = 1.0 / (1.0 + np.exp(-h))
    a = h * sig * u
    da = do @ w2_e                                   # [M,F]
    dw2 = do.T @ a                                   # [d,F]
    dh = da * u * sig * (1.0 + h * (1.0 - sig))      # silu'(h) = s (1 + h (1 - s))
    du = da * h * sig
    dx = dh @ w1 + du @ w3
    dw13 = np.concatenate([dh.T @ xr, du.T @ xr], axis=0)
    return dx, dw13, dw2


def expert_ffn_bwd(x_disp, dy_disp, expert_off, w13, w2):
    x_disp = _f64(x_disp)
    dy_disp = np.asarray(dy_disp, dtype=np.float64)
    expert_off = np.asarray(expert_off, dtype=np.int64)
    E = len(expert_off) - 1
    dx_disp = np.zeros_like(x_disp)
    dw13 = np.zeros(tuple(w13.shape), dtype=np.float64)
    dw2 = np.zeros(tuple(w2.shape), dtype=np.float64)
    for e in range(E):
        a, b = int(expert_off[e]), int(expert_off[e + 1])
        if b > a:
            dx_disp[a:b], dw13[e], dw2[e] = swiglu_expert_bwd(x_disp[a:b], dy_disp[a:b],
                                                              w13[e], w2[e])
    return dx_disp, dw13, dw2


def dispatch_bwd(dx_disp, pair_slot) -> np.ndarray:
    """Transpose of dispatch: dx[t] = sum_j dx_disp[pair_slot[t,j]]."""
    dx_disp = np.asarray(dx_disp, dtype=np.float64)
    pair_slot = np.asarray(pair_slot, dtype=np.int64)
    T, k = pair_slot.shape
    dx = np.zeros((T, dx_disp.shape[1]), dtype=np.float64)
    for j in range(k):
        dx += dx_disp[pair_slot[:, j]]
    return dx


def route_bwd(x, w_router, idx, gates, dgates):
    """Backward of softmax-over-top-k gating and the router's linear layer.

    For the selected logits, dl_i = g_i (dg_i - sum_j g_j dg_j); the selection
    itself is piecewise constant, so unselected logits get no gradient.
    Returns (dlogits_sel [T,k], dw_router [E,d], dx_router [T,d])."""
    x = _f64(x)
    w = _f64(w_router)
    idx = np.asarray(idx, dtype=np.int64)
    gates = np.asarray(gates, dtype=np.float64)
    dgates = np.asarray(dgates, dtype=np.float64)
    T, k = idx.shape
    E = w.shape[0]
    dl_sel = gates * (dgates - np.sum(gates * dgates, axis=1, keepdims=True))
    dL = np.zeros((T, E), dtype=np.float64)
    for j in range(k):
        dL[np.arange(T), idx[:, j]] += dl_sel[:, j]
    return dl_sel, dL.T @ x, dL @ w


def backward(x, w_router, w13, w2, dy, k: int) -> dict:
    """Forward, then all gradients of sum(dy * y) with respect to x, the router and
    the expert weights (renormalised gating)."""
    f = forward(x, w_router, w13, w2, k)
    rows = x.shape[0] * k
    dy_disp, dgates = combine_bwd(dy, f["y_disp"], f["pair_slot"], f["gates"], rows)
    dx_disp, dw13, dw2 = expert_ffn_bwd(f["x_disp"], dy_disp, f["expert_off"], w13, w2)
    dl_sel, dw_router, dx_router = route_bwd(x, w_router, f["idx"], f["gates"], dgates)
    dx = dispatch_bwd(dx_disp, f["pair_slot"]) + dx_router
    f.update(dy_disp=dy_disp, dgates=dgates, dx_disp=dx_disp, dw13=dw13, dw2=dw2,
             dlogits_sel=dl_sel, dw_router=dw_router, dx=dx)
    return f


# --------------------------------------------------------------- error measures
def normwise_rel_err(got, ref) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i| (0 for two empty arrays)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    diff = float(np.max(np.abs(got - ref)))
    return diff / scale if scale > 0 else diff


def elementwise_rel_err(got, ref) -> float:
    """max_i |got_i - ref_i| / (|ref_i| + rms(ref)) (0 for two empty arrays): the
    elementwise reading of a relative-error bar. The rms term keeps outputs near zero
    from dividing by almost nothing (every output here is a sum of many products, so
    some sit at zero by chance)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    den = np.abs(ref) + rms
    diff = np.abs(got - ref)
    if rms == 0.0:
        return float(np.max(diff))
    return float(np.max(diff / den))
