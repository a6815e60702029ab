"""Seeded synthetic inputs for the Mixture-of-Experts layer.

This module is shared by the oracle's tests, the GPU parity tests and the benchmark.
It holds none of the layer's arithmetic: it only draws random tensors of the right
shapes and value distributions, rounds the draws to the storage dtype, and (for the
expert-parallel emulation) draws routing decisions from a Zipf popularity law.

Workloads (shapes follow the models the evaluation of "Enabling trillion-parameter
models on AWS EFA" (Perplexity, 2025) serves: hidden size 7168, 384 experts,
8 experts per token; the smaller ones are scaled-down layers of the same form):

* ``tiny_f32``        T=64,   d=128,  E=8,   k=2, F=256,  fp32, forward
* ``mid_bf16``        T=4096, d=2048, E=64,  k=6, F=1408, bf16, forward
* ``large_bf16``      T=8192, d=7168, E=384, k=8, F=2048, bf16, forward (34 GB weights)
* ``ep32_zipf``       32 source ranks x 128 tokens, d=7168, E=384, k=8, bf16,
                      Zipf(1.2) expert popularity, dispatch/combine only
* ``mid_bf16_train``  the ``mid_bf16`` shapes, forward + backward

Distributions: activations and upstream gradients ~ N(0, 1); router and expert
weights ~ N(0, 0.02^2) (standard deviation 0.02). Every tensor has its own generator
seeded from ``(seed, tensor id)``, so adding a tensor never changes another one.
Draws are made in float32 on the requested device and then rounded to the storage
dtype (bf16: round to nearest even, which is what ``Tensor.to`` does).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

__all__ = ["Workload", "WORKLOADS", "layer_inputs", "upstream_grad", "zipf_routing",
           "small_workload", "storage_dtype"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens (all source ranks together)
    d: int            # hidden size
    E: int            # experts
    k: int            # experts per token
    F: int            # expert FFN inner size (0: no expert FFN, dispatch/combine only)
    dtype: str        # "f32" or "bf16"
    n_src: int = 1    # source ranks (token groups); 1 = plain expert-major layout
    n_dst: int = 1    # destination ranks (expert groups)
    zipf_s: Optional[float] = None   # expert popularity exponent for given routing
    backward: bool = False
    seed: int = 0

    @property
    def pairs(self) -> int:
        return self.T * self.k

    @property
    def tokens_per_src(self) -> int:
        return self.T // self.n_src

    @property
    def cap_rows_per_dst(self) -> int:
        """Rows reserved per destination region: N*T*max(R, E/N) with T the tokens
        of one source rank ("Send and receive buffers" of the EFA article). For the
        single-region expert-major layout this is simply the number of pairs."""
        if self.n_dst == 1 and self.n_src == 1:
            return self.pairs
        return self.n_src * self.tokens_per_src * max(self.k, self.E // self.n_dst)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", T=64, d=128, E=8, k=2, F=256, dtype="f32"),
    "mid_bf16": Workload("mid_bf16", T=4096, d=2048, E=64, k=6, F=1408, dtype="bf16"),
    "large_bf16": Workload("large_bf16", T=8192, d=7168, E=384, k=8, F=2048, dtype="bf16"),
    "ep32_zipf": Workload("ep32_zipf", T=32 * 128, d=7168, E=384, k=8, F=0, dtype="bf16",
                          n_src=32, n_dst=32, zipf_s=1.2),
    "mid_bf16_train": Workload("mid_bf16_train", T=4096, d=2048, E=64, k=6, F=1408,
                               dtype="bf16", backward=True),
}


def small_workload(base: Workload, **changes) -> Workload:
    """A copy of ``base`` with some sizes changed (for oracle-sized parity cases)."""
    return dataclasses.replace(base, **changes)


def storage_dtype(wl: Workload) -> torch.dtype:
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


_TENSOR_IDS = {"x": 1, "w_router": 2, "w13": 3, "w2": 4, "dy": 5, "zipf": 6, "gates": 7,
               "y_disp": 8}


def _generator(seed: int, tensor: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + _TENSOR_IDS[tensor] * 7919) & 0x7FFF_FFFF_FFFF)
    return g


def _normal(shape, std: float, dtype, seed: int, tensor: str, device, chunks: int = 1):
    """Draw N(0, std^2) in float32, round to ``dtype``. ``chunks`` splits the first
    dimension so that no float32 temporary larger than one chunk is ever held."""
    g = _generator(seed, tensor, device)
    out = torch.empty(shape, dtype=dtype, device=device)
    n0 = shape[0]
    step = max(1, math.ceil(n0 / chunks))
    for s in range(0, n0, step):
        e = min(n0, s + step)
        blk = torch.randn((e - s,) + tuple(shape[1:]), generator=g, device=device,
                          dtype=torch.float32)
        if std != 1.0:
            blk.mul_(std)
        out[s:e].copy_(blk)
        del blk
    return out


def layer_inputs(wl: Workload, device="cpu", with_experts: bool = True) -> dict:
    """x [T,d], w_router [E,d], and (if the workload has an FFN) w13 [E,2F,d] (rows
    0..F-1 = gate projection W1, rows F..2F-1 = up projection W3) and w2 [E,d,F]."""
    dt = storage_dtype(wl)
    out = {
        "x": _normal((wl.T, wl.d), 1.0, dt, wl.seed, "x", device),
        "w_router": _normal((wl.E, wl.d), 0.02, dt, wl.seed, "w_router", device),
    }
    if with_experts and wl.F > 0:
        out["w13"] = _normal((wl.E, 2 * wl.F, wl.d), 0.02, dt, wl.seed, "w13", device,
                             chunks=wl.E)
        out["w2"] = _normal((wl.E, wl.d, wl.F), 0.02, dt, wl.seed, "w2", device,
                            chunks=wl.E)
    return out


def upstream_grad(wl: Workload, device="cpu") -> torch.Tensor:
    """dL/dy [T,d] ~ N(0,1) in the storage dtype."""
    return _normal((wl.T, wl.d), 1.0, storage_dtype(wl), wl.seed, "dy", device)


def random_rows(wl: Workload, rows: int, device="cpu") -> torch.Tensor:
    """[rows, d] ~ N(0,1): stand-in expert outputs for dispatch/combine-only runs."""
    return _normal((rows, wl.d), 1.0, storage_dtype(wl), wl.seed, "y_disp", device)


def zipf_routing(wl: Workload, device="cpu"):
    """Given routing for the expert-parallel emulation.

    Expert popularity p_e proportional to (e+1)^(-s) (expert 0 the most popular).
    Each token draws k distinct experts by sampling without replacement from p
    (Gumbel-top-k on log p). Its k weights are positive uniform draws scaled to sum
    to one. Returns (topk_idx int32 [T,k], topk_w float32 [T,k]).
    """
    assert wl.zipf_s is not None
    g = _generator(wl.seed, "zipf", device)
    logp = -wl.zipf_s * torch.log(torch.arange(1, wl.E + 1, device=device,
                                               dtype=torch.float64))
    u = torch.rand((wl.T, wl.E), generator=g, device=device, dtype=torch.float64)
    u = u.clamp_min(1e-300)
    keys = logp[None, :] - torch.log(-torch.log(u))
    idx = torch.topk(keys, wl.k, dim=1).indices.to(torch.int32)
    g2 = _generator(wl.seed, "gates", device)
    w = torch.rand((wl.T, wl.k), generator=g2, device=device, dtype=torch.float64) + 0.5
    w = (w / w.sum(dim=1, keepdim=True)).to(torch.float32)
    return idx.contiguous(), w.contiguous()
