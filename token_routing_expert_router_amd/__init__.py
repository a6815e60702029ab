"""Python binding of libmoe, the MI355X-native Mixture-of-Experts layer.

Argument marshalling only: every step of the layer runs in libmoe's HIP kernels.
Each function has the name of the C entry point it calls (declared in
include/moe.h); tensors are torch tensors on the GPU, and the call is enqueued on
torch's current stream. Outputs may be passed in; otherwise they are allocated
with torch (device memory is the one thing PyTorch provides here).

If libmoe.so is missing or fails to load, every call raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["MoEError", "load", "library_path", "moe_abi_version", "moe_workspace_size",
           "moe_route", "moe_dispatch",
           "moe_dispatch_status", "moe_dispatch_noalloc", "moe_expert_ffn", "moe_expert_ffn_gate_up",
           "moe_expert_ffn_down", "moe_combine", "moe_combine_bwd",
           "moe_expert_ffn_bwd", "moe_route_bwd", "moe_dispatch_bwd", "moe_ep_recv_plan",
           "moe_ep_recv_gather", "moe_ep_recv_scatter", "moe_dispatch_fp8",
           "moe_ep_recv_gather_fp8", "moe_combine_partial", "moe_combine_partials", "moe_combine_add",
           "forward_shared", "forward_microbatched", "forward_ep_split", "Layout", "forward",
           "backward",
           "EXPORTED"]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_ROUTE_RENORM, MOE_ROUTE_FULL_SOFTMAX = 0, 1
_STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_ALIGN",
           4: "MOE_ERR_CAPACITY", 5: "MOE_ERR_BAD_INDEX", 6: "MOE_ERR_HIP",
           7: "MOE_ERR_UNSUPPORTED"}

_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

# entry point -> (restype, argtypes); the same list include/moe.h declares
EXPORTED = {
    "moe_abi_version": (_I32, []),
    "moe_status_str": (ctypes.c_char_p, [_I32]),
    "moe_workspace_size": (_SZ, [_I32, _I64, _I32, _I32, _P, _I64, _I64, _I64, _I32]),
    "moe_route": (_I32, [_P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P]),
    "moe_dispatch_workspace_size": (_SZ, [_I64, _I32, _I32, _P]),
    "moe_dispatch": (_I32, [_P, _P, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P,
                            _P, _SZ, _P]),
    "moe_dispatch_status": (_I32, [_P, _P]),
    "moe_dispatch_noalloc": (_I32, [_P, _P, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P,
                                    _P, _P]),
    "moe_expert_ffn_workspace_size": (_SZ, [_I32, _I64, _I64, _I64, _I32]),
    "moe_expert_ffn": (_I32, [_P, _P, _P, _P, _I32, _I64, _I64, _I64, _I32, _P, _P, _P, _SZ,
                              _P]),
    "moe_expert_ffn_gate_up": (_I32, [_P, _P, _P, _I32, _I64, _I64, _I64, _I32, _P, _P, _P]),
    "moe_expert_ffn_down": (_I32, [_P, _P, _P, _I32, _I64, _I64, _I64, _I32, _P, _P]),
    "moe_combine": (_I32, [_P, _P, _P, _I64, _I32, _I64, _I64, _I32, _P, _P]),
    "moe_combine_bwd": (_I32, [_P, _P, _P, _P, _I64, _I32, _I64, _I64, _I32, _P, _P, _P]),
    "moe_expert_ffn_bwd_workspace_size": (_SZ, [_I32, _I64, _I64, _I64, _I32]),
    "moe_expert_ffn_bwd": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I32, _P, _P,
                                  _P, _P, _SZ, _P]),
    "moe_route_bwd": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _P, _P, _P]),
    "moe_dispatch_bwd": (_I32, [_P, _P, _P, _P, _P, _I64, _I32, _I64, _I32, _I64, _I32, _P,
                                _P]),
    "moe_dispatch_fp8": (_I32, [_P, _P, _I64, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                                _P, _SZ, _P]),
    "moe_ep_recv_gather_fp8": (_I32, [_P, _P, _P, _I64, _I64, _P, _P]),
    "moe_combine_add": (_I32, [_P, _P, _P, _I64, _I32, _I64, _I64, _I32, _P, _P, _P]),
    "moe_combine_partial": (_I32, [_P, _P, _P, _I64, _I32, _I64, _I32, _I64, _I32, _P, _P]),
    "moe_combine_partials": (_I32, [_P, _P, _I64, _I32, _I64, _I32, _I64, _I32, _P, _P]),
    "moe_ep_recv_plan": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I64, _P, _P, _P]),
    "moe_ep_recv_gather": (_I32, [_P, _P, _I64, _I64, _I32, _P, _P]),
    "moe_ep_recv_scatter": (_I32, [_P, _P, _I64, _I64, _I32, _P, _P]),
}


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)}")


class _Layout(ctypes.Structure):
    _fields_ = [("n_src", ctypes.c_int32), ("n_dst", ctypes.c_int32),
                ("cap_rows_per_dst", ctypes.c_int64)]


class Layout:
    """Where dispatched rows go (see moe_layout_t). None means expert-major."""

    def __init__(self, n_src: int, n_dst: int, cap_rows_per_dst: int):
        self.n_src, self.n_dst, self.cap = int(n_src), int(n_dst), int(cap_rows_per_dst)

    def _c(self):
        return _Layout(self.n_src, self.n_dst, self.cap)


_lib = None


def load():
    """Load libmoe.so (once). Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"libmoe.so not found at {library_path}; build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(library_path)
        for name, (res, args) in EXPORTED.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise MoEError(fn, status)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous(), "tensors must be contiguous GPU tensors"
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def moe_abi_version() -> int:
    return int(load().moe_abi_version())


MOE_OP_DISPATCH, MOE_OP_EXPERT_FFN, MOE_OP_EXPERT_FFN_BWD = 0, 1, 2


def moe_workspace_size(op: int, *, T: int = 0, E: int = 0, k: int = 0,
                       layout: Optional["Layout"] = None, rows: int = 0, d: int = 0, F: int = 0,
                       dtype: torch.dtype = torch.bfloat16) -> int:
    """Workspace bytes of one call of operation `op` (moe_workspace_size)."""
    clay = layout._c() if layout else None
    return int(load().moe_workspace_size(op, T, E, k, ctypes.byref(clay) if clay is not None else None,
                                         rows, d, F, MOE_BF16 if dtype == torch.bfloat16 else MOE_F32))


# ------------------------------------------------------------------ forward
def moe_route(x, w_router, k: int, *, flags: int = MOE_ROUTE_RENORM, logits=None,
              want_logits: bool = False, topk_idx=None, topk_w=None, stream=None):
    """Router logits, top-k selection and gates. Returns (topk_idx, topk_w, logits)."""
    T, d = x.shape
    E = w_router.shape[0]
    dev = x.device
    if want_logits and logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _check("moe_route", load().moe_route(_ptr(x), _ptr(w_router), T, d, E, k, _dt(x), flags,
                                         _ptr(logits), _ptr(topk_idx), _ptr(topk_w),
                                         _stream(stream)))
    return topk_idx, topk_w, logits


def moe_dispatch(x, topk_idx, E: int, *, layout: Optional[Layout] = None, d: Optional[int] = None,
                 dtype: Optional[torch.dtype] = None, out: Optional[dict] = None, stream=None):
    """Plan (+ copy unless x is None). Returns a dict with counts, expert_off,
    chunk_off, pair_slot, row_pair, x_disp (None if x is None) and ws."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    if x is not None:
        d = x.shape[1]
        dtype = x.dtype
    n_src = layout.n_src if layout else 1
    n_dst = layout.n_dst if layout else 1
    cap = layout.cap if layout else T * k
    lib = load()
    clay = layout._c() if layout else None
    lay_ptr = ctypes.byref(clay) if clay is not None else None
    o = dict(out or {})
    ws_bytes = int(lib.moe_dispatch_workspace_size(T, E, k, lay_ptr))
    if o.get("ws") is None:
        o["ws"] = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    for name, shape in (("counts", (n_src, E)), ("expert_off", (E + 1,)),
                        ("chunk_off", (n_dst, n_src + 1)), ("pair_slot", (T, k)),
                        ("row_pair", (n_dst * cap,))):
        if o.get(name) is None:
            o[name] = torch.empty(shape, dtype=torch.int32, device=dev)
    if x is not None and o.get("x_disp") is None:
        o["x_disp"] = torch.empty((n_dst * cap, d), dtype=dtype, device=dev)
    if x is None:
        o["x_disp"] = None
    dt = _dt(x) if x is not None else (MOE_BF16 if dtype in (None, torch.bfloat16) else MOE_F32)
    _check("moe_dispatch", lib.moe_dispatch(
        _ptr(x), _ptr(topk_idx), T, d if d is not None else 8, E, k, dt, lay_ptr,
        _ptr(o["counts"]), _ptr(o["expert_off"]), _ptr(o["chunk_off"]), _ptr(o["pair_slot"]),
        _ptr(o["row_pair"]), _ptr(o["x_disp"]), _ptr(o["ws"]), o["ws"].numel(), _stream(stream)))
    return o


def moe_dispatch_noalloc(x, topk_idx, E: int, *, layout: Optional[Layout] = None,
                         out: Optional[dict] = None, stream=None):
    """moe_dispatch with its workspace in the library's fixed per-GPU array (no ws).
    Returns the plan dict (counts, expert_off, chunk_off, pair_slot, row_pair, x_disp);
    outputs not passed in `out` are allocated here, by torch, before the call."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    d = x.shape[1]
    n_src = layout.n_src if layout else 1
    n_dst = layout.n_dst if layout else 1
    cap = layout.cap if layout else T * k
    clay = layout._c() if layout else None
    o = dict(out or {})
    for name, shape in (("counts", (n_src, E)), ("expert_off", (E + 1,)),
                        ("chunk_off", (n_dst, n_src + 1)), ("pair_slot", (T, k)),
                        ("row_pair", (n_dst * cap,))):
        if o.get(name) is None:
            o[name] = torch.empty(shape, dtype=torch.int32, device=dev)
    if o.get("x_disp") is None:
        o["x_disp"] = torch.empty((n_dst * cap, d), dtype=x.dtype, device=dev)
    _check("moe_dispatch_noalloc", load().moe_dispatch_noalloc(
        _ptr(x), _ptr(topk_idx), T, d, E, k, _dt(x),
        ctypes.byref(clay) if clay is not None else None, _ptr(o["counts"]),
        _ptr(o["expert_off"]), _ptr(o["chunk_off"]), _ptr(o["pair_slot"]), _ptr(o["row_pair"]),
        _ptr(o["x_disp"]), _stream(stream)))
    return o


def moe_dispatch_fp8(x, topk_idx, E: int, *, layout: Optional[Layout] = None,
                     out: Optional[dict] = None, stream=None):
    """Plan + block-scaled fp8 payload (bf16 x, d % 128 == 0). Returns the plan dict
    of moe_dispatch with q_disp (uint8 [rows, d]) and q_scale (float32 [rows, d/128])."""
    T, k = topk_idx.shape
    d = x.shape[1]
    dev = x.device
    n_src = layout.n_src if layout else 1
    n_dst = layout.n_dst if layout else 1
    cap = layout.cap if layout else T * k
    lib = load()
    clay = layout._c() if layout else None
    lay_ptr = ctypes.byref(clay) if clay is not None else None
    o = dict(out or {})
    ws_bytes = int(lib.moe_dispatch_workspace_size(T, E, k, lay_ptr))
    if o.get("ws") is None:
        o["ws"] = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    for name, shape in (("counts", (n_src, E)), ("expert_off", (E + 1,)),
                        ("chunk_off", (n_dst, n_src + 1)), ("pair_slot", (T, k)),
                        ("row_pair", (n_dst * cap,))):
        if o.get(name) is None:
            o[name] = torch.empty(shape, dtype=torch.int32, device=dev)
    if o.get("q_disp") is None:
        o["q_disp"] = torch.empty((n_dst * cap, d), dtype=torch.uint8, device=dev)
    if o.get("q_scale") is None:
        o["q_scale"] = torch.empty((n_dst * cap, d // 128), dtype=torch.float32, device=dev)
    _check("moe_dispatch_fp8", lib.moe_dispatch_fp8(
        _ptr(x), _ptr(topk_idx), T, d, E, k, lay_ptr, _ptr(o["counts"]), _ptr(o["expert_off"]),
        _ptr(o["chunk_off"]), _ptr(o["pair_slot"]), _ptr(o["row_pair"]), _ptr(o["q_disp"]),
        _ptr(o["q_scale"]), _ptr(o["ws"]), o["ws"].numel(), _stream(stream)))
    return o


def moe_dispatch_status(ws, stream=None) -> int:
    """Synchronises, then returns the device flag of the last dispatch on ws."""
    return int(load().moe_dispatch_status(_ptr(ws), _stream(stream)))


def moe_expert_ffn(x_disp, expert_off, w13, w2, *, y_disp=None, hu_save=None, ws=None,
                   stream=None):
    rows, d = x_disp.shape
    E, F2, _ = w13.shape
    F = F2 // 2
    lib = load()
    need = int(lib.moe_expert_ffn_workspace_size(E, rows, d, F, _dt(x_disp)))
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x_disp.device)
    if y_disp is None:
        y_disp = torch.empty((rows, d), dtype=x_disp.dtype, device=x_disp.device)
    _check("moe_expert_ffn", lib.moe_expert_ffn(
        _ptr(x_disp), _ptr(expert_off), _ptr(w13), _ptr(w2), E, rows, d, F, _dt(x_disp),
        _ptr(y_disp), _ptr(hu_save), _ptr(ws), ws.numel(), _stream(stream)))
    return y_disp


def moe_expert_ffn_gate_up(x_disp, expert_off, w13, *, act=None, hu_save=None, stream=None):
    rows, d = x_disp.shape
    E, F2, _ = w13.shape
    F = F2 // 2
    if act is None:
        act = torch.empty((rows, F), dtype=x_disp.dtype, device=x_disp.device)
    _check("moe_expert_ffn_gate_up", load().moe_expert_ffn_gate_up(
        _ptr(x_disp), _ptr(expert_off), _ptr(w13), E, rows, d, F, _dt(x_disp), _ptr(act),
        _ptr(hu_save), _stream(stream)))
    return act


def moe_expert_ffn_down(act, expert_off, w2, *, y_disp=None, stream=None):
    rows, F = act.shape
    E, d, _ = w2.shape
    if y_disp is None:
        y_disp = torch.empty((rows, d), dtype=act.dtype, device=act.device)
    _check("moe_expert_ffn_down", load().moe_expert_ffn_down(
        _ptr(act), _ptr(expert_off), _ptr(w2), E, rows, d, F, _dt(act), _ptr(y_disp),
        _stream(stream)))
    return y_disp


def moe_combine(y_disp, pair_slot, topk_w, *, y=None, stream=None):
    T, k = pair_slot.shape
    rows, d = y_disp.shape
    if y is None:
        y = torch.empty((T, d), dtype=y_disp.dtype, device=y_disp.device)
    _check("moe_combine", load().moe_combine(_ptr(y_disp), _ptr(pair_slot), _ptr(topk_w), T, k,
                                             d, rows, _dt(y_disp), _ptr(y), _stream(stream)))
    return y


# ----------------------------------------------------------------- backward
def moe_combine_bwd(dy, y_disp, pair_slot, topk_w, *, dy_disp=None, dtopk_w=None, stream=None):
    T, k = pair_slot.shape
    rows, d = y_disp.shape
    if dy_disp is None:
        dy_disp = torch.empty((rows, d), dtype=dy.dtype, device=dy.device)
    if dtopk_w is None:
        dtopk_w = torch.empty((T, k), dtype=torch.float32, device=dy.device)
    _check("moe_combine_bwd", load().moe_combine_bwd(
        _ptr(dy), _ptr(y_disp), _ptr(pair_slot), _ptr(topk_w), T, k, d, rows, _dt(dy),
        _ptr(dy_disp), _ptr(dtopk_w), _stream(stream)))
    return dy_disp, dtopk_w


def moe_expert_ffn_bwd(x_disp, dy_disp, hu_save, expert_off, w13, w2, *, dx_disp=None,
                       dw13=None, dw2=None, ws=None, stream=None):
    rows, d = x_disp.shape
    E, F2, _ = w13.shape
    F = F2 // 2
    dev = x_disp.device
    lib = load()
    need = int(lib.moe_expert_ffn_bwd_workspace_size(E, rows, d, F, _dt(x_disp)))
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if dx_disp is None:
        dx_disp = torch.empty((rows, d), dtype=x_disp.dtype, device=dev)
    if dw13 is None:
        dw13 = torch.empty((E, 2 * F, d), dtype=torch.float32, device=dev)
    if dw2 is None:
        dw2 = torch.empty((E, d, F), dtype=torch.float32, device=dev)
    _check("moe_expert_ffn_bwd", lib.moe_expert_ffn_bwd(
        _ptr(x_disp), _ptr(dy_disp), _ptr(hu_save), _ptr(expert_off), _ptr(w13), _ptr(w2), E,
        rows, d, F, _dt(x_disp), _ptr(dx_disp), _ptr(dw13), _ptr(dw2), _ptr(ws), ws.numel(),
        _stream(stream)))
    return dx_disp, dw13, dw2


def moe_route_bwd(x, topk_idx, topk_w, dtopk_w, expert_off, row_pair, E: int, *,
                  dlogits_sel=None, dw_router=None, stream=None):
    T, d = x.shape
    k = topk_idx.shape[1]
    if dlogits_sel is None:
        dlogits_sel = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if dw_router is None:
        dw_router = torch.empty((E, d), dtype=torch.float32, device=x.device)
    _check("moe_route_bwd", load().moe_route_bwd(
        _ptr(x), _ptr(topk_idx), _ptr(topk_w), _ptr(dtopk_w), _ptr(expert_off), _ptr(row_pair),
        T, d, E, k, _dt(x), _ptr(dlogits_sel), _ptr(dw_router), _stream(stream)))
    return dlogits_sel, dw_router


def moe_dispatch_bwd(dx_disp, pair_slot, *, topk_idx=None, dlogits_sel=None, w_router=None,
                     dx=None, stream=None):
    T, k = pair_slot.shape
    rows, d = dx_disp.shape
    E = w_router.shape[0] if w_router is not None else 0
    if dx is None:
        dx = torch.empty((T, d), dtype=dx_disp.dtype, device=dx_disp.device)
    _check("moe_dispatch_bwd", load().moe_dispatch_bwd(
        _ptr(dx_disp), _ptr(pair_slot), _ptr(topk_idx), _ptr(dlogits_sel), _ptr(w_router), T, k,
        d, E, rows, _dt(dx_disp), _ptr(dx), _stream(stream)))
    return dx


def moe_combine_add(y_disp, pair_slot, topk_w, residual, *, y=None, stream=None):
    """y[t] = residual[t] + sum_j topk_w[t,j] * y_disp[pair_slot[t,j]]."""
    T, k = pair_slot.shape
    rows, d = y_disp.shape
    if y is None:
        y = torch.empty((T, d), dtype=y_disp.dtype, device=y_disp.device)
    _check("moe_combine_add", load().moe_combine_add(
        _ptr(y_disp), _ptr(pair_slot), _ptr(topk_w), T, k, d, rows, _dt(y_disp), _ptr(residual),
        _ptr(y), _stream(stream)))
    return y


def moe_combine_partial(y_disp, pair_slot, topk_w, n_dst: int, cap: int, *, partial=None,
                        stream=None):
    """Per (token, destination) gate-weighted partial sums [n_dst*T, d] (rank-major)."""
    T, k = pair_slot.shape
    d = y_disp.shape[1]
    if partial is None:
        partial = torch.empty((n_dst * T, d), dtype=y_disp.dtype, device=y_disp.device)
    _check("moe_combine_partial", load().moe_combine_partial(
        _ptr(y_disp), _ptr(pair_slot), _ptr(topk_w), T, k, d, n_dst, cap, _dt(y_disp),
        _ptr(partial), _stream(stream)))
    return partial


def moe_combine_partials(partial, pair_slot, n_dst: int, cap: int, *, y=None, stream=None):
    """y[t] = sum over t's destinations (ascending) of partial[r*T + t]."""
    T, k = pair_slot.shape
    d = partial.shape[1]
    if y is None:
        y = torch.empty((T, d), dtype=partial.dtype, device=partial.device)
    _check("moe_combine_partials", load().moe_combine_partials(
        _ptr(partial), _ptr(pair_slot), T, k, d, n_dst, cap, _dt(partial), _ptr(y),
        _stream(stream)))
    return y


# ------------------------------------------------- receive side (rank-major layout)
def moe_ep_recv_plan(counts, chunk_off, r: int, cap: int, *, local_off=None, row_src=None,
                     stream=None):
    """Destination r's expert-major order of its region: (local_off [E/n_dst+1],
    row_src [cap]) from a rank-major dispatch plan's counts and chunk_off."""
    n_src, E = counts.shape
    n_dst = chunk_off.shape[0]
    dev = counts.device
    if local_off is None:
        local_off = torch.empty(E // n_dst + 1, dtype=torch.int32, device=dev)
    if row_src is None:
        row_src = torch.empty(cap, dtype=torch.int32, device=dev)
    _check("moe_ep_recv_plan", load().moe_ep_recv_plan(
        _ptr(counts), _ptr(chunk_off), n_src, n_dst, E, r, cap, _ptr(local_off), _ptr(row_src),
        _stream(stream)))
    return local_off, row_src


def moe_ep_recv_gather(x_region, row_src, *, x_local=None, stream=None):
    """x_local[j] = x_region[row_src[j]] for the live rows (the rest untouched)."""
    cap, d = x_region.shape
    if x_local is None:
        x_local = torch.empty_like(x_region)
    _check("moe_ep_recv_gather", load().moe_ep_recv_gather(
        _ptr(x_region), _ptr(row_src), cap, d, _dt(x_region), _ptr(x_local), _stream(stream)))
    return x_local


def moe_ep_recv_gather_fp8(q_region, scale_region, row_src=None, *, x_local=None, stream=None):
    """x_local[j] = bf16(decode(q[row_src[j]]) * scale) (row j itself if row_src is None)."""
    cap, d = q_region.shape
    if x_local is None:
        x_local = torch.empty((cap, d), dtype=torch.bfloat16, device=q_region.device)
    _check("moe_ep_recv_gather_fp8", load().moe_ep_recv_gather_fp8(
        _ptr(q_region), _ptr(scale_region), _ptr(row_src), cap, d, _ptr(x_local),
        _stream(stream)))
    return x_local


def moe_ep_recv_scatter(y_local, row_src, y_region, *, stream=None):
    """y_region[row_src[j]] = y_local[j] for the live rows."""
    cap, d = y_local.shape
    _check("moe_ep_recv_scatter", load().moe_ep_recv_scatter(
        _ptr(y_local), _ptr(row_src), cap, d, _dt(y_local), _ptr(y_region), _stream(stream)))
    return y_region


# ------------------------------------------------- overlap (two streams)
def forward_shared(x, w_router, w13, w2, w13_shared, w2_shared, k: int, *, side_stream=None,
                   out: Optional[dict] = None):
    """The layer plus one shared expert (a SwiGLU applied to every token, here the grouped
    GEMM with E = 1). The shared expert runs on `side_stream` while route, dispatch and the
    routed experts run on the current stream; moe_combine_add then adds its output into
    the combine ([EFA] Dispatch and combine: the dispatch's sender half returns and the
    GPU does other work, such as the shared expert, while the transfer is in flight).
    With side_stream None everything runs on the current stream, in the same order."""
    T, d = x.shape
    main = torch.cuda.current_stream()
    side = side_stream if side_stream is not None else main
    o = dict(out or {})
    if o.get("shared_off") is None:
        o["shared_off"] = torch.tensor([0, T], dtype=torch.int32, device=x.device)
    if side is not main:
        side.wait_stream(main)
    with torch.cuda.stream(side):
        shared = moe_expert_ffn(x, o["shared_off"], w13_shared.unsqueeze(0),
                                w2_shared.unsqueeze(0), y_disp=o.get("shared"), stream=side)
    idx, gates, _ = moe_route(x, w_router, k, topk_idx=o.get("topk_idx"), topk_w=o.get("topk_w"))
    plan = moe_dispatch(x, idx, w_router.shape[0], out=o.get("plan"))
    y_disp = moe_expert_ffn(plan["x_disp"], plan["expert_off"], w13, w2, y_disp=o.get("y_disp"),
                            ws=o.get("ws"))
    if side is not main:
        main.wait_stream(side)
        shared.record_stream(main)
    y = moe_combine_add(y_disp, plan["pair_slot"], gates, shared, y=o.get("y"))
    o.update(topk_idx=idx, topk_w=gates, plan=plan, y_disp=y_disp, shared=shared, y=y)
    return o


def forward_microbatched(x, w_router, w13, w2, k: int, n_micro: int = 2, *, streams=None,
                         y=None):
    """The layer on n_micro consecutive slices of the tokens, slice i on streams[i % len]
    so that one slice's memory-bound steps overlap another's grouped GEMM ([EFA] the
    dispatch and combine are split into halves to allow overlap and micro-batching).
    Every token's result equals the whole-batch forward bit for bit."""
    T, d = x.shape
    main = torch.cuda.current_stream()
    streams = streams or [main]
    if y is None:
        y = torch.empty((T, d), dtype=x.dtype, device=x.device)
    bounds = [T * i // n_micro for i in range(n_micro + 1)]
    for s in streams:
        if s is not main:
            s.wait_stream(main)
    for i in range(n_micro):
        s = streams[i % len(streams)]
        a, b = bounds[i], bounds[i + 1]
        if b == a:
            continue
        with torch.cuda.stream(s):
            xi = x[a:b]
            idx, gates, _ = moe_route(xi, w_router, k, stream=s)
            plan = moe_dispatch(xi, idx, w_router.shape[0], stream=s)
            y_disp = moe_expert_ffn(plan["x_disp"], plan["expert_off"], w13, w2, stream=s)
            moe_combine(y_disp, plan["pair_slot"], gates, y=y[a:b], stream=s)
            for t in (idx, gates, y_disp, *[v for v in plan.values() if v is not None]):
                t.record_stream(s)
    for s in streams:
        if s is not main:
            main.wait_stream(s)
    return y


def forward_ep_split(x, w_router, w13, w2, k: int, n_dst: int, *, w13_shared=None,
                     w2_shared=None, streams=None, out: Optional[dict] = None):
    """The layer on the rank-major (emulated expert-parallel) path, in its two halves.

    send:    moe_route, then moe_dispatch into n_dst destination regions of
             cap = T * max(k, E/n_dst) rows each (one contiguous chunk per sender);
    receive: for every destination r, moe_ep_recv_plan + moe_ep_recv_gather into its
             local expert-major order, its grouped GEMM over its E/n_dst experts
             (moe_expert_ffn_gate_up / _down with those experts' weights), and
             moe_ep_recv_scatter of the outputs back into its region;
    combine: moe_combine_add over the whole rank-major buffer, starting from the shared
             expert's output (a SwiGLU on every token, E = 1) when w13_shared is given.

    ([EFA] Dispatch and combine: the sender and receiver halves are separate kernels, so
    that the GPU can do other work, such as a shared expert, while the transfer is in
    flight.) streams = [main, side]: the shared expert runs on side while main runs the
    send half, and the destinations' receive paths alternate between main and side, so
    one destination's memory-bound gather and scatter overlap another's GEMM; each
    expert's weights are still read once. With streams None everything runs on the
    current stream in the same order. With one source the local order of a destination
    is the expert-major order restricted to its experts, so y equals forward()'s y (plus
    the shared expert's output) bit for bit."""
    T, d = x.shape
    E = w_router.shape[0]
    F = w13.shape[1] // 2
    assert E % n_dst == 0
    epr = E // n_dst
    cap = T * max(k, epr)
    main = torch.cuda.current_stream()
    streams = list(streams) if streams else [main]
    side = streams[1] if len(streams) > 1 else main
    o = dict(out or {})
    dev = x.device
    for s in streams:
        if s is not main:
            s.wait_stream(main)
    shared = None
    if w13_shared is not None:
        if o.get("shared_off") is None:
            o["shared_off"] = torch.tensor([0, T], dtype=torch.int32, device=dev)
        with torch.cuda.stream(side):
            shared = moe_expert_ffn(x, o["shared_off"], w13_shared.unsqueeze(0),
                                    w2_shared.unsqueeze(0), y_disp=o.get("shared"), stream=side)
    # send half
    idx, gates, _ = moe_route(x, w_router, k, topk_idx=o.get("topk_idx"), topk_w=o.get("topk_w"),
                              stream=main)
    lay = Layout(1, n_dst, cap)
    plan = moe_dispatch(x, idx, E, layout=lay, out=o.get("plan"), stream=main)
    sent = torch.cuda.Event()
    sent.record(main)
    if o.get("y_disp") is None:
        o["y_disp"] = torch.empty((n_dst * cap, d), dtype=x.dtype, device=dev)
    y_disp = o["y_disp"]
    # receive half, destination r on streams[r % len(streams)]; one set of local buffers
    # per stream (work on one stream runs in order)
    bufs = o.setdefault("recv_bufs", {})
    for r in range(n_dst):
        s = streams[r % len(streams)]
        if r < len(streams):
            s.wait_event(sent)
        b = bufs.get(r % len(streams))
        if b is None:
            b = dict(x_local=torch.empty((cap, d), dtype=x.dtype, device=dev),
                     act=torch.empty((cap, F), dtype=x.dtype, device=dev),
                     y_local=torch.empty((cap, d), dtype=x.dtype, device=dev),
                     local_off=torch.empty(epr + 1, dtype=torch.int32, device=dev),
                     row_src=torch.empty(cap, dtype=torch.int32, device=dev))
            bufs[r % len(streams)] = b
        with torch.cuda.stream(s):
            region = plan["x_disp"][r * cap:(r + 1) * cap]
            moe_ep_recv_plan(plan["counts"], plan["chunk_off"], r, cap, local_off=b["local_off"],
                             row_src=b["row_src"], stream=s)
            moe_ep_recv_gather(region, b["row_src"], x_local=b["x_local"], stream=s)
            moe_expert_ffn_gate_up(b["x_local"], b["local_off"], w13[r * epr:(r + 1) * epr],
                                   act=b["act"], stream=s)
            moe_expert_ffn_down(b["act"], b["local_off"], w2[r * epr:(r + 1) * epr],
                                y_disp=b["y_local"], stream=s)
            moe_ep_recv_scatter(b["y_local"], b["row_src"], y_disp[r * cap:(r + 1) * cap],
                                stream=s)
    for s in streams:
        if s is not main:
            main.wait_stream(s)
    if shared is not None:
        y = moe_combine_add(y_disp, plan["pair_slot"], gates, shared, y=o.get("y"), stream=main)
    else:
        y = moe_combine(y_disp, plan["pair_slot"], gates, y=o.get("y"), stream=main)
    o.update(topk_idx=idx, topk_w=gates, plan=plan, y_disp=y_disp, shared=shared, y=y)
    return o


# ------------------------------------------------------------ whole layer
def backward(x, w_router, w13, w2, fwd: dict, dy, *, stream=None):
    """Gradients of sum(dy * y) for a forward() run with save_for_backward=True:
    combine_bwd -> route_bwd -> expert_ffn_bwd -> dispatch_bwd (the router's backward
    needs only the gate gradients, so dx_disp is written right before it is gathered).
    Returns a dict with dx, dw_router, dw13, dw2 and the intermediates."""
    E = w_router.shape[0]
    dy_disp, dgates = moe_combine_bwd(dy, fwd["y_disp"], fwd["pair_slot"], fwd["topk_w"],
                                      stream=stream)
    dl, dwr = moe_route_bwd(x, fwd["topk_idx"], fwd["topk_w"], dgates, fwd["expert_off"],
                            fwd["row_pair"], E, stream=stream)
    dx_disp, dw13, dw2 = moe_expert_ffn_bwd(fwd["x_disp"], dy_disp, fwd["hu_save"],
                                            fwd["expert_off"], w13, w2, stream=stream)
    dx = moe_dispatch_bwd(dx_disp, fwd["pair_slot"], topk_idx=fwd["topk_idx"], dlogits_sel=dl,
                          w_router=w_router, stream=stream)
    return dict(dy_disp=dy_disp, dgates=dgates, dx_disp=dx_disp, dw13=dw13, dw2=dw2,
                dlogits_sel=dl, dw_router=dwr, dx=dx)



def forward(x, w_router, w13, w2, k: int, *, save_for_backward: bool = False, stream=None):
    """route -> dispatch -> expert FFN -> combine. Returns a dict of all outputs."""
    E = w_router.shape[0]
    F = w13.shape[1] // 2
    idx, gates, _ = moe_route(x, w_router, k, stream=stream)
    plan = moe_dispatch(x, idx, E, stream=stream)
    hu = None
    if save_for_backward:
        hu = torch.empty((plan["x_disp"].shape[0], 2 * F), dtype=x.dtype, device=x.device)
    y_disp = moe_expert_ffn(plan["x_disp"], plan["expert_off"], w13, w2, hu_save=hu,
                            stream=stream)
    y = moe_combine(y_disp, plan["pair_slot"], gates, stream=stream)
    return dict(topk_idx=idx, topk_w=gates, y_disp=y_disp, y=y, hu_save=hu, **plan)
