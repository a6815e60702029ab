"""The C ABI on the CPU: libmoe.so loads, exports every entry point include/moe.h
declares, and rejects bad arguments on the host before any HIP call (so these run
without a GPU: every call here returns before touching the device)."""
import ctypes
import os
import re

import pytest

import token_routing_expert_router_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INVALID, SHAPE, ALIGN, CAPACITY, BAD_INDEX, HIP, UNSUPPORTED = range(8)
F32, BF16 = 0, 1


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return moe.load()


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    # the binding declares the same set
    assert set(names) == set(moe.EXPORTED)


def test_abi_version_and_status_strings(lib):
    assert lib.moe_abi_version() == 1
    for s in range(8):
        assert lib.moe_status_str(s)
    assert lib.moe_status_str(99) == b"unknown status"


FAKE = 1 << 20          # a 16-byte aligned non-null address never dereferenced


def test_route_host_validation(lib):
    r = lib.moe_route
    assert r(FAKE, FAKE, 10, 64, 8, 9, BF16, 0, None, FAKE, FAKE, None) == SHAPE      # k > E
    assert r(FAKE, FAKE, 10, 64, 8, 0, BF16, 0, None, FAKE, FAKE, None) == INVALID    # k = 0
    assert r(FAKE, FAKE, 10, 64, 8, 2, 7, 0, None, FAKE, FAKE, None) == INVALID       # dtype
    assert r(FAKE, FAKE, 10, 64, 8, 2, BF16, 5, None, FAKE, FAKE, None) == INVALID    # flags
    assert r(FAKE, FAKE, 10, 60, 8, 2, BF16, 0, None, FAKE, FAKE, None) == ALIGN      # 120 B rows
    assert r(FAKE + 8, FAKE, 10, 64, 8, 2, BF16, 0, None, FAKE, FAKE, None) == ALIGN
    # bf16 buffer offsets are 32-bit: rows beyond 2^26 elements, or router weights of
    # 2^31 bytes, are refused before any launch
    assert r(FAKE, FAKE, 10, (1 << 26) + 8, 8, 2, BF16, 0, None, FAKE, FAKE, None) == UNSUPPORTED
    assert r(FAKE, FAKE, 10, 1 << 22, 512, 2, BF16, 0, None, FAKE, FAKE, None) == UNSUPPORTED
    assert r(None, FAKE, 10, 64, 8, 2, BF16, 0, None, FAKE, FAKE, None) == INVALID
    assert r(FAKE, FAKE, 10, 64, 1100, 2, BF16, 0, None, FAKE, FAKE, None) == UNSUPPORTED
    assert r(FAKE, FAKE, 10, 64, 600, 2, F32, 0, None, FAKE, FAKE, None) == UNSUPPORTED
    assert r(FAKE, FAKE, 10, 64, 64, 33, BF16, 0, None, FAKE, FAKE, None) == UNSUPPORTED
    assert r(None, None, 0, 64, 8, 2, BF16, 0, None, None, None, None) == OK          # empty


def _layout(n_src, n_dst, cap):
    return ctypes.byref(moe._Layout(n_src, n_dst, cap))


def test_dispatch_host_validation(lib):
    d = lib.moe_dispatch
    ws_sz = lib.moe_dispatch_workspace_size(4096, 384, 8, _layout(32, 32, 49152))
    assert ws_sz > 0
    args = lambda **kw: [kw.get("x", FAKE), FAKE, kw.get("T", 4096), kw.get("d", 7168),
                         kw.get("E", 384), kw.get("k", 8), BF16, kw.get("lay", _layout(32, 32, 49152)),
                         FAKE, FAKE, FAKE, FAKE, FAKE, kw.get("xd", FAKE), kw.get("ws", FAKE),
                         kw.get("wsb", ws_sz), None]
    # tight bound: 32 * 128 * min(8, 12) = 32768 rows per destination
    assert d(*args(lay=_layout(32, 32, 32767))) == CAPACITY
    assert d(*args(lay=_layout(32, 30, 49152))) == SHAPE         # 384 % 30
    assert d(*args(lay=_layout(33, 32, 49152))) == SHAPE         # 4096 % 33
    assert d(*args(lay=_layout(0, 32, 49152))) == INVALID
    assert d(*args(wsb=ws_sz - 1)) == CAPACITY
    assert d(*args(ws=FAKE + 16)) == ALIGN                        # 256-byte workspace
    assert d(*args(x=None)) == INVALID                            # x and x_disp together
    assert d(*args(k=400)) == SHAPE
    assert d(*args(E=2048, lay=None, k=8, T=16)) == UNSUPPORTED


def test_ffn_combine_bwd_host_validation(lib):
    f = lib.moe_expert_ffn
    need = lib.moe_expert_ffn_workspace_size(64, 24576, 2048, 1408, BF16)
    assert need >= 24576 * 1408 * 2
    base = [FAKE, FAKE, FAKE, FAKE, 64, 24576, 2048, 1408, BF16, FAKE, None, FAKE, need, None]
    bad = list(base); bad[7] = 1400                                 # F % 64
    assert f(*bad) == UNSUPPORTED
    bad = list(base); bad[12] = need - 1
    assert f(*bad) == CAPACITY
    bad = list(base); bad[11] = FAKE + 16
    assert f(*bad) == ALIGN
    bad = list(base); bad[2] = None
    assert f(*bad) == INVALID
    c = lib.moe_combine
    assert c(FAKE, FAKE, FAKE, 10, 2, 60, 20, BF16, FAKE, None) == ALIGN
    assert c(FAKE, FAKE, FAKE, 10, 0, 64, 20, BF16, FAKE, None) == INVALID
    assert c(None, None, None, 0, 2, 64, 0, BF16, None, None) == OK
    assert c(FAKE, FAKE, FAKE, 10, 65, 64, 20, BF16, FAKE, None) == UNSUPPORTED   # k > 64
    cb = lib.moe_combine_bwd
    assert cb(FAKE, FAKE, FAKE, FAKE, 10, 40, 64, 20, BF16, FAKE, FAKE, None) == UNSUPPORTED
    db = lib.moe_dispatch_bwd
    assert db(FAKE, FAKE, None, FAKE, None, 10, 2, 64, 8, 20, BF16, FAKE, None) == INVALID
    assert db(FAKE, FAKE, None, None, None, 10, 65, 64, 8, 20, BF16, FAKE, None) == UNSUPPORTED


def test_ep_recv_host_validation(lib):
    p = lib.moe_ep_recv_plan
    assert p(FAKE, FAKE, 32, 32, 384, 32, 49152, FAKE, FAKE, None) == SHAPE      # r >= n_dst
    assert p(FAKE, FAKE, 32, 5, 384, 0, 49152, FAKE, FAKE, None) == SHAPE       # E % n_dst
    assert p(FAKE, FAKE, 64, 1, 1024, 0, 100, FAKE, FAKE, None) == UNSUPPORTED  # epr*n_src
    assert p(None, FAKE, 32, 32, 384, 0, 49152, FAKE, FAKE, None) == INVALID
    assert p(FAKE, FAKE, 0, 32, 384, 0, 49152, FAKE, FAKE, None) == INVALID
    g, s = lib.moe_ep_recv_gather, lib.moe_ep_recv_scatter
    assert g(FAKE, FAKE, 100, 60, BF16, FAKE, None) == ALIGN                    # 120-byte rows
    assert g(FAKE + 8, FAKE, 100, 64, BF16, FAKE, None) == ALIGN
    assert s(FAKE, None, 100, 64, BF16, FAKE, None) == INVALID
    assert s(None, None, 0, 64, BF16, None, None) == OK                         # nothing to do
    assert g(FAKE, FAKE, 1 << 31, 64, BF16, FAKE, None) == UNSUPPORTED


def test_fp8_dispatch_host_validation(lib):
    f = lib.moe_dispatch_fp8
    ws_sz = lib.moe_dispatch_workspace_size(4096, 64, 6, None)
    base = [FAKE, FAKE, 4096, 2048, 64, 6, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
            ws_sz, None]
    bad = list(base); bad[3] = 2000                      # d % 128
    assert f(*bad) == UNSUPPORTED
    bad = list(base); bad[12] = None                     # no payload buffer
    assert f(*bad) == INVALID
    bad = list(base); bad[12] = FAKE + 8                 # codes not 16-byte aligned
    assert f(*bad) == ALIGN
    bad = list(base); bad[15] = ws_sz - 1
    assert f(*bad) == CAPACITY
    g = lib.moe_ep_recv_gather_fp8
    assert g(FAKE, FAKE, None, 100, 2000, FAKE, None) == UNSUPPORTED
    assert g(FAKE, FAKE + 4, None, 100, 2048, FAKE, None) == ALIGN
    assert g(None, FAKE, None, 100, 2048, FAKE, None) == INVALID
    assert g(None, None, None, 0, 2048, None, None) == OK


def test_partial_combine_host_validation(lib):
    p, q = lib.moe_combine_partial, lib.moe_combine_partials
    assert p(FAKE, FAKE, FAKE, 10, 2, 64, 65, 100, BF16, FAKE, None) == UNSUPPORTED   # n_dst
    assert p(FAKE, FAKE, None, 10, 2, 64, 4, 100, BF16, FAKE, None) == INVALID        # gates
    assert p(FAKE, FAKE, FAKE, 10, 2, 60, 4, 100, BF16, FAKE, None) == ALIGN
    assert q(FAKE, FAKE, 10, 2, 64, 0, 100, BF16, FAKE, None) == INVALID              # n_dst 0
    assert q(None, None, 0, 2, 64, 4, 100, BF16, None, None) == OK


def test_combine_add_host_validation(lib):
    a = lib.moe_combine_add
    assert a(FAKE, FAKE, FAKE, 10, 2, 64, 20, BF16, None, FAKE, None) == INVALID     # residual
    assert a(FAKE, FAKE, FAKE, 10, 2, 64, 20, BF16, FAKE + 8, FAKE, None) == ALIGN


def test_expert_major_dispatch_accepts_large_batches(lib):
    """The expert-major plan scan walks its blocks in batches and has no LDS limit, so
    large prefill batches pass every host check. Each case runs up to the workspace-size
    check, which comes after the shape checks, and gives that check's code; so no call
    here reaches a launch."""
    d = lib.moe_dispatch
    for T, E, k in ((16384, 512, 8), (32768, 384, 8), (8192, 1024, 8), (262144, 64, 6)):
        ws_sz = lib.moe_dispatch_workspace_size(T, E, k, None)
        assert ws_sz > 0
        st = d(FAKE, FAKE, T, 7168, E, k, BF16, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
               ws_sz - 1, None)
        assert st == CAPACITY, (T, E, k, st)
    # the rank-major scan keeps its whole plan in one workgroup's LDS (32768 ints):
    # 64 sources of 4096 tokens at E = 1024 need 1024 blocks x 1024 experts of it
    lay = _layout(64, 64, 64 * 4096 * 16)
    ws_sz = lib.moe_dispatch_workspace_size(64 * 4096, 1024, 8, lay)
    st = d(FAKE, FAKE, 64 * 4096, 64, 1024, 8, BF16, lay, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
           ws_sz, None)
    assert st == UNSUPPORTED


def test_empty_batch_plan_host_validation(lib):
    """T = 0: the plan outputs are still written (zeros, row_pair -1), so they and the
    workspace must be given; topk_idx, pair_slot, x and x_disp are not needed."""
    d = lib.moe_dispatch
    ws_sz = lib.moe_dispatch_workspace_size(0, 8, 2, None)
    assert ws_sz > 0
    assert d(None, None, 0, 64, 8, 2, BF16, None, None, FAKE, FAKE, None, None, None, FAKE,
             ws_sz, None) == INVALID                       # no counts
    assert d(None, None, 0, 64, 8, 2, BF16, None, FAKE, FAKE, FAKE, None, None, None, FAKE + 16,
             ws_sz, None) == ALIGN                         # workspace not 256-byte aligned
    lay = _layout(4, 4, 100)
    assert d(None, None, 0, 64, 8, 2, BF16, lay, FAKE, FAKE, FAKE, None, None, None, FAKE,
             ws_sz, None) == INVALID                       # 400 rows but no row_pair
    rb = lib.moe_route_bwd
    assert rb(None, None, None, None, None, None, 0, 64, 8, 2, BF16, None, None, None) == INVALID
    assert rb(None, None, None, None, None, None, 0, 64, 8, 2, BF16, None, FAKE + 8,
              None) == ALIGN


def test_workspace_size_by_operation(lib):
    lay = _layout(32, 32, 49152)
    ws = lib.moe_workspace_size
    assert ws(0, 4096, 384, 8, lay, 0, 0, 0, BF16) == lib.moe_dispatch_workspace_size(4096, 384, 8, lay)
    assert ws(0, 4096, 64, 6, None, 0, 0, 0, BF16) == lib.moe_dispatch_workspace_size(4096, 64, 6, None)
    assert ws(1, 0, 64, 0, None, 24576, 2048, 1408, BF16) == \
        lib.moe_expert_ffn_workspace_size(64, 24576, 2048, 1408, BF16)
    assert ws(2, 0, 64, 0, None, 24576, 2048, 1408, BF16) == \
        lib.moe_expert_ffn_bwd_workspace_size(64, 24576, 2048, 1408, BF16)
    assert ws(1, 0, 64, 0, None, 24576, 2048, 1408, BF16) > 0
    assert ws(7, 4096, 64, 6, None, 24576, 2048, 1408, BF16) == 0      # no such operation
    assert ws(0, -1, 64, 6, None, 0, 0, 0, BF16) == 0                 # invalid sizes


def test_route_accepts_1024_experts_in_bf16(lib):
    r = lib.moe_route
    # past every argument check, the null logits/idx pointers are the only fault:
    # E = 1024 is accepted for bf16 (INVALID from the null topk_idx), refused for f32
    assert r(FAKE, FAKE, 10, 64, 1024, 8, BF16, 0, None, None, FAKE, None) == INVALID
    assert r(FAKE, FAKE, 10, 64, 1024, 8, F32, 0, None, None, FAKE, None) == UNSUPPORTED
    assert r(FAKE, FAKE, 10, 64, 1025, 8, BF16, 0, None, None, FAKE, None) == UNSUPPORTED


def test_noalloc_dispatch_rejects_plans_past_its_array(lib):
    """The allocation-free dispatch refuses, before any HIP call, a plan whose workspace
    exceeds its fixed 4 MiB array."""
    n = lib.moe_dispatch_noalloc
    T, E, k = 200_000, 1024, 8
    assert lib.moe_dispatch_workspace_size(T, E, k, None) > 4 << 20
    assert n(FAKE, FAKE, T, 64, E, k, BF16, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == CAPACITY
    assert n(FAKE, FAKE, 10, 64, 8, 9, BF16, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
