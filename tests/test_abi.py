"""C ABI checks that need no GPU: the library loads, exports every function
include/sol.h declares, and rejects bad arguments on the host before any HIP
call.  Every case below breaks exactly one rule that is checked before a
launch, so none of them reaches the device.

The argument-error cases pass made-up device addresses (0x10000, ...).  They
run only where no GPU is visible: on a machine with a GPU, a regression in a
host check would otherwise launch kernels on those addresses.  There, a
call that got past its checks fails with SOL_ERR_HIP (no device) instead.
"""

from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sol.h")
LIB = os.path.join(ROOT, "block_sparse_attention_sol_amd", "libsol.so")


def _gpu_visible() -> bool:
    # the ROCm kernel driver's device node; checking it initialises nothing
    return os.path.exists("/dev/kfd")


# cases that hand the library made-up device addresses
fake_pointers = pytest.mark.skipif(_gpu_visible(), reason="made-up device addresses: run only "
                                   "where no GPU is visible, so a regressed host check cannot "
                                   "launch kernels on them")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    from block_sparse_attention_sol_amd import sol
    return sol


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sol_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["sol_route", "sol_attn_fwd", "sol_attn_dense_fwd", "sol_status_str",
              "sol_route_workspace_bytes", "sol_num_blocks"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_status_strings(lib):
    for code in range(7):
        assert isinstance(lib.status_str(code), str) and lib.status_str(code)
    assert lib.status_str(0) == "ok"
    assert lib.status_str(99) == "unknown status"


def test_num_blocks(lib):
    assert lib.num_blocks(38247) == 598
    assert lib.num_blocks(64) == 1 and lib.num_blocks(65) == 2 and lib.num_blocks(0) == 0


def _desc(lib, B=1, N=1000, H=2, D=128, sn=None, sh=None, sb=None):
    sh = D if sh is None else sh
    sn = H * D if sn is None else sn
    sb = N * sn if sb is None else sb
    return lib.Desc(B, N, H, D, sb, sn, sh, sb, sn, sh)


def _packed_desc(lib, B=3, N=1000, H=2, D=128, T=2000, cu=0x90000, sb=0, osb=0):
    """Packed variable-length batch: [T, H, D] tensors with row offsets at `cu`."""
    d = lib.Desc(B, N, H, D, sb, H * D, D, osb, H * D, D)
    d.cu_seqlens = cu
    d.total_rows = T
    return d


def _route(lib, desc, q=0x10000, k=0x20000, tau=1.0, sink=64, scale=0.0, idx=0x30000,
           cnt=0x40000, tot=0x50000, order=None, ws=0x60000, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return lib.lib.sol_route(q, k, ctypes.byref(desc), ctypes.c_float(tau), sink,
                             ctypes.c_float(scale), idx, cnt, tot, order, ws, ws_bytes, None)


def _attn(lib, desc, q=0x10000, k=0x20000, v=0x30000, idx=0x40000, cnt=0x50000, order=None,
          sink=64, scale=0.0, o=0x60000, lse=None):
    return lib.lib.sol_attn_fwd(q, k, v, ctypes.byref(desc), idx, cnt, order, sink,
                                ctypes.c_float(scale), o, lse, None)


def test_workspace_size(lib):
    d = _desc(lib, N=38247, H=56)
    assert lib.lib.sol_route_workspace_bytes(ctypes.byref(d)) >= 2 * 56 * 598 * 128 * 4
    assert lib.lib.sol_route_workspace_bytes(ctypes.byref(_desc(lib, D=96))) == 0
    assert lib.lib.sol_route_workspace_bytes(None) == 0


@fake_pointers
@pytest.mark.parametrize("case,expect", [
    ("null_desc", 1), ("D96", 2), ("N0", 1), ("negative_sink", 1), ("null_q", 1),
    ("nan_tau", 1), ("negative_tau", 1), ("nan_scale", 1), ("misaligned_q", 3),
    ("odd_stride", 3), ("small_workspace", 4), ("null_workspace", 4), ("misaligned_ws", 3),
    ("misaligned_order", 3), ("too_many_blocks", 2), ("huge_span", 2),
    ("packed_batch_stride", 1), ("packed_out_batch_stride", 1), ("packed_negative_rows", 1),
    ("packed_too_many_rows", 2), ("packed_misaligned_offsets", 3),
])
def test_route_argument_errors(lib, case, expect):
    d = _desc(lib)
    kw = {}
    if case == "null_desc":
        st = lib.lib.sol_route(0x10000, 0x20000, None, ctypes.c_float(1.0), 0, ctypes.c_float(0),
                               0x30000, 0x40000, 0x50000, None, 0x60000, 1 << 30, None)
        assert st == expect
        return
    if case == "D96":
        d = _desc(lib, D=96)
    elif case == "N0":
        d = _desc(lib, N=0)
    elif case == "negative_sink":
        kw["sink"] = -1
    elif case == "null_q":
        kw["q"] = None
    elif case == "nan_tau":
        kw["tau"] = math.nan
    elif case == "negative_tau":
        kw["tau"] = -0.5
    elif case == "nan_scale":
        kw["scale"] = math.nan
    elif case == "misaligned_q":
        kw["q"] = 0x10008
    elif case == "odd_stride":
        d = _desc(lib, sn=2 * 128 + 4)
    elif case == "small_workspace":
        kw["ws_bytes"] = 100
    elif case == "null_workspace":
        kw["ws"] = None
    elif case == "misaligned_ws":
        kw["ws"] = 0x60010
    elif case == "misaligned_order":
        kw["order"] = 0x70002
    elif case == "too_many_blocks":
        d = _desc(lib, N=64 * 5000, H=1)          # 5000 candidate blocks > 4096
    elif case == "huge_span":
        d = _desc(lib, N=1 << 20, H=64, D=128)    # 32-bit per-head byte window exceeded
    elif case == "packed_batch_stride":
        d = _packed_desc(lib, sb=256000)          # packed rows take no batch stride
    elif case == "packed_out_batch_stride":
        d = _packed_desc(lib, osb=256000)
    elif case == "packed_negative_rows":
        d = _packed_desc(lib, T=-1)
    elif case == "packed_too_many_rows":
        d = _packed_desc(lib, T=1 << 31)          # offsets are int32
    elif case == "packed_misaligned_offsets":
        d = _packed_desc(lib, cu=0x90002)
    assert _route(lib, d, **kw) == expect


@fake_pointers
@pytest.mark.parametrize("case,expect", [
    ("D32", 2), ("null_v", 1), ("null_idx", 1), ("misaligned_o", 3), ("misaligned_lse", 3),
    ("negative_scale", 1), ("inf_scale", 1), ("odd_o_stride", 3), ("misaligned_order", 3),
    ("packed_batch_stride", 1), ("packed_misaligned_offsets", 3),
    ("o_is_k", 1), ("o_is_v", 1), ("o_is_q_other_strides", 1),
])
def test_attention_argument_errors(lib, case, expect):
    d = _desc(lib)
    kw = {}
    if case == "D32":
        d = _desc(lib, D=32)
    elif case == "null_v":
        kw["v"] = None
    elif case == "null_idx":
        kw["idx"] = None
    elif case == "misaligned_o":
        kw["o"] = 0x60002
    elif case == "misaligned_lse":
        kw["lse"] = 0x70001
    elif case == "negative_scale":
        kw["scale"] = -1.0
    elif case == "inf_scale":
        kw["scale"] = math.inf
    elif case == "odd_o_stride":
        d = lib.Desc(1, 1000, 2, 128, 256000, 256, 128, 256000, 260, 128)
    elif case == "misaligned_order":
        kw["order"] = 0x70002
    elif case == "packed_batch_stride":
        d = _packed_desc(lib, sb=256000)
    elif case == "packed_misaligned_offsets":
        d = _packed_desc(lib, cu=0x90001)
    elif case == "o_is_k":
        kw["o"] = 0x20000
    elif case == "o_is_v":
        kw["o"] = 0x30000
    elif case == "o_is_q_other_strides":
        d = lib.Desc(1, 1000, 2, 128, 256000, 256, 128, 512000, 512, 128)
        kw["o"] = 0x10000
    assert _attn(lib, d, **kw) == expect


@fake_pointers
def test_attention_in_place_over_q_with_equal_strides_passes_the_alias_check(lib):
    # O over Q is legal with equal strides; a misaligned LSE is then the first
    # rule broken (alignment, not argument), so nothing reaches the device
    d = _desc(lib)
    assert _attn(lib, d, o=0x10000, lse=0x70001) == 3
    st = lib.lib.sol_attn_dense_fwd(0x10000, 0x20000, 0x30000, ctypes.byref(d), ctypes.c_float(0),
                                    0x20000, None, None)
    assert st == 1                          # dense output over K


@fake_pointers
def test_dense_argument_errors(lib):
    d = _desc(lib, D=80)
    st = lib.lib.sol_attn_dense_fwd(0x10000, 0x20000, 0x30000, ctypes.byref(d), ctypes.c_float(0),
                                    0x40000, None, None)
    assert st == 2
    d = _desc(lib)
    st = lib.lib.sol_attn_dense_fwd(0x10000, None, 0x30000, ctypes.byref(d), ctypes.c_float(0),
                                    0x40000, None, None)
    assert st == 1


@fake_pointers
def test_gate_argument_errors(lib):
    d = _desc(lib)
    stats = 0x80000

    def gate(**kw):
        a = dict(q=0x10000, k=0x20000, v=0x30000, idx=0x40000, cnt=0x50000, order=None, sink=64,
                 scale=0.0, os=0x60000, od=0x70000, stats=stats)
        a.update(kw)
        return lib.lib.sol_gate_fwd(a["q"], a["k"], a["v"], ctypes.byref(d), a["idx"], a["cnt"],
                                    a["order"], a["sink"], ctypes.c_float(a["scale"]), a["os"],
                                    a["od"], a["stats"], None)
    assert gate(stats=None) == 1
    assert gate(od=None) == 1
    assert gate(od=0x60000) == 1            # the two outputs must differ
    assert gate(os=0x10000) == 1            # neither output may be an input:
    assert gate(od=0x10000) == 1            # the second pass reads Q, K and V
    assert gate(os=0x20000) == 1            # after the first one has written
    assert gate(od=0x30000) == 1
    assert gate(stats=0x80004) == 3         # float64 statistics need 8-byte alignment
    assert gate(od=0x70002) == 3
    assert gate(sink=-1) == 1
    d = _packed_desc(lib, osb=1024)
    assert gate() == 1                      # a packed batch takes no output batch stride


def _producer(lib, desc, q=0x10000, k=0x20000, gq=0x30000, gk=0x31000, eps=1e-6, cos=0x40000,
              sin=0x50000, sink=64, qo=0x60000, ko=0x70000, ws=0x80000, ws_bytes=1 << 40):
    return lib.lib.sol_qk_norm_rope_pool(q, k, ctypes.byref(desc), gq, gk, ctypes.c_float(eps),
                                         cos, sin, sink, qo, ko, ws, ws_bytes, None)


@fake_pointers
@pytest.mark.parametrize("case,expect", [
    ("null_gamma", 1), ("one_rope_table", 1), ("nan_eps", 1), ("negative_eps", 1),
    ("inf_eps", 1), ("same_outputs", 1), ("q_out_is_k", 1), ("in_place_other_strides", 1),
    ("misaligned_gamma", 3), ("misaligned_cos", 3), ("misaligned_out", 3), ("small_workspace", 4),
    ("D96", 2), ("negative_sink", 1),
])
def test_producer_argument_errors(lib, case, expect):
    d = _desc(lib)
    kw = {}
    if case == "null_gamma":
        kw["gk"] = None
    elif case == "one_rope_table":
        kw["sin"] = None
    elif case == "nan_eps":
        kw["eps"] = math.nan
    elif case == "negative_eps":
        kw["eps"] = -1e-6
    elif case == "inf_eps":
        kw["eps"] = math.inf
    elif case == "same_outputs":
        kw["ko"] = 0x60000
    elif case == "q_out_is_k":
        kw["qo"] = 0x20000
    elif case == "in_place_other_strides":
        d = lib.Desc(1, 1000, 2, 128, 256000, 256, 128, 512000, 512, 128)
        kw["qo"] = 0x10000
    elif case == "misaligned_gamma":
        kw["gq"] = 0x30004
    elif case == "misaligned_cos":
        kw["cos"] = 0x40008
    elif case == "misaligned_out":
        kw["ko"] = 0x70002
    elif case == "small_workspace":
        kw["ws_bytes"] = 64
    elif case == "D96":
        d = _desc(lib, D=96)
    elif case == "negative_sink":
        kw["sink"] = -3
    assert _producer(lib, d, **kw) == expect


@fake_pointers
def test_producer_in_place_with_equal_strides_passes_the_checks(lib):
    # equal strides make in place legal; a null workspace is then the first
    # (and only) rule broken, so nothing reaches the device
    d = _desc(lib)
    assert _producer(lib, d, qo=0x10000, ko=0x20000, ws=None) == 4


@fake_pointers
def test_route_pooled_argument_errors(lib):
    d = _desc(lib)

    def rp(**kw):
        a = dict(tau=1.0, sink=64, scale=0.0, idx=0x30000, cnt=0x40000, tot=0x50000, order=None,
                 ws=0x60000, ws_bytes=1 << 40, desc=d)
        a.update(kw)
        return lib.lib.sol_route_pooled(ctypes.byref(a["desc"]), ctypes.c_float(a["tau"]),
                                        a["sink"], ctypes.c_float(a["scale"]), a["idx"], a["cnt"],
                                        a["tot"], a["order"], a["ws"], a["ws_bytes"], None)
    assert rp(tau=math.nan) == 1
    assert rp(tau=-1.0) == 1
    assert rp(idx=None) == 1
    assert rp(tot=0x50004) == 3
    assert rp(order=0x70002) == 3
    assert rp(ws=None) == 4
    assert rp(ws_bytes=8) == 4
    assert rp(ws=0x60040) == 3
    assert rp(desc=_desc(lib, N=64 * 5000, H=1)) == 2
    assert lib.lib.sol_route_pooled(None, ctypes.c_float(1.0), 0, ctypes.c_float(0.0), 0x30000,
                                    0x40000, 0x50000, None, 0x60000, 1 << 30, None) == 1


@fake_pointers
def test_route_noalloc_argument_errors(lib):
    """sol_route_noalloc: sol_route's checks, and a call whose scratch need
    exceeds the static array is refused (SOL_ERR_SCRATCH) before any launch."""
    def rn(desc, q=0x10000, k=0x20000, tau=1.0, sink=64, idx=0x30000, cnt=0x40000, tot=0x50000,
           order=None):
        return lib.lib.sol_route_noalloc(q, k, ctypes.byref(desc), ctypes.c_float(tau), sink,
                                         ctypes.c_float(0.0), idx, cnt, tot, order, None)
    d = _desc(lib)
    assert rn(d, q=None) == 1
    assert rn(d, tau=math.nan) == 1
    assert rn(d, tot=0x50004) == 3
    assert rn(_desc(lib, D=96)) == 2
    # the pages' shape fits (34.3 MB); two copies of it (68.7 MB) do not
    page = _desc(lib, N=38247, H=56)
    assert lib.lib.sol_route_workspace_bytes(ctypes.byref(page)) <= lib.NOALLOC_SCRATCH_BYTES
    two = _desc(lib, B=2, N=38247, H=56)
    assert lib.lib.sol_route_workspace_bytes(ctypes.byref(two)) > lib.NOALLOC_SCRATCH_BYTES
    assert rn(two, sink=951) == lib.SOL_ERR_SCRATCH == 6
    assert lib.status_str(6) == "call needs more scratch than the static buffer holds"
