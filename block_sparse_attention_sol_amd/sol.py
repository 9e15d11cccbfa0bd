"""Thin ctypes binding of libsol.so (C ABI in include/sol.h).

Argument marshalling only: every step of routing and attention runs in the
HIP kernels of libsol.  PyTorch provides device memory and the current
stream.  Importing this module fails loudly when libsol.so has not been built
(``python block_sparse_attention_sol_amd/build.py``); there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsol.so")

BLOCK = 64

(SOL_OK, SOL_ERR_ARG, SOL_ERR_UNSUPPORTED, SOL_ERR_ALIGN, SOL_ERR_WORKSPACE, SOL_ERR_HIP,
 SOL_ERR_SCRATCH) = range(7)

# bytes of the library's static routing scratch (sol_route_noalloc)
NOALLOC_SCRATCH_BYTES = 48 << 20


class SolError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} (status {status})")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("H", ctypes.c_int32),
                ("D", ctypes.c_int32),
                ("qkv_sb", ctypes.c_int64), ("qkv_sn", ctypes.c_int64), ("qkv_sh", ctypes.c_int64),
                ("o_sb", ctypes.c_int64), ("o_sn", ctypes.c_int64), ("o_sh", ctypes.c_int64),
                ("cu_seqlens", ctypes.c_void_p), ("total_rows", ctypes.c_int64)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libsol.so not built at {_LIB_PATH}; run "
                          "`python block_sparse_attention_sol_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    dp = ctypes.POINTER(Desc)
    lib.sol_num_blocks.argtypes, lib.sol_num_blocks.restype = [i32], i32
    lib.sol_route_workspace_bytes.argtypes, lib.sol_route_workspace_bytes.restype = [dp], sz
    lib.sol_route.argtypes = [vp, vp, dp, f32, i32, f32, vp, vp, vp, vp, vp, sz, vp]
    lib.sol_route.restype = ctypes.c_int
    lib.sol_attn_fwd.argtypes = [vp, vp, vp, dp, vp, vp, vp, i32, f32, vp, vp, vp]
    lib.sol_attn_fwd.restype = ctypes.c_int
    lib.sol_attn_dense_fwd.argtypes = [vp, vp, vp, dp, f32, vp, vp, vp]
    lib.sol_attn_dense_fwd.restype = ctypes.c_int
    lib.sol_gate_fwd.argtypes = [vp, vp, vp, dp, vp, vp, vp, i32, f32, vp, vp, vp, vp]
    lib.sol_gate_fwd.restype = ctypes.c_int
    lib.sol_qk_norm_rope_pool.argtypes = [vp, vp, dp, vp, vp, f32, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.sol_qk_norm_rope_pool.restype = ctypes.c_int
    lib.sol_route_pooled.argtypes = [dp, f32, i32, f32, vp, vp, vp, vp, vp, sz, vp]
    lib.sol_route_pooled.restype = ctypes.c_int
    lib.sol_route_noalloc.argtypes = [vp, vp, dp, f32, i32, f32, vp, vp, vp, vp, vp]
    lib.sol_route_noalloc.restype = ctypes.c_int
    lib.sol_status_str.argtypes, lib.sol_status_str.restype = [ctypes.c_int], ctypes.c_char_p
    return lib


lib = _load()


def status_str(status: int) -> str:
    return lib.sol_status_str(int(status)).decode()


def num_blocks(N: int) -> int:
    return int(lib.sol_num_blocks(int(N)))


def _check(status: int, what: str) -> None:
    if status != SOL_OK:
        raise SolError(status, what)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def packed_offsets(lengths, device) -> tuple[torch.Tensor, int]:
    """Row offsets (int32 [B + 1] on `device`) and the longest length of a packed
    variable-length batch whose samples have the given lengths."""
    lengths = [int(n) for n in lengths]
    if not lengths or min(lengths) < 0:
        raise ValueError("need one or more non-negative sample lengths")
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    return torch.tensor(cu, dtype=torch.int32, device=device), max(max(lengths), 1)


def _shape(q: torch.Tensor, cu_seqlens, max_seqlen):
    """(B, N, H, D) of a call: from [B, N, H, D] tensors, or from packed [T, H, D]
    tensors with row offsets cu_seqlens (N = max_seqlen, the longest sample)."""
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError("expected [B, N, H, D] tensors")
        return tuple(q.shape)
    if q.dim() != 3:
        raise ValueError("a packed batch takes [T, H, D] tensors")
    if (cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2 or cu_seqlens.dtype != torch.int32
            or cu_seqlens.device != q.device):
        raise ValueError("cu_seqlens must be int32 [B + 1] on the tensors' device")
    if max_seqlen is None or int(max_seqlen) < 1:
        raise ValueError("a packed batch needs max_seqlen >= 1 (the longest sample)")
    T, H, D = q.shape
    return cu_seqlens.numel() - 1, int(max_seqlen), H, D


def make_desc(q: torch.Tensor, o: torch.Tensor | None = None, cu_seqlens=None,
              max_seqlen=None) -> Desc:
    """Descriptor of [B, N, H, D] bf16 tensors (or packed [T, H, D] ones with row
    offsets cu_seqlens): Q/K/V strides from q, O strides from o."""
    B, N, H, D = _shape(q, cu_seqlens, max_seqlen)
    o = q if o is None else o
    if q.stride(-1) != 1 or o.stride(-1) != 1:
        raise SolError(SOL_ERR_UNSUPPORTED, "stride along D must be 1")
    if cu_seqlens is None:
        return Desc(B, N, H, D, q.stride(0), q.stride(1), q.stride(2), o.stride(0), o.stride(1),
                    o.stride(2), None, 0)
    return Desc(B, N, H, D, 0, q.stride(0), q.stride(1), 0, o.stride(0), o.stride(1),
                cu_seqlens.data_ptr(), q.shape[0])


def _check_qkv(q, k, v=None):
    ts = [q, k] + ([v] if v is not None else [])
    for t in ts:
        if not t.is_cuda or t.dtype != torch.bfloat16:
            raise ValueError("Q, K, V must be bf16 CUDA(HIP) tensors")
        if t.shape != q.shape or t.stride() != q.stride():
            raise ValueError("Q, K, V must share shape and strides")


def _check_buffer(t, dtype, shape, device, name, contiguous=True):
    """The C ABI takes bare pointers, so the sizes the kernels index by are
    checked here: a smaller buffer would be read or written past its end."""
    if (t.dtype != dtype or tuple(t.shape) != tuple(shape) or t.device != device
            or (contiguous and not t.is_contiguous())):
        raise ValueError(f"{name} must be a{' contiguous' if contiguous else ''} {dtype} tensor "
                         f"of shape {tuple(shape)} on {device}")


def _check_out(o, q, name="out"):
    if o.dtype != torch.bfloat16 or o.shape != q.shape or o.device != q.device or o.stride(-1) != 1:
        raise ValueError(f"{name} must be bf16 with q's shape, on q's device, unit stride along D")


def _check_lists(q, blk_idx, blk_cnt, order, cu_seqlens, max_seqlen):
    B, N, H, _ = _shape(q, cu_seqlens, max_seqlen)
    NB = num_blocks(N)
    _check_buffer(blk_idx, torch.int16, (B, H, NB, NB), q.device, "blk_idx")
    _check_buffer(blk_cnt, torch.int32, (B, H, NB), q.device, "blk_cnt")
    if order is not None:
        _check_buffer(order, torch.int32, (B, H, NB), q.device, "order")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def route_workspace_bytes(q: torch.Tensor, cu_seqlens=None, max_seqlen=None) -> int:
    return int(lib.sol_route_workspace_bytes(ctypes.byref(make_desc(q, None, cu_seqlens,
                                                                    max_seqlen))))


def route_outputs(q: torch.Tensor, cu_seqlens=None, max_seqlen=None):
    """Empty (blk_idx, blk_cnt, totals, order) tensors for route() on q's shape."""
    B, N, H, D = _shape(q, cu_seqlens, max_seqlen)
    NB = num_blocks(N)
    return (torch.empty((B, H, NB, NB), dtype=torch.int16, device=q.device),
            torch.empty((B, H, NB), dtype=torch.int32, device=q.device),
            torch.empty(2, dtype=torch.int64, device=q.device),
            torch.empty((B, H, NB), dtype=torch.int32, device=q.device))


def route(q: torch.Tensor, k: torch.Tensor, tau: float, sink: int, scale: float = 0.0,
          workspace: torch.Tensor | None = None, out=None, cu_seqlens=None, max_seqlen=None):
    """Online block routing.  Returns (blk_idx int16 [B,H,NB,NB], blk_cnt int32 [B,H,NB],
    totals int64 [2], order int32 [B,H,NB]) on q's device; only the first blk_cnt entries
    of each row of blk_idx are set; order is the attention schedule (longest list first).
    With cu_seqlens, q and k are packed [T, H, D] and N is max_seqlen."""
    _check_qkv(q, k)
    desc = make_desc(q, None, cu_seqlens, max_seqlen)
    idx, cnt, totals, order = (route_outputs(q, cu_seqlens, max_seqlen) if out is None
                               else out)
    _check_lists(q, idx, cnt, order, cu_seqlens, max_seqlen)
    _check_buffer(totals, torch.int64, (2,), q.device, "totals")
    need = int(lib.sol_route_workspace_bytes(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib.sol_route(q.data_ptr(), k.data_ptr(), ctypes.byref(desc), ctypes.c_float(tau),
                       int(sink), ctypes.c_float(scale), idx.data_ptr(), cnt.data_ptr(),
                       totals.data_ptr(), order.data_ptr() if order is not None else None,
                       workspace.data_ptr(), _nbytes(workspace), _stream(q))
    _check(st, "sol_route")
    return idx, cnt, totals, order


def route_noalloc(q: torch.Tensor, k: torch.Tensor, tau: float, sink: int, scale: float = 0.0,
                  out=None, cu_seqlens=None, max_seqlen=None):
    """route() without a workspace: the library's static per-GPU scratch holds the
    block means (sol_route_noalloc), so with ``out`` given nothing is allocated.
    Calls that overlap on one GPU race on that scratch.  Same returns as route()."""
    _check_qkv(q, k)
    desc = make_desc(q, None, cu_seqlens, max_seqlen)
    idx, cnt, totals, order = (route_outputs(q, cu_seqlens, max_seqlen) if out is None
                               else out)
    _check_lists(q, idx, cnt, order, cu_seqlens, max_seqlen)
    _check_buffer(totals, torch.int64, (2,), q.device, "totals")
    st = lib.sol_route_noalloc(q.data_ptr(), k.data_ptr(), ctypes.byref(desc), ctypes.c_float(tau),
                               int(sink), ctypes.c_float(scale), idx.data_ptr(), cnt.data_ptr(),
                               totals.data_ptr(),
                               order.data_ptr() if order is not None else None, _stream(q))
    _check(st, "sol_route_noalloc")
    return idx, cnt, totals, order


def _lse_buffer(q, B, H, N, return_lse, lse_out):
    if lse_out is not None:
        if (lse_out.dtype != torch.float32 or tuple(lse_out.shape) != (B, H, N)
                or not lse_out.is_contiguous() or lse_out.device != q.device):
            raise ValueError("lse_out must be a contiguous float32 [B, H, N] tensor")
        return lse_out
    return torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None


def attn(q, k, v, blk_idx, blk_cnt, sink: int, scale: float = 0.0, out=None, return_lse=False,
         order=None, cu_seqlens=None, max_seqlen=None, lse_out=None):
    """Sink + routed block-sparse attention forward.  Returns O (and LSE [B,H,N] fp32,
    into ``lse_out`` when given).  ``order`` is the schedule from route() (None:
    sequence order; results are the same).  With cu_seqlens the tensors are
    packed [T, H, D] and N is max_seqlen."""
    _check_qkv(q, k, v)
    B, N, H, D = _shape(q, cu_seqlens, max_seqlen)
    o = torch.empty_like(q) if out is None else out
    _check_out(o, q)
    lse = _lse_buffer(q, B, H, N, return_lse, lse_out)
    return_lse = lse is not None
    _check_lists(q, blk_idx, blk_cnt, order, cu_seqlens, max_seqlen)
    desc = make_desc(q, o, cu_seqlens, max_seqlen)
    st = lib.sol_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(desc),
                          blk_idx.data_ptr(), blk_cnt.data_ptr(),
                          order.data_ptr() if order is not None else None, int(sink),
                          ctypes.c_float(scale),
                          o.data_ptr(), lse.data_ptr() if lse is not None else None, _stream(q))
    _check(st, "sol_attn_fwd")
    return (o, lse) if return_lse else o


def attn_dense(q, k, v, scale: float = 0.0, out=None, return_lse=False, cu_seqlens=None,
               max_seqlen=None, lse_out=None):
    """Full softmax attention (routing disabled)."""
    _check_qkv(q, k, v)
    B, N, H, D = _shape(q, cu_seqlens, max_seqlen)
    o = torch.empty_like(q) if out is None else out
    _check_out(o, q)
    lse = _lse_buffer(q, B, H, N, return_lse, lse_out)
    return_lse = lse is not None
    desc = make_desc(q, o, cu_seqlens, max_seqlen)
    st = lib.sol_attn_dense_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                ctypes.byref(desc), ctypes.c_float(scale), o.data_ptr(),
                                lse.data_ptr() if lse is not None else None, _stream(q))
    _check(st, "sol_attn_dense_fwd")
    return (o, lse) if return_lse else o


def gate(q, k, v, blk_idx, blk_cnt, sink: int, scale: float = 0.0, order=None, cu_seqlens=None,
         max_seqlen=None):
    """Sparse-vs-dense gate: returns (o_sparse, o_dense, stats) with stats a float64
    tensor [max_abs, sum_abs, sum_sq_diff, sum_sq_dense, count, mean_abs, l2_rel]
    on q's device, all computed by the library."""
    _check_qkv(q, k, v)
    _check_lists(q, blk_idx, blk_cnt, order, cu_seqlens, max_seqlen)
    o_s, o_d = torch.empty_like(q), torch.empty_like(q)
    stats = torch.empty(7, dtype=torch.float64, device=q.device)
    desc = make_desc(q, o_s, cu_seqlens, max_seqlen)
    st = lib.sol_gate_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(desc),
                          blk_idx.data_ptr(), blk_cnt.data_ptr(),
                          order.data_ptr() if order is not None else None, int(sink),
                          ctypes.c_float(scale), o_s.data_ptr(), o_d.data_ptr(), stats.data_ptr(),
                          _stream(q))
    _check(st, "sol_gate_fwd")
    return o_s, o_d, stats


def forward(q, k, v, tau: float, sink: int, scale: float = 0.0, return_lse=False,
            cu_seqlens=None, max_seqlen=None):
    """Routing then sparse attention on the current stream; returns (O, [LSE,] idx, cnt, totals)."""
    idx, cnt, totals, order = route(q, k, tau, sink, scale, cu_seqlens=cu_seqlens,
                                    max_seqlen=max_seqlen)
    res = attn(q, k, v, idx, cnt, sink, scale, return_lse=return_lse, order=order,
               cu_seqlens=cu_seqlens, max_seqlen=max_seqlen)
    if return_lse:
        return res[0], res[1], idx, cnt, totals
    return res, idx, cnt, totals


def qk_norm_rope_pool(q, k, gamma_q, gamma_k, eps: float, rope_cos=None, rope_sin=None,
                      sink: int = 0, out=None, workspace=None, cu_seqlens=None, max_seqlen=None):
    """QK-norm + RoPE of q and k into bf16 outputs, with the block means of the outputs
    written into the routing workspace.  Returns (q_out, k_out, workspace); pass the
    workspace to route_pooled().  ``out`` = (q_out, k_out) may be (q, k) (in place).
    gamma_* are float32 [D]; rope_cos / rope_sin float32 [N, D/2] or None."""
    _check_qkv(q, k)
    # the outputs first: their strides (not q's) are the descriptor's O strides;
    # empty_like of a strided view (say of a merged QKV projection) is dense
    q_out, k_out = (torch.empty_like(q), torch.empty_like(k)) if out is None else out
    desc = make_desc(q, q_out, cu_seqlens, max_seqlen)
    for t in (q_out, k_out):
        if (not t.is_cuda or t.dtype != torch.bfloat16 or t.shape != q.shape
                or t.stride() != q_out.stride()):
            raise ValueError("q_out and k_out must be bf16 with q's shape and one set of strides")
    for t in (gamma_q, gamma_k, rope_cos, rope_sin):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()
                              or t.device != q.device):
            raise ValueError("gamma and RoPE tables must be contiguous float32 on q's device")
    D = q.shape[-1]
    if gamma_q.numel() != D or gamma_k.numel() != D:
        raise ValueError("gamma_q and gamma_k need D entries")
    if rope_cos is not None and (rope_sin is None or rope_cos.shape != rope_sin.shape
                                 or rope_cos.dim() != 2 or rope_cos.shape[1] != D // 2
                                 or rope_cos.shape[0] < desc.N):
        raise ValueError("rope_cos and rope_sin must both be float32 [>= N, D/2]")
    need = int(lib.sol_route_workspace_bytes(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib.sol_qk_norm_rope_pool(q.data_ptr(), k.data_ptr(), ctypes.byref(desc),
                                   gamma_q.data_ptr(), gamma_k.data_ptr(), ctypes.c_float(eps),
                                   rope_cos.data_ptr() if rope_cos is not None else None,
                                   rope_sin.data_ptr() if rope_sin is not None else None,
                                   int(sink), q_out.data_ptr(), k_out.data_ptr(),
                                   workspace.data_ptr(), _nbytes(workspace), _stream(q))
    _check(st, "sol_qk_norm_rope_pool")
    return q_out, k_out, workspace


def route_pooled(q, workspace, tau: float, sink: int, scale: float = 0.0, out=None,
                 cu_seqlens=None, max_seqlen=None):
    """Routing from the block means that qk_norm_rope_pool() left in ``workspace``
    (q gives the shape only; its data is not read).  Same returns as route()."""
    desc = make_desc(q, None, cu_seqlens, max_seqlen)
    idx, cnt, totals, order = (route_outputs(q, cu_seqlens, max_seqlen) if out is None
                               else out)
    _check_lists(q, idx, cnt, order, cu_seqlens, max_seqlen)
    _check_buffer(totals, torch.int64, (2,), q.device, "totals")
    if workspace.device != q.device:
        raise ValueError("workspace must be on q's device")
    st = lib.sol_route_pooled(ctypes.byref(desc), ctypes.c_float(tau), int(sink),
                              ctypes.c_float(scale), idx.data_ptr(), cnt.data_ptr(),
                              totals.data_ptr(), order.data_ptr() if order is not None else None,
                              workspace.data_ptr(), _nbytes(workspace), _stream(q))
    _check(st, "sol_route_pooled")
    return idx, cnt, totals, order


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
