"""GPU parity of the QK-norm + RoPE producer and of routing from its block means.

sol_qk_norm_rope_pool's bf16 outputs are compared bit for bit with the
oracle's float32 mirror (both sides take every rounding in the same float32
order, so the bf16 outputs are integers to compare).  sol_route_pooled's
lists, counts and totals are compared bit for bit with the oracle's routing
of the mirror's outputs, and with sol_route run on the producer's own outputs
(the block means must be exactly the routing pool of those outputs).
"""

from __future__ import annotations

import math
from dataclasses import replace

import numpy as np
import pytest

import synth
from oracle import oracle as orc
from tests.helpers import check_schedule, compare_masks, gpu_lists_to_mask, log, to_dev

pytestmark = pytest.mark.gpu

EPS = synth.NORM_EPS


@pytest.fixture(scope="module")
def sol():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import block_sparse_attention_sol_amd as s
    return s


def _f32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda")


def _bits(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _weights(N, D, rope):
    gq, gk = synth.norm_weights(D)
    cos, sin = synth.rope_tables(N, D) if rope else (None, None)
    return gq, gk, cos, sin


def _route_vs_oracle(sol, idx, cnt, totals, order, q_ref_bits, k_ref_bits, N, S, tau):
    import torch
    torch.cuda.synchronize()
    idx, cnt, totals, order = (x.cpu().numpy() for x in (idx, cnt, totals, order))
    check_schedule(order, cnt)
    r = orc.route(synth.bf16_bits_to_f32(q_ref_bits), synth.bf16_bits_to_f32(k_ref_bits), N, S, tau)
    compare_masks(gpu_lists_to_mask(idx, cnt, r.geom.NB), r)
    np.testing.assert_array_equal(cnt, r.cnt)
    assert int(totals[0]) == r.routed_pairs and int(totals[1]) == r.attended_pairs
    return r


def _same_route(a, b):
    import torch
    idx_a, cnt_a, tot_a, _ = a
    idx_b, cnt_b, tot_b, _ = b
    assert torch.equal(cnt_a, cnt_b) and torch.equal(tot_a, tot_b)
    mask = torch.arange(idx_a.shape[-1], device=idx_a.device) < cnt_a[..., None]
    assert torch.equal(torch.where(mask, idx_a, 0), torch.where(mask, idx_b, 0))


@pytest.mark.parametrize("name,N,H,D,S,rope", [
    ("tiny", 1024, 4, 64, 64, True),
    ("mid", 3001, 3, 128, 256, True),
    ("mid", 2000, 5, 128, 951, False),
    ("mid", 1, 2, 128, 0, True),
    ("tiny", 130, 3, 64, 200, True),          # S >= N: no candidates
    ("mid", 4097, 2, 128, 65, True),
])
def test_producer_bit_exact_and_routing_from_means(sol, name, N, H, D, S, rope):
    w = replace(synth.WORKLOADS[name], N=N, H=H, D=D, sink=S)
    q_bits, k_bits, _ = synth.make_qkv(w)
    gq, gk, cos, sin = _weights(N, D, rope)
    q, k = to_dev(q_bits), to_dev(k_bits)
    q_out, k_out, ws = sol.qk_norm_rope_pool(q, k, _f32(gq), _f32(gk), EPS,
                                             None if cos is None else _f32(cos),
                                             None if sin is None else _f32(sin), sink=S)
    got = sol.route_pooled(q, ws, w.tau, S)
    q_ref = orc.qk_norm_rope(q_bits, gq, EPS, cos, sin)
    k_ref = orc.qk_norm_rope(k_bits, gk, EPS, cos, sin)
    np.testing.assert_array_equal(_bits(q_out), q_ref)
    np.testing.assert_array_equal(_bits(k_out), k_ref)
    r = _route_vs_oracle(sol, *got, q_ref, k_ref, N, S, w.tau)
    # the means are exactly the routing pool of the outputs
    _same_route(got, sol.route(q_out, k_out, w.tau, S))
    log(f"producer {name} N={N} H={H} D={D} S={S} rope={rope}: routed {r.routed_pairs}")


def test_producer_in_place(sol):
    import torch
    w = replace(synth.WORKLOADS["mid"], N=1500, H=3)
    q_bits, k_bits, _ = synth.make_qkv(w)
    gq, gk, cos, sin = _weights(w.N, w.D, True)
    q, k = to_dev(q_bits), to_dev(k_bits)
    args = (_f32(gq), _f32(gk), EPS, _f32(cos), _f32(sin))
    q_sep, k_sep, ws_sep = sol.qk_norm_rope_pool(q, k, *args, sink=w.sink)
    q_sep, k_sep, ws_sep = q_sep.clone(), k_sep.clone(), ws_sep.clone()
    q_in, k_in, ws = sol.qk_norm_rope_pool(q, k, *args, sink=w.sink, out=(q, k))
    torch.cuda.synchronize()
    assert q_in.data_ptr() == q.data_ptr()
    assert torch.equal(q.view(torch.int16), q_sep.view(torch.int16))
    assert torch.equal(k.view(torch.int16), k_sep.view(torch.int16))
    _same_route(sol.route_pooled(q, ws, w.tau, w.sink), sol.route_pooled(q, ws_sep, w.tau, w.sink))


def test_producer_strided_views(sol):
    """Q and K as views of one merged [B, N, 3, H, D] projection, outputs into
    another merged buffer: same bits as contiguous inputs and outputs."""
    import torch
    w = replace(synth.WORKLOADS["mid"], N=700, H=4)
    q_bits, k_bits, _ = synth.make_qkv(w)
    gq, gk, cos, sin = _weights(w.N, w.D, True)
    args = (_f32(gq), _f32(gk), EPS, _f32(cos), _f32(sin))
    q, k = to_dev(q_bits), to_dev(k_bits)
    merged = torch.empty((1, w.N, 3, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    merged[:, :, 0] = q
    merged[:, :, 1] = k
    outm = torch.zeros((1, w.N, 2, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    sol.qk_norm_rope_pool(merged[:, :, 0], merged[:, :, 1], *args, sink=w.sink,
                          out=(outm[:, :, 0], outm[:, :, 1]))
    q_out, k_out, _ = sol.qk_norm_rope_pool(q, k, *args, sink=w.sink)
    torch.cuda.synchronize()
    assert torch.equal(outm[:, :, 0].contiguous().view(torch.int16), q_out.view(torch.int16))
    assert torch.equal(outm[:, :, 1].contiguous().view(torch.int16), k_out.view(torch.int16))


def test_producer_merged_views_default_outputs(sol):
    """Q and K as views of one merged [B, N, 3, H, D] projection with out=None:
    the binding allocates dense outputs and must describe them by their own
    strides (not the inputs'), so outputs and block means equal the
    contiguous call's bit for bit."""
    import torch
    w = replace(synth.WORKLOADS["mid"], N=700, H=4)
    q_bits, k_bits, _ = synth.make_qkv(w)
    gq, gk, cos, sin = _weights(w.N, w.D, True)
    args = (_f32(gq), _f32(gk), EPS, _f32(cos), _f32(sin))
    q, k = to_dev(q_bits), to_dev(k_bits)
    merged = torch.empty((1, w.N, 3, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    merged[:, :, 0] = q
    merged[:, :, 1] = k
    qv, kv = merged[:, :, 0], merged[:, :, 1]
    q_m, k_m, ws_m = sol.qk_norm_rope_pool(qv, kv, *args, sink=w.sink)
    assert q_m.is_contiguous() and k_m.is_contiguous()
    q_c, k_c, ws_c = sol.qk_norm_rope_pool(q, k, *args, sink=w.sink)
    torch.cuda.synchronize()
    assert torch.equal(q_m.view(torch.int16), q_c.view(torch.int16))
    assert torch.equal(k_m.view(torch.int16), k_c.view(torch.int16))
    # the block means: the routing from them is the same bit for bit
    _same_route(sol.route_pooled(qv, ws_m, w.tau, w.sink), sol.route_pooled(q, ws_c, w.tau, w.sink))


def test_producer_packed_batch(sol):
    import torch
    lengths, H, D, S = [1000, 0, 64, 777, 2053, 130, 96], 3, 128, 96
    base = synth.WORKLOADS["mid"]
    calls = [replace(base, name=f"p{i}", N=n, H=H, D=D, sink=S, seed=i)
             for i, n in enumerate(lengths)]
    q_bits, k_bits, _, cu = synth.packed_batch(calls)
    gq, gk, cos, sin = _weights(max(lengths), D, True)
    q, k = to_dev(q_bits), to_dev(k_bits)
    cud = torch.tensor(np.asarray(cu, np.int32), device="cuda")
    vk = dict(cu_seqlens=cud, max_seqlen=max(lengths))
    q_out, k_out, ws = sol.qk_norm_rope_pool(q, k, _f32(gq), _f32(gk), EPS, _f32(cos), _f32(sin),
                                             sink=S, **vk)
    idx, cnt, totals, order = sol.route_pooled(q, ws, base.tau, S, **vk)
    q_ref = orc.qk_norm_rope_packed(q_bits, cu, gq, EPS, cos, sin)
    k_ref = orc.qk_norm_rope_packed(k_bits, cu, gk, EPS, cos, sin)
    np.testing.assert_array_equal(_bits(q_out), q_ref)
    np.testing.assert_array_equal(_bits(k_out), k_ref)
    _same_route((idx, cnt, totals, order), sol.route(q_out, k_out, base.tau, S, **vk))
    routes = orc.route_packed(synth.bf16_bits_to_f32(q_ref), synth.bf16_bits_to_f32(k_ref), cu, S,
                              base.tau)
    cnt_h, idx_h = cnt.cpu().numpy(), idx.cpu().numpy()
    for b, r in enumerate(routes):
        if r is None:
            continue
        nb = r.geom.NB
        compare_masks(gpu_lists_to_mask(idx_h[b:b + 1, :, :nb], cnt_h[b:b + 1, :, :nb], nb), r)
    # rows after the last sample (T > cu[B]) are neither read into the means
    # nor written: the same call with 50 extra rows gives the same outputs
    pad = 50
    qp, kp = (torch.cat([x, torch.full((pad, H, D), 3.0, dtype=x.dtype, device=x.device)])
              for x in (q, k))
    sentinel = torch.full_like(qp, -2.0)
    qo, ko = sentinel.clone(), sentinel.clone()
    _, _, wsp = sol.qk_norm_rope_pool(qp, kp, _f32(gq), _f32(gk), EPS, _f32(cos), _f32(sin),
                                      sink=S, out=(qo, ko), **vk)
    got_p = sol.route_pooled(qp, wsp, base.tau, S, **vk)
    torch.cuda.synchronize()
    T = q.shape[0]
    assert torch.equal(qo[:T].view(torch.int16), q_out.view(torch.int16))
    assert torch.equal(ko[:T].view(torch.int16), k_out.view(torch.int16))
    assert torch.equal(qo[T:], sentinel[T:]) and torch.equal(ko[T:], sentinel[T:])
    _same_route(got_p, (idx, cnt, totals, order))


def test_producer_page_shape(sol):
    """The pages' shape [1, 38247, 56, 128]: outputs of every head bit-exact, the
    whole routed mask equal to the oracle's on the mirror's outputs, and the
    producer timed against its HBM bytes."""
    import torch
    w = synth.WORKLOADS["page_fused"]
    q_bits, k_bits, _ = synth.make_qkv(w)
    gq, gk, cos, sin = _weights(w.N, w.D, True)
    q, k = to_dev(q_bits), to_dev(k_bits)
    args = (_f32(gq), _f32(gk), EPS, _f32(cos), _f32(sin))
    q_out, k_out, ws = sol.qk_norm_rope_pool(q, k, *args, sink=w.sink)
    got = sol.route_pooled(q, ws, w.tau, w.sink)
    q_ref = orc.qk_norm_rope(q_bits, gq, EPS, cos, sin)
    k_ref = orc.qk_norm_rope(k_bits, gk, EPS, cos, sin)
    np.testing.assert_array_equal(_bits(q_out), q_ref)
    np.testing.assert_array_equal(_bits(k_out), k_ref)
    r = _route_vs_oracle(sol, *got, q_ref, k_ref, w.N, w.sink, w.tau)
    _same_route(got, sol.route(q_out, k_out, w.tau, w.sink))
    dens = orc.densities(r, 1, w.H)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        sol.qk_norm_rope_pool(q, k, *args, sink=w.sink, out=(q_out, k_out), workspace=ws)
    s.record()
    for _ in range(10):
        sol.qk_norm_rope_pool(q, k, *args, sink=w.sink, out=(q_out, k_out), workspace=ws)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / 10
    nbytes = 4 * q.numel() * 2
    log(f"producer page: {ms:.3f} ms, {nbytes / (ms * 1e-3) / 1e9:.0f} GB/s over Q, K in and out; "
        f"route density after the producer {dens['route'][0] / dens['route'][1]:.4%}")
    assert math.isfinite(ms)
