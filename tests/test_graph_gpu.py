"""The forward under HIP graph capture: every entry point allocates nothing and
clears its counters with kernels, so a captured forward replays correctly.

Each test captures the calls into a torch CUDA (HIP) graph, then replays it
several times with eager work in between (the outputs overwritten, new input
values copied into the captured buffers), and checks every replay bit for bit
against the eager calls on the same inputs.
"""

from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest

import synth
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sol():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import block_sparse_attention_sol_amd as s
    return s


def _capture(fn):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _lists_equal(idx_a, cnt_a, idx_b, cnt_b):
    import torch
    mask = torch.arange(idx_a.shape[-1], device=idx_a.device) < cnt_a[..., None]
    return torch.equal(cnt_a, cnt_b) and torch.equal(torch.where(mask, idx_a, 0),
                                                     torch.where(mask, idx_b, 0))


def test_route_and_attention_replay_in_a_graph(sol):
    import torch
    w = replace(synth.WORKLOADS["mid"], N=3001, H=4)
    inputs = [synth.make_qkv(replace(w, seed=s)) for s in (0, 1)]
    q, k, v = (to_dev(x) for x in inputs[0])
    ws = torch.empty(sol.route_workspace_bytes(q), dtype=torch.uint8, device="cuda")
    outs = sol.route_outputs(q)
    idx, cnt, totals, order = outs
    o = torch.empty_like(q)
    lse = torch.empty((1, w.H, w.N), dtype=torch.float32, device="cuda")

    def step():
        sol.route(q, k, w.tau, w.sink, workspace=ws, out=outs)
        sol.attn(q, k, v, idx, cnt, w.sink, out=o, lse_out=lse, order=order)

    refs = []
    for bits in inputs:                         # eager results for both input sets
        for dst, src in zip((q, k, v), bits):
            dst.copy_(to_dev(src))
        step()
        torch.cuda.synchronize()
        refs.append((idx.clone(), cnt.clone(), totals.clone(), o.clone(), lse.clone()))
    graph = _capture(step)
    for rep in range(4):
        which = rep % 2
        for dst, src in zip((q, k, v), inputs[which]):
            dst.copy_(to_dev(src))
        o.fill_(7.0)
        lse.fill_(-3.0)
        cnt.fill_(-1)
        totals.fill_(-5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        r_idx, r_cnt, r_tot, r_o, r_lse = refs[which]
        assert _lists_equal(idx, cnt, r_idx, r_cnt), rep
        assert torch.equal(totals, r_tot), rep
        assert torch.equal(o.view(torch.int16), r_o.view(torch.int16)), rep
        assert torch.equal(lse, r_lse), rep


def test_producer_path_and_dense_replay_in_a_graph(sol):
    import torch
    w = replace(synth.WORKLOADS["mid"], N=2500, H=3)
    q_bits, k_bits, v_bits = synth.make_qkv(w)
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    gq, gk = synth.norm_weights(w.D)
    cos, sin = synth.rope_tables(w.N, w.D)
    pargs = tuple(torch.from_numpy(x).to("cuda") for x in (gq, gk)) + (synth.NORM_EPS,) + \
        tuple(torch.from_numpy(x).to("cuda") for x in (cos, sin))
    qn, kn = torch.empty_like(q), torch.empty_like(k)
    ws = torch.empty(sol.route_workspace_bytes(q), dtype=torch.uint8, device="cuda")
    outs = sol.route_outputs(q)
    idx, cnt, totals, order = outs
    o, od = torch.empty_like(q), torch.empty_like(q)

    def step():
        sol.qk_norm_rope_pool(q, k, *pargs, sink=w.sink, out=(qn, kn), workspace=ws)
        sol.route_pooled(q, ws, 0.5, w.sink, out=outs)
        sol.attn(qn, kn, v, idx, cnt, w.sink, out=o, order=order)
        sol.attn_dense(qn, kn, v, out=od)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (qn, kn, idx, cnt, totals, o, od)]
    graph = _capture(step)
    for rep in range(3):
        for t in (qn, kn, o, od):
            t.fill_(5.0)
        cnt.fill_(-1)
        totals.fill_(-1)
        ws.fill_(255)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, exp in zip((qn, kn, o, od), (ref[0], ref[1], ref[5], ref[6])):
            assert torch.equal(got.view(torch.int16), exp.view(torch.int16)), rep
        assert _lists_equal(idx, cnt, ref[2], ref[3]), rep
        assert torch.equal(totals, ref[4]), rep
    assert int(ref[4][0]) > 0 and np.isfinite(ref[5].float().cpu().numpy()).all()


def test_packed_batch_replays_with_new_offsets(sol):
    """A captured packed-batch forward reads the row offsets from device memory
    when it runs, so replays with other sample lengths (same B, longest length
    and row count) need no recapture.  Each replay equals the eager calls on
    the same offsets bit for bit."""
    import torch
    H, D, S, N = 3, 128, 96, 1100
    base = synth.WORKLOADS["mid"]
    layouts = [[1000, 0, 640, 97], [64, 1100, 1, 572], [500, 500, 500, 237]]
    T = sum(layouts[0])
    assert all(sum(x) == T and max(x) <= N for x in layouts)
    calls = [replace(base, name=f"g{i}", N=n, H=H, D=D, sink=S, seed=40 + i)
             for i, n in enumerate(layouts[0])]
    q_bits, k_bits, v_bits, _ = synth.packed_batch(calls)
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    cu = torch.zeros(len(layouts[0]) + 1, dtype=torch.int32, device="cuda")
    vk = dict(cu_seqlens=cu, max_seqlen=N)
    ws = torch.empty(sol.route_workspace_bytes(q, **vk), dtype=torch.uint8, device="cuda")
    outs = sol.route_outputs(q, **vk)
    idx, cnt, totals, order = outs
    o = torch.empty_like(q)

    def set_offsets(lengths):
        cu.copy_(torch.tensor(np.cumsum([0] + lengths), dtype=torch.int32))

    def step():
        sol.route(q, k, base.tau, S, workspace=ws, out=outs, **vk)
        sol.attn(q, k, v, idx, cnt, S, out=o, order=order, **vk)

    refs = []
    for lengths in layouts:                     # eager results for every layout
        set_offsets(lengths)
        o.fill_(0.0)
        step()
        torch.cuda.synchronize()
        refs.append((idx.clone(), cnt.clone(), totals.clone(), o.clone()))
    set_offsets(layouts[0])
    graph = _capture(step)
    for rep in range(6):
        which = (rep + 1) % len(layouts)
        set_offsets(layouts[which])
        o.fill_(0.0)
        cnt.fill_(-1)
        totals.fill_(-5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        r_idx, r_cnt, r_tot, r_o = refs[which]
        assert _lists_equal(idx, cnt, r_idx, r_cnt), rep
        assert torch.equal(totals, r_tot), rep
        assert torch.equal(o.view(torch.int16), r_o.view(torch.int16)), rep
    assert not torch.equal(refs[0][2], refs[1][2])      # the layouts route differently
