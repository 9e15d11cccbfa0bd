"""sol_route_noalloc (routing with the library's static per-GPU scratch instead
of a caller workspace) against sol_route with a workspace, through the C ABI.

Routing is integer work, so the bar is bit for bit: lists, counts and totals
equal; the schedule is valid (a permutation with non-increasing counts;
blocks of equal count may come in any order).  Three calls in a row share the
one scratch array: the pages' shape (34.3 MB of scratch, near the 48 MiB
limit), then a smaller and a still smaller call, so each later call runs on
what the earlier one left behind.  (A call that needs more scratch than the
array holds is refused on the host; tests/test_abi.py checks that without a
GPU, so that a regressed check cannot write past the array here.)
"""

from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest

import synth
from tests.helpers import check_schedule, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sol():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import block_sparse_attention_sol_amd as s
    return s


def _same(sol, a, b):
    import torch
    idx_a, cnt_a, tot_a, ord_a = a
    idx_b, cnt_b, tot_b, ord_b = b
    torch.cuda.synchronize()
    assert torch.equal(cnt_a, cnt_b) and torch.equal(tot_a, tot_b)
    mask = torch.arange(idx_a.shape[-1], device=idx_a.device) < cnt_a[..., None]
    assert torch.equal(torch.where(mask, idx_a, 0), torch.where(mask, idx_b, 0))
    check_schedule(ord_a.cpu().numpy(), cnt_a.cpu().numpy())
    check_schedule(ord_b.cpu().numpy(), cnt_b.cpu().numpy())


def test_noalloc_equals_route_on_three_calls_in_a_row(sol):
    import torch
    page = synth.WORKLOADS["page"]
    mid = synth.WORKLOADS["mid"]
    calls = [page, replace(mid, N=3001, H=3), replace(synth.WORKLOADS["tiny"], N=700, H=2)]
    for w in calls:
        q_bits, k_bits, _ = synth.make_qkv(w)
        q, k = to_dev(q_bits), to_dev(k_bits)
        need = sol.route_workspace_bytes(q)
        log(f"noalloc {w.name} B={w.B} N={w.N} H={w.H} D={w.D}: workspace {need} bytes")
        assert need <= sol.NOALLOC_SCRATCH_BYTES
        # outputs start as garbage, so nothing can pass by being left over
        out = sol.route_outputs(q)
        for t in out:
            t.fill_(-7)
        got = sol.route_noalloc(q, k, w.tau, w.sink, out=out)
        ref = sol.route(q, k, w.tau, w.sink)
        _same(sol, got, ref)
        # and a second call on the same scratch, with another tau
        got2 = sol.route_noalloc(q, k, w.tau * 0.5, w.sink)
        ref2 = sol.route(q, k, w.tau * 0.5, w.sink)
        _same(sol, got2, ref2)
        log(f"noalloc {w.name}: equal to sol_route, routed {int(got[2][0].item())} pairs")
        del q, k
    torch.cuda.synchronize()


def test_noalloc_routing_replays_in_a_graph(sol):
    """The callers the entry point is for: routing captured into a HIP graph
    with no allocation.  The graph is replayed four times, with new input
    values copied into the captured buffers and the outputs overwritten in
    between (eager work between replays), and every replay equals eager
    sol_route on the same inputs bit for bit."""
    import torch
    w = replace(synth.WORKLOADS["mid"], N=3001, H=4)
    inputs = [synth.make_qkv(replace(w, seed=s))[:2] for s in (0, 1)]
    q, k = (to_dev(x) for x in inputs[0])
    outs = sol.route_outputs(q)

    def step():
        sol.route_noalloc(q, k, w.tau, w.sink, out=outs)

    refs = []
    for bits in inputs:
        for dst, src in zip((q, k), bits):
            dst.copy_(to_dev(src))
        refs.append(sol.route(q, k, w.tau, w.sink))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        which = rep % 2
        for dst, src in zip((q, k), inputs[which]):
            dst.copy_(to_dev(src))
        for t in outs:
            t.fill_(-3)
        graph.replay()
        torch.cuda.synchronize()
        _same(sol, outs, refs[which])
        log(f"noalloc graph replay {rep}: equal to eager sol_route on input set {which}")


def test_noalloc_packed_batch_equals_route(sol):
    """A packed variable-length batch (an empty sample, one inside the sink,
    one exactly one block, ragged tails) through the static scratch equals
    sol_route on the same batch bit for bit, at two thresholds."""
    import torch
    base = synth.WORKLOADS["mid"]
    lengths = [1000, 0, 64, 777, 2053, 130, 96]
    calls = [replace(base, name=f"packed{k}", N=n, H=3, D=128, sink=96, seed=k)
             for k, n in enumerate(lengths)]
    q_bits, k_bits, _, cu = synth.packed_batch(calls)
    q, k = to_dev(q_bits), to_dev(k_bits)
    cu_d = torch.tensor(np.asarray(cu, dtype=np.int32), device="cuda")
    vk = {"cu_seqlens": cu_d, "max_seqlen": max(lengths)}
    log(f"noalloc packed batch lengths {lengths}, H=3, D=128, sink 96")
    for tau in (base.tau, base.tau * 0.5):
        out = sol.route_outputs(q, **vk)
        for t in out:
            t.fill_(-7)
        got = sol.route_noalloc(q, k, tau, 96, out=out, **vk)
        ref = sol.route(q, k, tau, 96, **vk)
        _same(sol, got, ref)
        log(f"noalloc packed tau={tau:.4f}: equal to sol_route, routed {int(got[2][0].item())} pairs")
