"""GPU routing parity: lists, counts and totals from sol_route vs the oracle, bit for bit.

The GPU path is imported lazily so that collecting this file on a machine
without the built library (CPU-only runs use -m "not gpu") does not fail.
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


@pytest.fixture(scope="module")
def sol():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import block_sparse_attention_sol_amd as s
    return s


def _route_and_check(sol, q_bits, k_bits, N, S, tau, what):
    import torch
    q, k = to_dev(q_bits), to_dev(k_bits)
    idx, cnt, totals, order = sol.route(q, k, tau, S)
    torch.cuda.synchronize()
    idx, cnt, totals, order = idx.cpu().numpy(), cnt.cpu().numpy(), totals.cpu().numpy(), order.cpu().numpy()
    check_schedule(order, cnt)
    r = orc.route(synth.bf16_bits_to_f32(q_bits), synth.bf16_bits_to_f32(k_bits), N, S, tau)
    g = r.geom
    gsel = gpu_lists_to_mask(idx, cnt, g.NB)
    compare_masks(gsel, r)
    np.testing.assert_array_equal(cnt, r.cnt)
    assert int(totals[0]) == r.routed_pairs
    assert int(totals[1]) == r.attended_pairs
    B, _, H, _ = q_bits.shape
    dens = orc.densities(r, B, H)
    log(f"{what}: routed {dens['route'][0]}/{dens['route'][1]} "
        f"({dens['route'][0] / max(dens['route'][1], 1):.4%}), pairs {int(totals[1])}")
    return r


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_route_parity_small_configs(sol, name):
    w = synth.WORKLOADS[name]
    log(f"route parity {name}: B={w.B} N={w.N} H={w.H} D={w.D} S={w.sink} tau={w.tau}")
    q, k, _ = synth.make_qkv(w)
    _route_and_check(sol, q, k, w.N, w.sink, w.tau, name)


def test_route_parity_page_shape(sol):
    w = synth.WORKLOADS["page"]
    log(f"route parity page: N={w.N} H={w.H} S={w.sink} tau={w.tau}")
    q, k, _ = synth.make_qkv(w)
    r = _route_and_check(sol, q, k, w.N, w.sink, w.tau, "page")
    dens = r.routed_pairs / (w.B * w.H * r.geom.NB * r.geom.ncand)
    assert 0.18 <= dens <= 0.20


def test_route_parity_page_dense_selects_all(sol):
    w = synth.WORKLOADS["page"]
    q, k, _ = synth.make_qkv(replace(w, H=4))
    r = _route_and_check(sol, q, k, w.N, w.sink, math.inf, "page tau=inf")
    assert r.sel[..., r.geom.j0:].all()


def test_route_parity_varlen_calls(sol):
    for w in synth.varlen_calls()[:3]:
        log(f"route parity {w.name}: N={w.N}")
        q, k, _ = synth.make_qkv(replace(w, H=4))
        _route_and_check(sol, q, k, w.N, w.sink, w.tau, w.name)


EDGE = [
    # B, N, H, D, S, tau
    (1, 1, 1, 64, 0, 1.0),
    (1, 37, 2, 128, 0, 0.5),
    (2, 64, 1, 64, 0, 0.0),
    (1, 65, 3, 128, 1, 0.3),
    (1, 129, 1, 64, 64, 0.0),
    (2, 300, 2, 128, 63, 0.7),
    (1, 300, 2, 64, 65, 0.7),
    (1, 1000, 3, 128, 951, 0.4),
    (1, 1000, 2, 64, 1000, 1.0),
    (1, 700, 2, 128, 5000, 1.0),
    (1, 2047, 2, 128, 130, math.inf),
    (1, 70000, 1, 128, 951, 0.5),        # more than 1024 candidates: two slots per lane
]


@pytest.mark.parametrize("B,N,H,D,S,tau", EDGE)
def test_route_parity_edge_shapes(sol, B, N, H, D, S, tau):
    log(f"route edge B={B} N={N} H={H} D={D} S={S} tau={tau}")
    w = synth.Workload("edge", B=B, N=N, H=H, D=D, sink=S, tau=tau, kind="field", alpha=1.0,
                       seed=N + S)
    q, k, _ = synth.make_qkv(w)
    _route_and_check(sol, q, k, N, S, tau, "edge")


def _route_sweep_cases(n=8, seed=20261203):
    """Seeded random routing shapes up to N = 20000 (NB up to 313, so one or
    two candidate slots per lane), sink mode c % 4 and tau mode c % 2."""
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        N = int(rng.integers(2, 20000))
        S = [0, int(rng.integers(1, N)), min(951, N - 1), N + int(rng.integers(0, 100))][c % 4]
        tau = [float(rng.uniform(0.0, 0.6)), float(rng.uniform(0.6, 3.0))][c % 2]
        cases.append((int(rng.integers(1, 3)), N, int(rng.integers(1, 5)),
                      int(rng.choice([64, 128])), S, tau, 2000 + c))
    return cases


@pytest.mark.parametrize("B,N,H,D,S,tau,seed", _route_sweep_cases())
def test_route_parity_seeded_sweep(sol, B, N, H, D, S, tau, seed):
    """Lists, counts, totals and the schedule bit-exact on seeded random shapes."""
    log(f"route sweep B={B} N={N} H={H} D={D} S={S} tau={tau:.4g} seed={seed}")
    w = synth.Workload("sweep", B=B, N=N, H=H, D=D, sink=S, tau=tau,
                       kind="field" if seed % 2 else "tiny", alpha=1.0, seed=seed)
    q, k, _ = synth.make_qkv(w)
    _route_and_check(sol, q, k, N, S, tau, "sweep")


def test_route_strided_views_match_contiguous(sol):
    """Q and K as views of one merged [B, N, 3, H, D] projection."""
    import torch
    w = replace(synth.WORKLOADS["mid"], N=3000, H=4)
    q_bits, k_bits, v_bits = synth.make_qkv(w)
    qkv = torch.stack([to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)], dim=2)   # [B, N, 3, H, D]
    q, k = qkv[:, :, 0], qkv[:, :, 1]
    assert not q.is_contiguous()
    i1, c1, t1, _ = sol.route(q, k, w.tau, w.sink)
    i2, c2, t2, _ = sol.route(to_dev(q_bits), to_dev(k_bits), w.tau, w.sink)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(t1, t2)
    NB = sol.num_blocks(w.N)
    m1 = gpu_lists_to_mask(i1.cpu().numpy(), c1.cpu().numpy(), NB)
    m2 = gpu_lists_to_mask(i2.cpu().numpy(), c2.cpu().numpy(), NB)
    assert (m1 == m2).all()


def test_route_is_deterministic_and_needs_no_rebuild(sol):
    """Two different lengths on one build, twice each: identical results."""
    import torch
    for N in (5000, 5003):
        w = replace(synth.WORKLOADS["mid"], N=N, H=2)
        q_bits, k_bits, _ = synth.make_qkv(w)
        q, k = to_dev(q_bits), to_dev(k_bits)
        a = sol.route(q, k, w.tau, w.sink)
        b = sol.route(q, k, w.tau, w.sink)
        torch.cuda.synchronize()
        assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
