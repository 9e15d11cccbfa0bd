"""GPU attention parity: sol_attn_fwd / sol_attn_dense_fwd vs the float64 oracle.

Tolerance (bf16 output vs float64): max-abs <= 1e-2 and L2-relative <= 5e-3
over the valid rows compared.  Routing lists come from the GPU route, whose
parity with the oracle is checked first in each test, so both sides attend to
the same keys.
"""

from __future__ import annotations

import math
from dataclasses import replace

import numpy as np
import pytest

import synth
from oracle import oracle as orc
from tests.helpers import (LSE_MAX_ABS, assert_close, bf16_tensor_to_f64, compare_masks,
                           gpu_lists_to_mask, log, sample_blocks, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sol():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import block_sparse_attention_sol_amd as s
    return s


def _run(sol, w: synth.Workload, blocks=None, dense=False, tau=None, inputs=None):
    """GPU route + attention on workload w, compared with the oracle on `blocks` (or all).
    ``inputs`` are w's (q, k, v) bits when the caller already drew them."""
    import torch
    tau = w.tau if tau is None else tau
    q_bits, k_bits, v_bits = synth.make_qkv(w) if inputs is None else inputs
    q32, k32, v32 = (synth.bf16_bits_to_f32(x) for x in (q_bits, k_bits, v_bits))
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    if dense:
        o, lse = sol.attn_dense(q, k, v, return_lse=True)
        g = orc.geometry(w.N, w.N)
        O, L = orc.dense_attention(q32, k32, v32, blocks=blocks)
    else:
        idx, cnt, totals, order = sol.route(q, k, tau, w.sink)
        o, lse = sol.attn(q, k, v, idx, cnt, w.sink, return_lse=True, order=order)
        r = orc.route(q32, k32, w.N, w.sink, tau)
        g = r.geom
        gsel = gpu_lists_to_mask(idx.cpu().numpy(), cnt.cpu().numpy(), g.NB)
        compare_masks(gsel, r)
        O, L = orc.attention(q32, k32, v32, r.sel, g, blocks=blocks)
    torch.cuda.synchronize()
    got = bf16_tensor_to_f64(o)
    lse = lse.cpu().numpy().astype(np.float64)
    if blocks is None:
        ref, gv = O, got
        lref, lgot = L, lse
    else:
        ref, gv = [], []
        lref, lgot = [], []
        for b, h, i in blocks:
            rr = g.q_rows(i)
            ref.append(O[b, rr.start:rr.stop, h])
            gv.append(got[b, rr.start:rr.stop, h])
            lref.append(L[b, h, rr.start:rr.stop])
            lgot.append(lse[b, h, rr.start:rr.stop])
        ref, gv = np.concatenate(ref), np.concatenate(gv)
        lref, lgot = np.concatenate(lref), np.concatenate(lgot)
    e = assert_close(gv, ref, f"{w.name} O")
    lerr = float(np.abs(lgot - lref).max())
    log(f"{w.name} LSE max-abs {lerr:.3e}")
    assert lerr <= LSE_MAX_ABS
    return e


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_attention_parity_small_configs_all_rows(sol, name):
    w = synth.WORKLOADS[name]
    log(f"attention parity {name} (all rows)")
    _run(sol, w)


# heads compared on every query block at the pages' shape: the first and
# last head and two between them
PAGE_HEADS = (0, 19, 38, 55)


@pytest.fixture(scope="module")
def page_inputs():
    """The pages' shape [1, 38247, 56, 128] (sparse and dense share the tensors)."""
    return synth.make_qkv(synth.WORKLOADS["page"])


def test_attention_parity_page_shape_all_blocks_of_four_heads(sol, page_inputs):
    """Every query block (598 each, the ragged last one and the sink straddle
    block included) of four of the 56 heads, and in every other head the
    first, the straddle (14), the first fully routable (15) and the last
    block plus four seeded others, after a bit-exact comparison of the whole
    routing mask."""
    w = synth.WORKLOADS["page"]
    g = orc.geometry(w.N, w.sink)
    blocks = [(0, h, i) for h in PAGE_HEADS for i in range(g.NB)]
    rng = np.random.default_rng(56)
    fixed = {0, g.S // 64, g.S // 64 + 1, g.NB - 1}
    for h in range(w.H):
        if h in PAGE_HEADS:
            continue
        pick = set(fixed)
        while len(pick) < 8:
            pick.add(int(rng.integers(g.NB)))
        blocks += [(0, h, i) for i in sorted(pick)]
    log(f"attention parity page, all query blocks of heads {PAGE_HEADS} and 8 of each "
        f"other head: {len(blocks)} blocks")
    _run(sol, w, blocks=blocks, inputs=page_inputs)


def test_dense_parity_page_shape_all_blocks_of_one_head(sol, page_inputs):
    w = synth.WORKLOADS["page_dense"]
    g = orc.geometry(w.N, w.N)
    blocks = [(0, 27, i) for i in range(g.NB)]
    log(f"dense parity page, all {len(blocks)} query blocks of head 27")
    _run(sol, w, blocks=blocks, dense=True, inputs=page_inputs)


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
    (1, 700, 2, 128, 5000, 1.0),
    (1, 2047, 2, 128, 130, math.inf),
]


@pytest.mark.parametrize("B,N,H,D,S,tau", EDGE)
def test_attention_parity_edge_shapes(sol, B, N, H, D, S, tau):
    log(f"attention edge B={B} N={N} H={H} D={D} S={S} tau={tau}")
    w = synth.Workload("edge", B=B, N=N, H=H, D=D, sink=S, tau=tau, kind="field", alpha=1.0,
                       seed=N + S)
    _run(sol, w)


def _sweep_cases(n=12, seed=20261202):
    """Seeded random shapes with ragged N.  Case c takes sink mode c % 4 (none,
    random, 951 or the nearest below N, at least N: every key a sink key) and
    tau mode c % 3 (0: only the maximum and the diagonal, random, +inf: every
    candidate), so the twelve cases cover every pair of modes."""
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        N = int(rng.integers(2, 2600))
        S = [0, int(rng.integers(1, N)), min(951, N - 1), N + int(rng.integers(0, 100))][c % 4]
        tau = [0.0, float(rng.uniform(0.05, 2.5)), math.inf][c % 3]
        cases.append((int(rng.integers(1, 3)), N, int(rng.integers(1, 4)),
                      int(rng.choice([64, 128])), S, tau, 1000 + c))
    return cases


@pytest.mark.parametrize("B,N,H,D,S,tau,seed", _sweep_cases())
def test_attention_parity_seeded_sweep(sol, B, N, H, D, S, tau, seed):
    """Routed masks bit-exact and every valid row within tolerance on seeded
    random shapes (both generators' structure, either head width)."""
    log(f"attention sweep B={B} N={N} H={H} D={D} S={S} tau={tau:.4g} seed={seed}")
    kind = "field" if seed % 2 else "tiny"
    w = synth.Workload("sweep", B=B, N=N, H=H, D=D, sink=S, tau=tau, kind=kind, alpha=1.0,
                       seed=seed)
    _run(sol, w)


@pytest.fixture(scope="module")
def maxcand_inputs():
    w = synth.Workload("maxcand", B=1, N=263000, H=1, D=128, sink=951, tau=1.0, kind="field",
                       alpha=1.0, seed=11)
    return w, synth.make_qkv(w)


@pytest.mark.parametrize("tau", [math.inf, 0.5])
def test_maximum_candidates(sol, maxcand_inputs, tau):
    """The largest routing problem the library accepts: 4096 candidate key
    blocks per query block (N = 263000 with the 951-token sink, a ragged tail
    of 24 rows).  At tau = inf every list holds all 4096 candidates, the most
    a walk can take; routing is compared bit for bit and attention on sampled
    blocks (first, straddle, last included)."""
    w, inputs = maxcand_inputs
    g = orc.geometry(w.N, w.sink)
    assert g.ncand == 4096
    _run(sol, w, blocks=sample_blocks(g, 1, 1, 12, seed=5), tau=tau, inputs=inputs)


def test_maximum_candidates_head_dim_64(sol):
    """The 4096-candidate limit at D = 64 and two heads: routing bit for bit,
    attention on sampled blocks of both heads (first, straddle, last
    included)."""
    w = synth.Workload("maxcand64", B=1, N=263000, H=2, D=64, sink=951, tau=0.5, kind="field",
                       alpha=1.0, seed=12)
    g = orc.geometry(w.N, w.sink)
    assert g.ncand == 4096
    _run(sol, w, blocks=sample_blocks(g, 1, 2, 12, seed=6))


@pytest.mark.parametrize("N,D", [(1, 64), (200, 128), (1000, 64), (3001, 128)])
def test_dense_parity_edge_shapes(sol, N, D):
    w = synth.Workload("dense_edge", B=1, N=N, H=2, D=D, sink=0, tau=math.inf, kind="field",
                       alpha=1.0, seed=N)
    _run(sol, w, dense=True)


def test_density_one_sparse_equals_dense_bitwise(sol):
    import torch
    w = replace(synth.WORKLOADS["mid"], N=4000, H=4)
    q_bits, k_bits, v_bits = synth.make_qkv(w)
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    idx, cnt, _, order = sol.route(q, k, math.inf, w.sink)
    o1 = sol.attn(q, k, v, idx, cnt, w.sink, order=order)
    o2 = sol.attn_dense(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_schedule_changes_no_output_bit(sol):
    """The routing schedule (longest list first) only reorders work: outputs are
    bit-identical with it, without it, and with a reversed schedule."""
    import torch
    w = replace(synth.WORKLOADS["mid"], N=5000, H=3)
    q_bits, k_bits, v_bits = synth.make_qkv(w)
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    idx, cnt, _, order = sol.route(q, k, w.tau, w.sink)
    outs = [sol.attn(q, k, v, idx, cnt, w.sink, order=o, return_lse=True)
            for o in (order, None, order.flip(-1).contiguous())]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def test_padding_rows_contribute_exactly_zero(sol):
    """Rows past N hold NaN or 0 in a 64-aligned allocation: outputs bit-identical."""
    import torch
    w = replace(synth.WORKLOADS["mid"], N=3000 + 17, H=3)
    Np = 64 * sol.num_blocks(w.N)
    q_bits, k_bits, v_bits = synth.make_qkv(w)
    outs = []
    for fill in (0.0, float("nan")):
        bufs = []
        for bits in (q_bits, k_bits, v_bits):
            t = torch.full((w.B, Np, w.H, w.D), fill, dtype=torch.bfloat16, device="cuda")
            t[:, : w.N] = to_dev(bits)
            bufs.append(t[:, : w.N])
        q, k, v = bufs
        idx, cnt, tot, order = sol.route(q, k, w.tau, w.sink)
        o_full = torch.full((w.B, Np, w.H, w.D), fill, dtype=torch.bfloat16, device="cuda")
        o = sol.attn(q, k, v, idx, cnt, w.sink, out=o_full[:, : w.N], order=order)
        od = sol.attn_dense(q, k, v)
        torch.cuda.synchronize()
        outs.append((o.clone(), od.clone(), cnt.clone(), tot.clone(), o_full[:, w.N:].clone()))
    (a, ad, ca, ta, pa), (b, bd, cb, tb, pb) = outs
    assert torch.isfinite(a.float()).all() and torch.isfinite(ad.float()).all()
    assert torch.equal(a, b) and torch.equal(ad, bd) and torch.equal(ca, cb) and torch.equal(ta, tb)
    # rows past N are never written
    assert (pa.float() == 0).all() and torch.isnan(pb.float()).all()


def test_constant_values_and_zero_queries(sol):
    import torch
    w = replace(synth.WORKLOADS["mid"], N=2000, H=2)
    q_bits, k_bits, v_bits = synth.make_qkv(w)
    q, k = to_dev(q_bits), to_dev(k_bits)
    idx, cnt, _, order = sol.route(q, k, w.tau, w.sink)
    v = torch.full_like(q, 0.375)
    o = sol.attn(q, k, v, idx, cnt, w.sink, order=order)
    torch.cuda.synchronize()
    assert (o.float() - 0.375).abs().max().item() <= 1e-2
    # Q = 0: the mean of the attended values (oracle closed form)
    vz = to_dev(v_bits)
    oz = sol.attn(torch.zeros_like(q), k, vz, idx, cnt, w.sink, order=order)
    torch.cuda.synchronize()
    r = orc.route(synth.bf16_bits_to_f32(q_bits), synth.bf16_bits_to_f32(k_bits), w.N, w.sink, w.tau)
    O, _ = orc.attention(np.zeros((w.B, w.N, w.H, w.D), np.float32), synth.bf16_bits_to_f32(k_bits),
                         synth.bf16_bits_to_f32(v_bits), r.sel, r.geom)
    assert_close(bf16_tensor_to_f64(oz), O, "zero queries")


def test_strided_qkv_views_and_output(sol):
    import torch
    w = replace(synth.WORKLOADS["mid"], N=2500, H=4)
    q_bits, k_bits, v_bits = synth.make_qkv(w)
    qkv = torch.stack([to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)], dim=2)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    idx, cnt, _, order = sol.route(q, k, w.tau, w.sink)
    obuf = torch.zeros((w.B, w.N, w.H, 2 * w.D), dtype=torch.bfloat16, device="cuda")
    o = sol.attn(q, k, v, idx, cnt, w.sink, out=obuf[..., : w.D], order=order)
    ref = sol.attn(to_dev(q_bits), to_dev(k_bits), to_dev(v_bits), idx, cnt, w.sink, order=order)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
    assert (obuf[..., w.D:].float() == 0).all()


def test_varlen_sixteen_lengths_parity_and_stable_time(sol):
    """The variable-length workload: 16 seeded calls with N in [36000, 40000],
    H = 14, on the one ahead-of-time build.
    - Parity on every call: the whole routing mask (all 14 heads) bit for
      bit, counts and totals exact, and O and LSE on 16 sampled query blocks
      (the first, straddle and last blocks among them).
    - No rebuild: the time per effective FLOP (best of 5 repetitions per
      call) stays within 10% of the median over the calls, and the first
      call is no compile-time outlier (a 12-14 s JIT per new length would
      blow both by orders of magnitude)."""
    import torch
    calls = synth.varlen_calls()
    per_flop, best_ms, first_ms = [], [], None
    for n, w in enumerate(calls):
        q_bits, k_bits, v_bits = synth.make_qkv(w)
        q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
        best = math.inf
        for rep in range(5):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            idx, cnt, totals, order = sol.route(q, k, w.tau, w.sink)
            sol.attn(q, k, v, idx, cnt, w.sink, out=o, order=order, lse_out=lse)
            e.record()
            torch.cuda.synchronize()
            ms = s.elapsed_time(e)
            if n == 0 and rep == 0:
                first_ms = ms
            best = min(best, ms)
        pairs = int(totals[1].item())
        flop = 4.0 * w.D * pairs
        per_flop.append(best / flop)
        best_ms.append(best)
        log(f"{w.name}: N={w.N} best {best:.3f} ms, {flop / best / 1e9:.1f} TFLOP/s")
        # parity with the oracle
        q32, k32, v32 = (synth.bf16_bits_to_f32(x) for x in (q_bits, k_bits, v_bits))
        r = orc.route(q32, k32, w.N, w.sink, w.tau)
        cnt_h = cnt.cpu().numpy()
        compare_masks(gpu_lists_to_mask(idx.cpu().numpy(), cnt_h, r.geom.NB), r, f"{w.name} mask")
        np.testing.assert_array_equal(cnt_h, r.cnt)
        assert int(totals[0].item()) == r.routed_pairs and pairs == r.attended_pairs
        blocks = sample_blocks(r.geom, w.B, w.H, 16, seed=w.seed)
        O, L = orc.attention(q32, k32, v32, r.sel, r.geom, blocks=blocks)
        got, lg = bf16_tensor_to_f64(o), lse.cpu().numpy().astype(np.float64)
        ref_o, got_o, ref_l, got_l = [], [], [], []
        for b, h, i in blocks:
            rr = r.geom.q_rows(i)
            ref_o.append(O[b, rr.start:rr.stop, h])
            got_o.append(got[b, rr.start:rr.stop, h])
            ref_l.append(L[b, h, rr.start:rr.stop])
            got_l.append(lg[b, h, rr.start:rr.stop])
        assert_close(np.concatenate(got_o), np.concatenate(ref_o), f"{w.name} O")
        assert float(np.abs(np.concatenate(got_l) - np.concatenate(ref_l)).max()) <= LSE_MAX_ABS
        del q, k, v, o, q32, k32, v32, q_bits, k_bits, v_bits
    med = float(np.median(per_flop))
    worst = max(per_flop) / med
    log(f"varlen: worst / median time per FLOP = {worst:.3f}; first call {first_ms:.1f} ms")
    assert worst <= 1.10
    # the very first call (code objects already loaded at import) is no outlier
    assert first_ms <= 20 * float(np.median(best_ms))


@pytest.mark.parametrize("name,N,H", [("tiny", 1024, 4), ("mid", 3001, 3)])
def test_sparse_vs_dense_gate(sol, name, N, H):
    """sol_gate_fwd: its statistics equal numpy's on the two outputs it returns,
    both outputs match the oracle, and the gate's error matches the oracle's
    sparse-vs-dense error (float64 on both sides)."""
    import torch
    w = replace(synth.WORKLOADS[name], N=N, H=H)
    q_bits, k_bits, v_bits = synth.make_qkv(w)
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    idx, cnt, _, order = sol.route(q, k, w.tau, w.sink)
    o_s, o_d, stats = sol.gate(q, k, v, idx, cnt, w.sink, order=order)
    torch.cuda.synchronize()
    a, b = bf16_tensor_to_f64(o_s), bf16_tensor_to_f64(o_d)
    st = stats.cpu().numpy()
    diff = a - b
    assert st[0] == np.abs(diff).max()
    assert st[4] == diff.size
    np.testing.assert_allclose(st[1], np.abs(diff).sum(), rtol=1e-9)
    np.testing.assert_allclose(st[2], (diff ** 2).sum(), rtol=1e-9)
    np.testing.assert_allclose(st[3], (b ** 2).sum(), rtol=1e-9)
    q32, k32, v32 = (synth.bf16_bits_to_f32(x) for x in (q_bits, k_bits, v_bits))
    r = orc.route(q32, k32, w.N, w.sink, w.tau)
    Os, _ = orc.attention(q32, k32, v32, r.sel, r.geom)
    Od, _ = orc.dense_attention(q32, k32, v32)
    assert_close(a, Os, f"gate {name} sparse")
    assert_close(b, Od, f"gate {name} dense")
    # the library's own mean and relative L2 (float64 divide and sqrt)
    assert st[5] == st[1] / st[4]
    np.testing.assert_allclose(st[6], math.sqrt(st[2] / st[3]), rtol=1e-15)
    ref_l2 = float(np.linalg.norm(Os - Od) / np.linalg.norm(Od))
    ref_mean = float(np.abs(Os - Od).mean())
    log(f"gate {name}: max_abs {st[0]:.5f} mean_abs {st[5]:.6f} l2_rel {st[6]:.6f}; "
        f"oracle l2_rel {ref_l2:.5f} mean_abs {ref_mean:.5f}")
    assert abs(st[6] - ref_l2) <= 5e-3 + 0.02 * ref_l2
    assert abs(st[5] - ref_mean) <= 2e-3 + 0.02 * ref_mean


def test_binding_rejects_mis_sized_buffers(sol):
    """The C ABI takes bare pointers; the binding checks every buffer the kernels
    index by before the call, so a too-small or mistyped one raises instead of
    being written past its end.  A workspace of any dtype counts in bytes."""
    import torch
    w = replace(synth.WORKLOADS["mid"], N=700, H=2)
    q, k, v = (to_dev(x) for x in synth.make_qkv(w))
    idx, cnt, totals, order = sol.route(q, k, w.tau, w.sink)
    NB = sol.num_blocks(w.N)
    bad = [
        dict(out=torch.empty((1, w.N - 1, w.H, w.D), dtype=torch.bfloat16, device="cuda")),
        dict(out=torch.empty_like(q, dtype=torch.float32)),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            sol.attn(q, k, v, idx, cnt, w.sink, order=order, **kw)
        with pytest.raises(ValueError):
            sol.attn_dense(q, k, v, **kw)
    with pytest.raises(ValueError):
        sol.attn(q, k, v, idx[:, :, :NB - 1], cnt, w.sink)
    with pytest.raises(ValueError):
        sol.attn(q, k, v, idx, cnt.to(torch.int64), w.sink)
    with pytest.raises(ValueError):
        sol.attn(q, k, v, idx, cnt, w.sink, order=order[:, :1])
    with pytest.raises(ValueError):
        sol.route(q, k, w.tau, w.sink, out=(idx, cnt, totals[:1], order))
    # a float32 workspace of the right byte size is accepted
    nbytes = sol.route_workspace_bytes(q)
    ws32 = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device="cuda")
    i2, c2, t2, _ = sol.route(q, k, w.tau, w.sink, workspace=ws32)
    torch.cuda.synchronize()
    assert torch.equal(c2, cnt) and torch.equal(t2, totals)
