"""GPU parity of packed variable-length batches (several samples of different
lengths in one call, rows addressed through cumulative offsets).

Each sample is checked against the oracle's per-sample routing and attention
(lists bit for bit, O within max-abs 1e-2 beyond bf16 rounding and L2-relative
5e-3, LSE within LSE_MAX_ABS), and the packed call is checked bit for bit against the
same samples run as separate fixed-length calls on the GPU.
"""

from __future__ import annotations

import math
from dataclasses import replace

import numpy as np
import pytest

import synth
from oracle import oracle as orc
from tests.helpers import (LSE_MAX_ABS, assert_close, bf16_tensor_to_f64, check_schedule, compare_masks,
                           gpu_lists_to_mask, log, sample_blocks, to_dev)

pytestmark = pytest.mark.gpu

# lengths hit: an empty sample, a sample inside the sink (no candidates), one
# block exactly, ragged tails, and several tiles (the longest sample in the middle)
SMALL_LENGTHS = [1000, 0, 64, 777, 2053, 130, 96]
SMALL_SINK = 96


@pytest.fixture(scope="module")
def sol():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import block_sparse_attention_sol_amd as s
    return s


def _small_batch(D: int, H: int = 3):
    base = synth.WORKLOADS["mid"]
    calls = [replace(base, name=f"packed{k}", N=n, H=H, D=D, sink=SMALL_SINK, seed=k)
             for k, n in enumerate(SMALL_LENGTHS)]
    q, k, v, cu = synth.packed_batch(calls)
    return q, k, v, cu, base.tau


def _dev_offsets(cu):
    import torch
    return torch.tensor(np.asarray(cu, dtype=np.int32), device="cuda")


def _check_route(idx, cnt, totals, order, routes, cu):
    """Per-sample lists vs the oracle; entries past a sample's blocks as specified."""
    B, H, NB = cnt.shape
    routed = attended = 0
    for b in range(B):
        n = int(cu[b + 1] - cu[b])
        nb = -(-n // 64)
        np.testing.assert_array_equal(cnt[b, :, nb:], 0)
        np.testing.assert_array_equal(order[b, :, nb:], np.broadcast_to(np.arange(nb, NB), (H, NB - nb)))
        if n == 0:
            continue
        r = routes[b]
        check_schedule(order[b:b + 1, :, :nb], cnt[b:b + 1, :, :nb])
        gsel = gpu_lists_to_mask(idx[b:b + 1, :, :nb], cnt[b:b + 1, :, :nb], nb)
        compare_masks(gsel, r)
        np.testing.assert_array_equal(cnt[b:b + 1, :, :nb], r.cnt)
        routed += r.routed_pairs
        attended += r.attended_pairs
    assert int(totals[0]) == routed
    assert int(totals[1]) == attended
    return routed, attended


@pytest.mark.parametrize("D", [128, 64])
def test_packed_batch_matches_oracle_all_rows(sol, D):
    import torch
    q_bits, k_bits, v_bits, cu, tau = _small_batch(D)
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    cud, N = _dev_offsets(cu), max(SMALL_LENGTHS)
    idx, cnt, totals, order = sol.route(q, k, tau, SMALL_SINK, cu_seqlens=cud, max_seqlen=N)
    o, lse = sol.attn(q, k, v, idx, cnt, SMALL_SINK, return_lse=True, order=order,
                      cu_seqlens=cud, max_seqlen=N)
    torch.cuda.synchronize()
    q32, k32, v32 = (synth.bf16_bits_to_f32(x) for x in (q_bits, k_bits, v_bits))
    routes = orc.route_packed(q32, k32, cu, SMALL_SINK, tau)
    routed, attended = _check_route(idx.cpu().numpy(), cnt.cpu().numpy(), totals.cpu().numpy(),
                                    order.cpu().numpy(), routes, cu)
    log(f"packed D={D}: routed pairs {routed}, attended pairs {attended}")
    O, Ls = orc.attention_packed(q32, k32, v32, routes, cu)
    assert_close(bf16_tensor_to_f64(o), O, f"packed D={D} O")
    lse = lse.cpu().numpy()
    for b, L in enumerate(Ls):
        n = L.shape[1]
        if n:
            err = float(np.abs(lse[b, :, :n] - L).max())
            assert err <= LSE_MAX_ABS, (b, err)


def _packed_sweep_cases(n=6, seed=20261204):
    """Seeded random packed batches: 2 to 9 samples whose lengths mix empty,
    sub-block, exact-block and ragged multi-block samples, with a random sink,
    tau and head width."""
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        nsamp = int(rng.integers(2, 10))
        pool = [0, 1, 63, 64, 65, int(rng.integers(2, 64)), int(rng.integers(66, 1500))]
        lengths = [int(rng.choice(pool)) if rng.random() < 0.4 else int(rng.integers(1, 1800))
                   for _ in range(nsamp)]
        if max(lengths) == 0:
            lengths[0] = 200
        sink = int(rng.choice([0, 64, int(rng.integers(1, 300))]))
        tau = float(rng.choice([0.0, float(rng.uniform(0.1, 2.0))]))
        cases.append((tuple(lengths), int(rng.integers(1, 4)), int(rng.choice([64, 128])), sink,
                      tau, 3000 + c))
    return cases


@pytest.mark.parametrize("lengths,H,D,S,tau,seed", _packed_sweep_cases())
def test_packed_batch_seeded_sweep(sol, lengths, H, D, S, tau, seed):
    """Per-sample lists, counts, totals and schedule bit-exact, O on all rows
    within tolerance, LSE within LSE_MAX_ABS, on seeded random packed batches."""
    import torch
    log(f"packed sweep lengths={list(lengths)} H={H} D={D} S={S} tau={tau:.4g} seed={seed}")
    base = synth.WORKLOADS["mid"]
    calls = [replace(base, name=f"sw{i}", N=n, H=H, D=D, sink=S, tau=tau, seed=seed + 17 * i)
             for i, n in enumerate(lengths)]
    q_bits, k_bits, v_bits, cu = synth.packed_batch(calls)
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    cud, N = _dev_offsets(cu), max(lengths)
    idx, cnt, totals, order = sol.route(q, k, tau, S, cu_seqlens=cud, max_seqlen=N)
    o, lse = sol.attn(q, k, v, idx, cnt, S, return_lse=True, order=order, cu_seqlens=cud,
                      max_seqlen=N)
    torch.cuda.synchronize()
    q32, k32, v32 = (synth.bf16_bits_to_f32(x) for x in (q_bits, k_bits, v_bits))
    routes = orc.route_packed(q32, k32, cu, S, tau)
    _check_route(idx.cpu().numpy(), cnt.cpu().numpy(), totals.cpu().numpy(), order.cpu().numpy(),
                 routes, cu)
    O, Ls = orc.attention_packed(q32, k32, v32, routes, cu)
    assert_close(bf16_tensor_to_f64(o), O, "packed sweep O")
    lse = lse.cpu().numpy()
    for b, L in enumerate(Ls):
        n = L.shape[1]
        if n:
            assert float(np.abs(lse[b, :, :n] - L).max()) <= LSE_MAX_ABS, b


def test_packed_batch_equals_separate_calls_bitwise(sol):
    """Routing lists, counts, totals, O and LSE of the packed call equal the
    fixed-length calls of the samples one by one, bit for bit (the same
    kernels on the same rows), for the routed and the dense path."""
    import torch
    q_bits, k_bits, v_bits, cu, tau = _small_batch(128)
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    cud, N = _dev_offsets(cu), max(SMALL_LENGTHS)
    idx, cnt, totals, order = sol.route(q, k, tau, SMALL_SINK, cu_seqlens=cud, max_seqlen=N)
    o, lse = sol.attn(q, k, v, idx, cnt, SMALL_SINK, return_lse=True, order=order,
                      cu_seqlens=cud, max_seqlen=N)
    od, lsed = sol.attn_dense(q, k, v, return_lse=True, cu_seqlens=cud, max_seqlen=N)
    torch.cuda.synchronize()
    tot = [0, 0]
    for b in range(len(SMALL_LENGTHS)):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        n = s1 - s0
        if n == 0:
            continue
        nb = -(-n // 64)
        qs, ks, vs = (x[s0:s1].unsqueeze(0) for x in (q, k, v))
        i1, c1, t1, o1 = sol.route(qs, ks, tau, SMALL_SINK)
        a1, l1 = sol.attn(qs, ks, vs, i1, c1, SMALL_SINK, return_lse=True, order=o1)
        d1, ld1 = sol.attn_dense(qs, ks, vs, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(cnt[b, :, :nb], c1[0])
        for h in range(q.shape[1]):
            for i in range(nb):
                c = int(c1[0, h, i])
                assert torch.equal(idx[b, h, i, :c], i1[0, h, i, :c]), (b, h, i)
        tot[0] += int(t1[0])
        tot[1] += int(t1[1])
        assert torch.equal(o[s0:s1].view(torch.int16), a1[0].view(torch.int16)), b
        assert torch.equal(lse[b, :, :n], l1[0]), b
        assert torch.equal(od[s0:s1].view(torch.int16), d1[0].view(torch.int16)), b
        assert torch.equal(lsed[b, :, :n], ld1[0]), b
    assert [int(totals[0]), int(totals[1])] == tot


def test_packed_rows_outside_samples_untouched(sol):
    """Rows after the last sample (T > cu[B]) and LSE rows past each sample's
    length are never written."""
    import torch
    q_bits, k_bits, v_bits, cu, tau = _small_batch(128)
    T, H, D = q_bits.shape
    pad = 70
    q_bits, k_bits, v_bits = (np.concatenate([x, np.full((pad, H, D), 0x3F80, np.uint16)])
                              for x in (q_bits, k_bits, v_bits))
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    cud, N = _dev_offsets(cu), max(SMALL_LENGTHS)
    sentinel = torch.full_like(q, 7.0)
    idx, cnt, _, order = sol.route(q, k, tau, SMALL_SINK, cu_seqlens=cud, max_seqlen=N)
    for dense in (False, True):
        o = sentinel.clone()
        lse = torch.full((len(SMALL_LENGTHS), H, N), 3.5, dtype=torch.float32, device="cuda")
        if dense:
            sol.attn_dense(q, k, v, out=o, lse_out=lse, cu_seqlens=cud, max_seqlen=N)
        else:
            sol.attn(q, k, v, idx, cnt, SMALL_SINK, out=o, lse_out=lse, order=order,
                     cu_seqlens=cud, max_seqlen=N)
        torch.cuda.synchronize()
        assert torch.equal(o[T:], sentinel[T:]), dense
        assert torch.isfinite(o[:T].float()).all(), dense
        for b, n in enumerate(SMALL_LENGTHS):
            assert (lse[b, :, n:] == 3.5).all(), (dense, b)
            assert torch.isfinite(lse[b, :, :n]).all(), (dense, b)


def test_packed_dense_and_gate(sol):
    import torch
    q_bits, k_bits, v_bits, cu, tau = _small_batch(128, H=2)
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    cud, N = _dev_offsets(cu), max(SMALL_LENGTHS)
    idx, cnt, _, order = sol.route(q, k, tau, SMALL_SINK, cu_seqlens=cud, max_seqlen=N)
    o_s, o_d, stats = sol.gate(q, k, v, idx, cnt, SMALL_SINK, order=order, cu_seqlens=cud,
                               max_seqlen=N)
    torch.cuda.synchronize()
    q32, k32, v32 = (synth.bf16_bits_to_f32(x) for x in (q_bits, k_bits, v_bits))
    routes = orc.route_packed(q32, k32, cu, SMALL_SINK, tau)
    Os, _ = orc.attention_packed(q32, k32, v32, routes, cu)
    Od, _ = orc.attention_packed(q32, k32, v32, routes, cu, dense=True)
    a, b = bf16_tensor_to_f64(o_s), bf16_tensor_to_f64(o_d)
    assert_close(a, Os, "packed gate sparse")
    assert_close(b, Od, "packed gate dense")
    st = stats.cpu().numpy()
    diff = a - b
    assert st[0] == np.abs(diff).max()
    assert st[4] == diff.size
    np.testing.assert_allclose(st[1], np.abs(diff).sum(), rtol=1e-9)
    np.testing.assert_allclose(st[2], (diff ** 2).sum(), rtol=1e-9)
    np.testing.assert_allclose(st[3], (b ** 2).sum(), rtol=1e-9)


def test_packed_varlen_page_samples(sol):
    """Four samples of the variable-length workload (N in [36000, 40000],
    H = 14, 951-token sink) in one packed call: bit-identical to the four
    fixed-length calls, routing of every sample equal to the oracle's, sampled
    attention rows within tolerance, and no slower than the separate calls."""
    import torch
    calls = synth.varlen_calls()[:4]
    q_bits, k_bits, v_bits, cu = synth.packed_batch(calls)
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    w0 = calls[0]
    cud, N = _dev_offsets(cu), max(c.N for c in calls)
    idx, cnt, totals, order = sol.route(q, k, w0.tau, w0.sink, cu_seqlens=cud, max_seqlen=N)
    o = sol.attn(q, k, v, idx, cnt, w0.sink, order=order, cu_seqlens=cud, max_seqlen=N)
    torch.cuda.synchronize()
    q32, k32, v32 = (synth.bf16_bits_to_f32(x) for x in (q_bits, k_bits, v_bits))
    del q_bits, k_bits, v_bits
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    got = bf16_tensor_to_f64(o)
    for b, w in enumerate(calls):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        nb = w.n_blocks
        qs, ks, vs = (x[s0:s1].unsqueeze(0) for x in (q, k, v))
        i1, c1, t1, o1 = sol.route(qs, ks, w.tau, w.sink)
        a1 = sol.attn(qs, ks, vs, i1, c1, w.sink, order=o1)
        torch.cuda.synchronize()
        assert torch.equal(cnt[b, :, :nb], c1[0])
        assert torch.equal(o[s0:s1].view(torch.int16), a1[0].view(torch.int16)), b
        r = orc.route(q32[None, s0:s1], k32[None, s0:s1], w.N, w.sink, w.tau)
        gsel = gpu_lists_to_mask(idx_h[b:b + 1, :, :nb], cnt_h[b:b + 1, :, :nb], nb)
        compare_masks(gsel, r)
        blocks = sample_blocks(r.geom, 1, w.H, 24, seed=b)
        O, _ = orc.attention(q32[None, s0:s1], k32[None, s0:s1], v32[None, s0:s1], r.sel, r.geom,
                             blocks=blocks)
        ref, gv = [], []
        for _, h, i in blocks:
            rr = r.geom.q_rows(i)
            ref.append(O[0, rr.start:rr.stop, h])
            gv.append(got[s0 + rr.start:s0 + rr.stop, h])
        assert_close(np.concatenate(gv), np.concatenate(ref), f"packed {w.name}")

    def best_ms(fn, reps=3):
        best = math.inf
        for _ in range(reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            best = min(best, s.elapsed_time(e))
        return best

    def packed():
        i, c, _, od = sol.route(q, k, w0.tau, w0.sink, cu_seqlens=cud, max_seqlen=N)
        sol.attn(q, k, v, i, c, w0.sink, out=o, order=od, cu_seqlens=cud, max_seqlen=N)

    views = [tuple(x[int(cu[b]):int(cu[b + 1])].unsqueeze(0) for x in (q, k, v))
             for b in range(len(calls))]
    outs = [torch.empty_like(vw[0]) for vw in views]

    def separate():
        for (qs, ks, vs), ob in zip(views, outs):
            i, c, _, od = sol.route(qs, ks, w0.tau, w0.sink)
            sol.attn(qs, ks, vs, i, c, w0.sink, out=ob, order=od)

    t_p, t_s = best_ms(packed), best_ms(separate)
    log(f"packed 4 x varlen: {t_p:.2f} ms in one call, {t_s:.2f} ms as four calls; "
        f"{4 * 128 * int(totals[1]) / t_p / 1e9:.1f} TFLOP/s packed")
    assert t_p <= 1.10 * t_s
