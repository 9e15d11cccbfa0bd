"""Pins for the oracle's attention (sink + routed keys merged by log-sum-exp).

The oracle computes the sink part and the routed part separately and merges
them by log-sum-exp.  These tests check it against a single masked softmax
over the token-level key set (torch's CPU scaled_dot_product_attention in
float64, a library routine), against textbook dense attention at density 1,
and against closed forms (constant V, zero Q, block-diagonal attention).
"""

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import oracle as orc


def _inputs(B, N, H, D, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, N, H, D)).astype(np.float32) * 1.5
    k = rng.standard_normal((B, N, H, D)).astype(np.float32) * 1.5
    v = rng.standard_normal((B, N, H, D)).astype(np.float32)
    return q, k, v


def _token_mask(sel_bh, g):
    """[N, N] boolean: query row attends key column (sink + routed keys)."""
    N = g.N
    m = np.zeros((N, N), bool)
    m[:, : g.Ssink] = True
    for i in range(g.NB):
        for j in np.nonzero(sel_bh[i])[0]:
            r = g.r_keys(j)
            m[64 * i: 64 * i + 64, r.start:r.stop] = True
    return m


def _sdpa_masked(q, k, v, masks):
    """Library reference: one masked softmax per (b, h), float64, torch CPU."""
    B, N, H, D = q.shape
    out = np.zeros((B, N, H, D))
    for b in range(B):
        for h in range(H):
            qt = torch.from_numpy(q[b, :, h].astype(np.float64))[None, None]
            kt = torch.from_numpy(k[b, :, h].astype(np.float64))[None, None]
            vt = torch.from_numpy(v[b, :, h].astype(np.float64))[None, None]
            mt = torch.from_numpy(masks[b][h])[None, None]
            o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt)
            out[b, :, h] = o[0, 0].numpy()
    return out


CASES = [
    # B, N, H, D, S, tau
    (1, 1024, 2, 64, 64, 0.5),
    (1, 700, 3, 128, 951, 1.0),        # sink longer than the sequence: dense
    (2, 333, 1, 64, 0, 0.2),           # no sink
    (1, 500, 2, 128, 63, 0.8),         # sink shorter than one block
    (1, 500, 2, 64, 65, 0.8),          # sink straddles block 1
    (1, 129, 1, 64, 128, 0.0),         # one routable key in the last block
    (1, 1, 1, 64, 0, 1.0),             # a single token
    (1, 37, 2, 128, 5, 1.0),           # one ragged block
]


@pytest.mark.parametrize("B,N,H,D,S,tau", CASES)
def test_lse_merge_equals_single_masked_softmax(B, N, H, D, S, tau):
    q, k, v = _inputs(B, N, H, D, seed=N * 7 + S)
    r = orc.route(q, k, N, S, tau)
    g = r.geom
    O, L = orc.attention(q, k, v, r.sel, g)
    masks = [[_token_mask(r.sel[b, h], g) for h in range(H)] for b in range(B)]
    ref = _sdpa_masked(q, k, v, masks)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    # natural-log LSE of the scaled logits over the attended keys
    scale = 1.0 / math.sqrt(D)
    for b in range(B):
        for h in range(H):
            z = (q[b, :, h].astype(np.float64) @ k[b, :, h].astype(np.float64).T) * scale
            z[~masks[b][h]] = -np.inf
            np.testing.assert_allclose(L[b, h], logsumexp(z, axis=1), rtol=0, atol=1e-12)


def _sweep_cases(n=30, seed=2024):
    """Seeded sweep: N in 1..300 (no multiple of 64), S in {0, 1, 63, 64, 65, N},
    D in {64, 128}, H in {1, 3}, tau in {0, 0.3, 1, inf}."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        N = int(rng.integers(1, 301))
        if N % 64 == 0:
            continue
        S = int(rng.choice([0, 1, 63, 64, 65, N]))
        out.append((1, N, int(rng.choice([1, 3])), int(rng.choice([64, 128])), S,
                    float(rng.choice([0.0, 0.3, 1.0, math.inf]))))
    return out


@pytest.mark.parametrize("B,N,H,D,S,tau", _sweep_cases())
def test_lse_merge_seeded_sweep(B, N, H, D, S, tau):
    """The same check as above over a seeded sweep of small shapes."""
    test_lse_merge_equals_single_masked_softmax(B, N, H, D, S, tau)


@pytest.mark.parametrize("N,S", [(1000, 64), (333, 0), (77, 200)])
def test_density_one_is_dense_attention(N, S):
    B, H, D = 1, 2, 64
    q, k, v = _inputs(B, N, H, D, seed=5)
    r = orc.route(q, k, N, S, math.inf)
    O, L = orc.attention(q, k, v, r.sel, r.geom)
    full = [[np.ones((N, N), bool) for _ in range(H)] for _ in range(B)]
    ref = _sdpa_masked(q, k, v, full)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    Od, Ld = orc.dense_attention(q, k, v)
    np.testing.assert_allclose(Od, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Ld, L, rtol=0, atol=1e-12)


def test_no_sink_diagonal_only_is_block_diagonal_attention():
    B, N, H, D = 1, 300, 1, 64
    q, k, v = _inputs(B, N, H, D, seed=9)
    g = orc.geometry(N, 0)
    sel = np.zeros((B, H, g.NB, g.NB), bool)
    sel[:, :, np.arange(g.NB), np.arange(g.NB)] = True
    O, _ = orc.attention(q, k, v, sel, g)
    for i in range(g.NB):
        rows = slice(64 * i, min(64 * i + 64, N))
        qt = torch.from_numpy(q[0, rows, 0].astype(np.float64))[None, None]
        kt = torch.from_numpy(k[0, rows, 0].astype(np.float64))[None, None]
        vt = torch.from_numpy(v[0, rows, 0].astype(np.float64))[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0].numpy()
        np.testing.assert_allclose(O[0, rows, 0], ref, rtol=0, atol=1e-12)


def test_constant_values_give_constant_output():
    B, N, H, D = 1, 600, 2, 128
    q, k, _ = _inputs(B, N, H, D, seed=3)
    v = np.full((B, N, H, D), 0.375, np.float32)
    r = orc.route(q, k, N, 100, 0.7)
    O, _ = orc.attention(q, k, v, r.sel, r.geom)
    np.testing.assert_allclose(O, 0.375, rtol=0, atol=1e-14)


def test_zero_query_gives_mean_of_attended_values():
    B, N, H, D = 1, 520, 2, 64
    q, k, v = _inputs(B, N, H, D, seed=4)
    r = orc.route(q, k, N, 130, 0.5)             # route on the real queries
    qz = np.zeros_like(q)
    O, L = orc.attention(qz, k, v, r.sel, r.geom)
    for h in range(H):
        m = _token_mask(r.sel[0, h], r.geom)
        ref = (m.astype(np.float64) @ v[0, :, h].astype(np.float64)) / m.sum(1, keepdims=True)
        np.testing.assert_allclose(O[0, :, h], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[0, h], np.log(m.sum(1)), rtol=0, atol=1e-12)


def test_swapping_two_routed_blocks_leaves_output_unchanged():
    B, N, H, D = 1, 640, 1, 64
    q, k, v = _inputs(B, N, H, D, seed=6)
    g = orc.geometry(N, 64)
    sel = np.zeros((B, H, g.NB, g.NB), bool)
    sel[0, 0, :, [3, 7]] = True
    O, _ = orc.attention(q, k, v, sel, g)
    k2, v2 = k.copy(), v.copy()
    a, b = slice(192, 256), slice(448, 512)
    k2[0, a], k2[0, b] = k[0, b], k[0, a]
    v2[0, a], v2[0, b] = v[0, b], v[0, a]
    O2, _ = orc.attention(q, k2, v2, sel, g)
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-13)


def test_sampled_blocks_match_full_run():
    B, N, H, D = 1, 900, 2, 64
    q, k, v = _inputs(B, N, H, D, seed=8)
    r = orc.route(q, k, N, 70, 0.6)
    O, L = orc.attention(q, k, v, r.sel, r.geom)
    Os, Ls = orc.attention(q, k, v, r.sel, r.geom, blocks=[(0, 1, 3), (0, 0, 14)])
    np.testing.assert_array_equal(Os[0, 192:256, 1], O[0, 192:256, 1])
    np.testing.assert_array_equal(Os[0, 896:900, 0], O[0, 896:900, 0])
    assert np.isnan(Os[0, :192]).all()
