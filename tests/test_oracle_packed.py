"""Pins for the oracle's packed variable-length batches.

A packed batch is a set of independent samples stored back to back; each has
its own blocks, sink, routing and attention.  The oracle's packed functions
are checked against things they do not share code with: the batched
[B, N, H, D] oracle at equal lengths, one masked softmax over the whole packed
sequence in which a query sees only its own sample's keys, the reversal of
the sample order, and the closed forms of an empty sample and a sample no
longer than the sink.
"""

import math

import numpy as np

from oracle import oracle as orc


def _packed(lengths, H, D, seed):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    x = [rng.standard_normal((T, H, D)).astype(np.float32) * s for s in (1.5, 1.5, 1.0)]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return x[0], x[1], x[2], cu


def test_equal_lengths_match_the_batched_oracle():
    B, N, H, D, S, tau = 3, 200, 2, 64, 70, 0.05
    q, k, v, cu = _packed([N] * B, H, D, 1)
    routes = orc.route_packed(q, k, cu, S, tau)
    qb, kb, vb = (x.reshape(B, N, H, D) for x in (q, k, v))
    rb = orc.route(qb, kb, N, S, tau)
    for b in range(B):
        np.testing.assert_array_equal(routes[b].sel[0], rb.sel[b])
        np.testing.assert_array_equal(routes[b].cnt[0], rb.cnt[b])
    assert sum(r.attended_pairs for r in routes) == rb.attended_pairs
    O, Ls = orc.attention_packed(q, k, v, routes, cu)
    Ob, Lb = orc.attention(qb, kb, vb, rb.sel, rb.geom)
    np.testing.assert_array_equal(O, Ob.reshape(B * N, H, D))
    for b in range(B):
        np.testing.assert_array_equal(Ls[b], Lb[b])


def test_matches_one_masked_softmax_over_the_packed_sequence():
    lengths, H, D, S, tau = [70, 0, 130, 33, 64], 2, 16, 40, 0.2
    q, k, v, cu = _packed(lengths, H, D, 2)
    routes = orc.route_packed(q, k, cu, S, tau)
    O, Ls = orc.attention_packed(q, k, v, routes, cu)
    T = int(cu[-1])
    scale = 1.0 / math.sqrt(D)
    for h in range(H):
        # token-level key set of every packed row: its own sample's sink keys
        # and the routable keys of the blocks routed to its block
        allow = np.zeros((T, T), bool)
        for b, r in enumerate(routes):
            if r is None:
                continue
            s0, g = int(cu[b]), r.geom
            for t in range(g.N):
                allow[s0 + t, s0:s0 + g.Ssink] = True
                for j in np.nonzero(r.sel[0, h, t // 64])[0]:
                    kr = g.r_keys(j)
                    allow[s0 + t, s0 + kr.start:s0 + kr.stop] = True
        z = (q[:, h].astype(np.float64) @ k[:, h].astype(np.float64).T) * scale
        z = np.where(allow, z, -np.inf)
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        ref = (e @ v[:, h].astype(np.float64)) / e.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(O[:, h], ref, rtol=1e-12, atol=1e-12)
        lse = (m[:, 0] + np.log(e.sum(axis=1)))
        for b in range(len(lengths)):
            np.testing.assert_allclose(Ls[b][h], lse[cu[b]:cu[b + 1]], rtol=1e-12, atol=1e-12)


def test_reversing_the_samples_reverses_the_results():
    lengths, H, D, S, tau = [150, 90, 257], 2, 32, 64, 0.1
    q, k, v, cu = _packed(lengths, H, D, 3)
    routes = orc.route_packed(q, k, cu, S, tau)
    O, _ = orc.attention_packed(q, k, v, routes, cu)
    rev = lengths[::-1]
    cu_r = np.concatenate([[0], np.cumsum(rev)])
    perm = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in range(len(lengths))[::-1]])
    qr, kr, vr = q[perm], k[perm], v[perm]
    routes_r = orc.route_packed(qr, kr, cu_r, S, tau)
    O_r, _ = orc.attention_packed(qr, kr, vr, routes_r, cu_r)
    np.testing.assert_array_equal(O_r, O[perm])
    for b in range(len(lengths)):
        np.testing.assert_array_equal(routes_r[len(lengths) - 1 - b].sel, routes[b].sel)


def test_empty_sample_and_sample_inside_the_sink():
    lengths, H, D, S = [0, 50, 200], 2, 32, 64
    q, k, v, cu = _packed(lengths, H, D, 4)
    routes = orc.route_packed(q, k, cu, S, 0.1)
    assert routes[0] is None
    # 50 rows <= S: every key is a sink key, no candidates, every list empty
    r1 = routes[1]
    assert r1.geom.ncand == 0 and int(r1.cnt.sum()) == 0
    assert r1.attended_pairs == H * 50 * 50
    O, Ls = orc.attention_packed(q, k, v, routes, cu)
    assert Ls[0].shape == (H, 0)
    Od, _ = orc.dense_attention(q[None, 0:50], k[None, 0:50], v[None, 0:50])
    np.testing.assert_allclose(O[0:50], Od[0], rtol=0, atol=1e-13)
    # rows outside the samples do not exist in a packed batch without a gap
    assert not np.isnan(O).any()
