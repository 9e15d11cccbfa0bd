"""Pins for the oracle's routing (pooling, scores, selection, densities).

Each test checks the oracle against something other than its own formula: a
float64 recomputation with a rounding-error bound, values fixed by hand, an
orthogonal construction whose selected set is known in advance, a brute-force
token-level count, or an invariant of the selection rule.
"""

import math

import numpy as np
import pytest

from oracle import oracle as orc

U32 = 2.0 ** -24  # float32 unit roundoff


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


# --------------------------------------------------------------------------- geometry
@pytest.mark.parametrize("N,S,NB,j0", [
    (1024, 64, 16, 1), (38247, 951, 598, 14), (8192, 256, 128, 4), (1, 0, 1, 0),
    (100, 0, 2, 0), (100, 100, 2, 2), (100, 500, 2, 2), (130, 64, 3, 1), (130, 63, 3, 0),
])
def test_geometry(N, S, NB, j0):
    g = orc.geometry(N, S)
    assert (g.NB, g.j0) == (NB, j0)
    # every candidate has at least one routable key; the block before j0 has none
    for j in range(g.j0, g.NB):
        assert len(g.r_keys(j)) > 0
    if g.j0 > 0 and g.j0 < g.NB:
        assert len(g.r_keys(g.j0 - 1)) == 0
    # sink + routable keys of all blocks partition [0, N)
    keys = list(range(g.Ssink)) + [t for j in range(g.NB) for t in g.r_keys(j)]
    assert sorted(keys) == list(range(N))


def test_page_straddle_block():
    # 951 = 14 * 64 + 55: block 14 holds sink keys 896..950 and routable keys 951..959
    g = orc.geometry(38247, 951)
    assert g.r_keys(14) == range(951, 960)
    assert g.q_rows(597) == range(38208, 38247)      # 39 valid rows in the last block


# --------------------------------------------------------------------------- pooling
def test_pool_queries_exact_values():
    # integers are exact in float32: the mean is exact, including the ragged tail
    N, D = 64 + 39, 8
    x = np.zeros((1, N, 1, D), np.float32)
    x[0, :, 0, :] = np.arange(N, dtype=np.float32)[:, None]
    qb = orc.pool_queries(x, orc.geometry(N, 0))
    assert qb.shape == (1, 1, 2, D)
    np.testing.assert_array_equal(qb[0, 0, 0], np.full(D, 31.5, np.float32))
    np.testing.assert_array_equal(qb[0, 0, 1], np.full(D, np.float32(sum(range(64, N)) / 39)))


def test_pool_keys_use_routable_rows_only():
    # sink rows and rows past N must not reach the key means
    N, S, D = 200, 70, 4
    k = np.full((1, N, 1, D), 1e6, np.float32)
    for t in range(S, N):
        k[0, t, 0, :] = t
    g = orc.geometry(N, S)
    kb = orc.pool_keys(k, g)
    assert g.j0 == 1
    assert np.isnan(kb[0, 0, 0]).all()
    np.testing.assert_array_equal(kb[0, 0, 1], np.full(D, np.float32(np.mean(np.arange(70, 128)))))
    np.testing.assert_array_equal(kb[0, 0, 3], np.full(D, np.float32(np.mean(np.arange(192, 200)))))


@pytest.mark.parametrize("N,S", [(1000, 0), (1000, 100), (777, 700), (64, 0), (65, 1)])
def test_pool_within_float64_error_bound(N, S):
    B, H, D = 2, 3, 16
    x = _rand((B, N, H, D), seed=N + S, scale=3.0)
    g = orc.geometry(N, S)
    qb = orc.pool_queries(x, g).astype(np.float64)
    kb = orc.pool_keys(x, g).astype(np.float64)
    x64 = x.astype(np.float64)
    for i in range(g.NB):
        rows = list(g.q_rows(i))
        m = x64[:, rows].mean(axis=1).transpose(0, 1, 2)            # [B, H, D]
        bound = len(rows) * U32 * np.abs(x64[:, rows]).sum(axis=1) / len(rows) + 2 * U32 * np.abs(m)
        assert np.all(np.abs(qb[:, :, i] - m) <= bound + 1e-30)
    for j in range(g.j0, g.NB):
        rows = list(g.r_keys(j))
        m = x64[:, rows].mean(axis=1)
        bound = len(rows) * U32 * np.abs(x64[:, rows]).sum(axis=1) / len(rows) + 2 * U32 * np.abs(m)
        assert np.all(np.abs(kb[:, :, j] - m) <= bound + 1e-30)


# --------------------------------------------------------------------------- scores
def test_scores_fma_chain_order_exact():
    """One fused rounding per step, d ascending: the residual of a*a survives.

    q = [1, a], k = [-r, a] with a = 1 + 2^-12 and r = fl32(a^2) = 1 + 2^-11.
    Ascending FMA chain: acc = -r, then fma(a, a, -r) = a^2 - r = 2^-24 exactly.
    A separate multiply and add would give 0; the reversed order gives 0 too.
    """
    a = np.float32(1 + 2.0 ** -12)
    r = np.float32(a * a)
    assert float(r) == 1 + 2.0 ** -11
    q = np.array([[[[1.0, a]]]], np.float32)            # [B=1, H=1, NB=1, D=2]
    k = np.array([[[[-r, a]]]], np.float32)
    g = orc.Geometry(N=64, S=0, NB=1, Ssink=0, j0=0)
    scale = np.float32(0.75)
    s = orc.block_scores(q, k, g, scale)
    assert s[0, 0, 0, 0] == np.float32(2.0 ** -24) * scale


@pytest.mark.parametrize("D", [64, 128])
def test_scores_within_float64_error_bound_and_not_transposed(D):
    B, H, NB = 1, 2, 12
    g = orc.geometry(NB * 64, 130)                      # j0 = 2
    qb = _rand((B, H, NB, D), 1)
    kb = _rand((B, H, NB, D), 2)
    kb[:, :, : g.j0] = np.nan
    scale = orc.default_scale32(D)
    s = orc.block_scores(qb, kb, g, scale).astype(np.float64)
    assert np.isnan(s[..., : g.j0]).all()
    q64, k64 = qb.astype(np.float64), kb[:, :, g.j0:].astype(np.float64)
    ref = np.einsum("bhid,bhjd->bhij", q64, k64) * float(scale)
    absd = np.einsum("bhid,bhjd->bhij", np.abs(q64), np.abs(k64)) * float(scale)
    bound = (D + 1) * U32 * absd + U32 * np.abs(ref)
    got = s[..., g.j0:]
    assert np.all(np.abs(got - ref) <= bound)
    # a swapped (j, i) reading would miss by far more than the bound
    assert np.abs(got[:, :, :10, :10] - ref[:, :, :10, :10].transpose(0, 1, 3, 2)).max() > 1e-2


def test_scale_constant():
    assert orc.default_scale32(128) == np.float32(0.08838834764831845)
    assert orc.default_scale32(64) == np.float32(0.125)


# --------------------------------------------------------------------------- selection
def _orthogonal_case(seed, NB=20, j0=2, D=64, c=4.0):
    """K block j is c * e_pi(j) on every row; Q block i is the sum of e_pi(j) over A_i.

    Then qbar_i . kbar_j = c when j in A_i and 0 otherwise (exact in float32).
    """
    rng = np.random.default_rng(seed)
    N = NB * 64
    S = j0 * 64
    perm = rng.permutation(D)[:NB]
    A = [set(rng.choice(np.arange(j0, NB), size=rng.integers(1, 5), replace=False).tolist())
         for _ in range(NB)]
    k = np.zeros((1, N, 1, D), np.float32)
    q = np.zeros((1, N, 1, D), np.float32)
    for j in range(NB):
        k[0, 64 * j: 64 * j + 64, 0, perm[j]] = c
    for i in range(NB):
        for j in A[i]:
            q[0, 64 * i: 64 * i + 64, 0, perm[j]] = 1.0
    return q, k, N, S, A, c


@pytest.mark.parametrize("seed", range(5))
def test_selection_orthogonal_construction(seed):
    q, k, N, S, A, c = _orthogonal_case(seed)
    D = q.shape[-1]
    r = orc.route(q, k, N, S, tau=0.5 * c / math.sqrt(D))
    g = r.geom
    for i in range(g.NB):
        expect = set(A[i]) | ({i} if i >= g.j0 else set())
        assert set(np.nonzero(r.sel[0, 0, i])[0].tolist()) == expect, i
    assert r.routed_pairs == sum(len(set(A[i]) | ({i} if i >= g.j0 else set())) for i in range(g.NB))


def test_selection_empty_query_block_keeps_everything():
    # a zero query block scores 0 against every key block: all tie with the max
    q, k, N, S, A, c = _orthogonal_case(0)
    q[0, 64 * 5: 64 * 6] = 0.0
    r = orc.route(q, k, N, S, tau=0.01)
    assert r.sel[0, 0, 5, r.geom.j0:].all()


@pytest.fixture(scope="module")
def random_route_inputs():
    B, N, H, D = 1, 1500, 3, 64
    q = _rand((B, N, H, D), 11, 2.0)
    k = _rand((B, N, H, D), 12, 2.0)
    # shared block component so that scores spread
    blk = _rand((B, -(-N // 64), H, D), 13, 2.0)
    k += blk[:, np.arange(N) // 64]
    q += blk[:, np.arange(N) // 64] * 0.5
    return q, k, N, 200


def test_selection_invariants(random_route_inputs):
    q, k, N, S = random_route_inputs
    taus = [0.0, 0.3, 1.0, 3.0, 10.0, math.inf]
    routes = [orc.route(q, k, N, S, tau) for tau in taus]
    g = routes[0].geom
    for r in routes:
        # the forced diagonal, and nothing before j0
        d = np.arange(g.j0, g.NB)
        assert r.sel[:, :, d, d].all()
        assert not r.sel[..., : g.j0].any()
        assert (r.cnt >= 1)[:, :, g.j0:].all()
    # monotone in tau
    for a, b in zip(routes, routes[1:]):
        assert not (a.sel & ~b.sel).any()
    # tau = inf selects every candidate
    assert routes[-1].sel[..., g.j0:].all()
    # tau = 0 keeps exactly the argmax ties and the diagonal
    s = routes[0].scores[..., g.j0:]
    top = s == s.max(axis=-1, keepdims=True)
    expect = np.zeros_like(routes[0].sel)
    expect[..., g.j0:] = top
    expect[:, :, np.arange(g.j0, g.NB), np.arange(g.j0, g.NB)] = True
    np.testing.assert_array_equal(routes[0].sel, expect)
    # the dense flag equals tau = inf
    rd = orc.route(q, k, N, S, 1.0, dense=True)
    np.testing.assert_array_equal(rd.sel, routes[-1].sel)


def test_block_lists_ascending(random_route_inputs):
    q, k, N, S = random_route_inputs
    r = orc.route(q, k, N, S, 1.0)
    idx, cnt = orc.block_lists(r.sel)
    np.testing.assert_array_equal(cnt, r.cnt)
    for b, h, i in np.ndindex(*cnt.shape):
        lst = idx[b, h, i, : cnt[b, h, i]]
        assert np.all(np.diff(lst) > 0)
        assert (idx[b, h, i, cnt[b, h, i]:] == -1).all()


def test_tie_list_flags_exact_ties():
    q, k, N, S, A, c = _orthogonal_case(3)
    D = q.shape[-1]
    tau = 0.5 * c / math.sqrt(D)
    r = orc.route(q, k, N, S, tau)
    ties = orc.tie_list(r.scores, r.thresh, r.geom)
    assert len(ties) == 0
    # tau equal to the gap puts the zero scores exactly on the threshold
    tau = float(np.float32(c) * orc.default_scale32(D))
    r = orc.route(q, k, N, S, tau)
    ties = orc.tie_list(r.scores, r.thresh, r.geom)
    assert len(ties) > 0


# --------------------------------------------------------------------------- densities
@pytest.mark.parametrize("N,S,tau", [(1500, 200, 1.0), (1500, 0, 0.3), (700, 690, 1.0),
                                     (300, 1000, 1.0), (129, 64, 0.0)])
def test_attended_pairs_and_densities_brute_force(random_route_inputs, N, S, tau):
    q, k, _, _ = random_route_inputs
    q, k = q[:, :N].copy(), k[:, :N].copy()
    B, _, H, _ = q.shape
    r = orc.route(q, k, N, S, tau)
    g = r.geom
    pairs = 0
    blocks = 0
    for b in range(B):
        for h in range(H):
            mask = np.zeros((N, N), bool)         # token level: query row x key
            mask[:, : min(S, N)] = True
            for i in range(g.NB):
                for j in np.nonzero(r.sel[b, h, i])[0]:
                    lo, hi = max(64 * j, S), min(64 * j + 64, N)
                    mask[64 * i: 64 * i + 64, lo:hi] = True
            pairs += int(mask.sum())
            for i in range(g.NB):
                for j in range(g.NB):
                    blocks += bool(mask[64 * i: 64 * i + 64, 64 * j: 64 * j + 64].any())
    assert r.attended_pairs == pairs
    dens = orc.densities(r, B, H)
    assert dens["pair"] == (pairs, B * H * N * N)
    assert dens["block"] == (blocks, B * H * g.NB * g.NB)
    assert dens["route"] == (int(r.sel.sum()), B * H * g.NB * g.ncand)
