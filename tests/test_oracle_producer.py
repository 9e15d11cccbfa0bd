"""Pins for the oracle's QK-norm + RoPE producer.

The float32 definition (score_ref.c) is checked against the float64
definition within a rounding bound derived from the arithmetic, on inputs
where each term matters (eps included), and its order of summation against a
hand-worked case where every other order gives other bits; the float64 definition is checked against
closed forms and the defining properties of the two operations: a constant
row normalises to its sign, the RMS of a normalised row is one, a rotation
keeps each pair's length, the quarter turn and the identity act as stated,
and the rotated dot product of a query and a key depends only on the
distance of their positions.
"""

import math

import numpy as np
import pytest

import synth
from oracle import oracle as orc

U32 = 2.0 ** -24


def _bits(x: np.ndarray) -> np.ndarray:
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def _rows(N, H, D, seed, scale=1.0):
    return _bits(np.random.default_rng(seed).standard_normal((1, N, H, D)) * scale)


def _half_ulp_bf16(x):
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 0.5 * np.exp2(np.floor(np.log2(ax)) - 7)


@pytest.mark.parametrize("D,scale,eps,rope", [
    (128, 1.0, 1e-6, True), (64, 3.0, 1e-6, True), (128, 1e-3, 1e-6, True),   # eps ~ ms
    (128, 1.0, 0.0, False), (64, 1e-3, 1e-5, False),
])
def test_mirror_within_rounding_of_the_definition(D, scale, eps, rope):
    N, H = 300, 3
    x = _rows(N, H, D, 1, scale)
    gq, _ = synth.norm_weights(D, 3)
    cos, sin = synth.rope_tables(N, D) if rope else (None, None)
    got = synth.bf16_bits_to_f32(orc.qk_norm_rope(x, gq, eps, cos, sin)).astype(np.float64)
    ref = orc.qk_norm_rope_f64(synth.bf16_bits_to_f32(x), gq, eps, cos, sin)
    # float32 error before the bf16 rounding: the sum of squares (D terms),
    # sqrt, divide and two products, and the rotation: below 64 D u of the
    # pair's length, far under the bf16 half ulp
    pair = np.sqrt(ref[..., 0::2] ** 2 + ref[..., 1::2] ** 2).repeat(2, axis=-1)
    err32 = 64 * D * U32 * pair
    tol = _half_ulp_bf16(np.maximum(np.abs(ref), np.abs(got))) + 2 * err32
    assert (np.abs(got - ref) <= tol).all(), float((np.abs(got - ref) - tol).max())
    # and the mirror is really rounding: most values sit well inside half an ulp
    assert np.mean(np.abs(got - ref) <= 0.5 * _half_ulp_bf16(ref) + err32) > 0.4


@pytest.mark.parametrize("D", [64, 128])
def test_sum_of_squares_order_exact(D):
    """The sum of squares is one running float32 sum over d ascending from +0.

    Worked by hand (u = 2^-24; g = 1 + 2^-8 + 2^-20 for every channel, eps 0,
    no rotation).  Row A puts the large values first: x = 4096 at d = 0
    (and d = 1 when D = 128), every other x = 1.  Ascending, ss reaches
    2^24 (D 64) or 2^25 (D 128), and every following 1 is absorbed (at
    2^24 an added 1 is a tie that rounds to the even 2^24), so
    ss / D = 2^18, r = 2^-9 exactly, and a channel with x = 1 gives
    y = 2^-9 g, just above the bf16 midpoint 2^-9 (1 + 2^-8): it rounds
    up to 2^-9 (1 + 2^-7); x = 4096 gives 8 g -> 8 (1 + 2^-7).  Row B puts
    the large values last.  Ascending, the ones add up first (D - 1 or
    D - 2 of them), the large squares then round the sum to 2^24 + 64 or
    2^25 + 128, so ss / D = 2^18 + 1, sqrt rounds to 512 + 2^-10,
    r = 2^-9 (1 - 2^-19), and y = r g lands 2^-29 below the midpoint: x = 1
    gives 2^-9, x = 4096 gives 8.

    Other orders give other bits: partial sums of 8-channel chunks added
    as a tree make row A's ss 2^24 + 56 (or 2^25 + 120), which rounds
    every x = 1 channel down; descending order makes row B's ss 2^24 (or
    2^25), which rounds them up.
    """
    nbig = 1 if D == 64 else 2
    x = np.ones((1, 2, 1, D), np.float32)
    x[0, 0, 0, :nbig] = 4096.0
    x[0, 1, 0, D - nbig:] = 4096.0
    g = np.full(D, 1 + 2.0 ** -8 + 2.0 ** -20, np.float32)
    out = synth.bf16_bits_to_f32(orc.qk_norm_rope(_bits(x), g, 0.0)).astype(np.float64)
    up, big_up = 2.0 ** -9 * (1 + 2.0 ** -7), 8.0 * (1 + 2.0 ** -7)
    np.testing.assert_array_equal(out[0, 0, 0, :nbig], big_up)
    np.testing.assert_array_equal(out[0, 0, 0, nbig:], up)
    np.testing.assert_array_equal(out[0, 1, 0, D - nbig:], 8.0)
    np.testing.assert_array_equal(out[0, 1, 0, : D - nbig], 2.0 ** -9)


def test_eps_and_weights_change_the_result():
    # rows small enough that eps dominates: dropping eps or gamma must show
    N, H, D = 64, 1, 128
    x = _rows(N, H, D, 2, 1e-3)
    g = np.full(D, 1.0, np.float32)
    with_eps = orc.qk_norm_rope(x, g, 1e-5, None, None)
    no_eps = orc.qk_norm_rope(x, g, 0.0, None, None)
    assert np.mean(with_eps != no_eps) > 0.9
    g2 = g.copy()
    g2[5] = 2.0
    a = synth.bf16_bits_to_f32(orc.qk_norm_rope(x, g2, 0.0, None, None))
    b = synth.bf16_bits_to_f32(no_eps)
    np.testing.assert_array_equal(a[..., 5], 2 * b[..., 5])
    np.testing.assert_array_equal(np.delete(a, 5, axis=-1), np.delete(b, 5, axis=-1))


def test_constant_row_normalises_to_its_sign():
    # x_d = a for every d: ms = a^2, so y = a / |a| exactly when eps = 0
    N, H, D = 3, 2, 128
    x = np.zeros((1, N, H, D), np.float32)
    x[0, 0] = 0.25
    x[0, 1] = -3.0
    x[0, 2] = 1.5
    out = synth.bf16_bits_to_f32(orc.qk_norm_rope(_bits(x), np.ones(D, np.float32), 0.0))
    np.testing.assert_array_equal(out[0, 0], 1.0)
    np.testing.assert_array_equal(out[0, 1], -1.0)
    np.testing.assert_array_equal(out[0, 2], 1.0)


def test_definition_rms_is_one_and_pairs_keep_length():
    N, H, D = 50, 2, 64
    x = np.random.default_rng(4).standard_normal((1, N, H, D)) * 2
    y = orc.qk_norm_rope_f64(x, np.ones(D), 0.0)
    np.testing.assert_allclose((y * y).mean(axis=-1), 1.0, rtol=1e-12)
    cos, sin = synth.rope_tables(N, D)
    o = orc.qk_norm_rope_f64(x, np.ones(D), 0.0, cos.astype(np.float64), sin.astype(np.float64))
    # the float32 tables hold cos^2 + sin^2 = 1 to within a few float32 ulps
    np.testing.assert_allclose(o[..., 0::2] ** 2 + o[..., 1::2] ** 2,
                               y[..., 0::2] ** 2 + y[..., 1::2] ** 2, rtol=8 * U32)


def test_quarter_turn_and_identity():
    N, H, D = 4, 1, 64
    x = _rows(N, H, D, 5)
    g = np.ones(D, np.float32)
    plain = orc.qk_norm_rope(x, g, 1e-6)
    one, zero = np.ones((N, D // 2), np.float32), np.zeros((N, D // 2), np.float32)
    np.testing.assert_array_equal(orc.qk_norm_rope(x, g, 1e-6, one, zero), plain)
    # cos 0, sin 1: (a, b) -> (-b, a); bf16 negation is exact
    turned = synth.bf16_bits_to_f32(orc.qk_norm_rope(x, g, 1e-6, zero, one))
    p = synth.bf16_bits_to_f32(plain)
    np.testing.assert_array_equal(turned[..., 0::2], -p[..., 1::2])
    np.testing.assert_array_equal(turned[..., 1::2], p[..., 0::2])


def test_rotated_dot_product_depends_on_distance_only():
    D = 64
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, 1, D))
    k = rng.standard_normal((1, 1, 1, D))
    cos, sin = synth.rope_tables(200, D)
    cos, sin = cos.astype(np.float64), sin.astype(np.float64)

    def dot(m, n):
        qm = orc.qk_norm_rope_f64(q, np.ones(D), 0.0, cos[m:m + 1], sin[m:m + 1])
        kn = orc.qk_norm_rope_f64(k, np.ones(D), 0.0, cos[n:n + 1], sin[n:n + 1])
        return float((qm * kn).sum())
    for m, n, shift in [(3, 10, 50), (100, 7, 60), (0, 0, 123)]:
        # float32 tables: angles agree to about 1e-7 relative
        assert abs(dot(m, n) - dot(m + shift, n + shift)) < 1e-4 * D
    assert abs(dot(3, 10) - dot(3, 11)) > 1e-3          # the distance does matter


def test_packed_positions_restart_per_sample():
    H, D = 2, 64
    lengths = [70, 0, 33]
    x = _bits(np.random.default_rng(7).standard_normal((sum(lengths), H, D)))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    g = np.ones(D, np.float32)
    cos, sin = synth.rope_tables(max(lengths), D)
    out = orc.qk_norm_rope_packed(x, cu, g, 1e-6, cos, sin)
    for b in range(len(lengths)):
        s0, s1 = cu[b], cu[b + 1]
        if s1 > s0:
            np.testing.assert_array_equal(out[s0:s1], orc.qk_norm_rope(x[None, s0:s1], g, 1e-6,
                                                                       cos, sin)[0])
