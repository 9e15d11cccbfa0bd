"""Shared helpers for the parity tests (GPU path vs the CPU oracle)."""

from __future__ import annotations

import math
import sys

import numpy as np

import synth
from oracle import oracle as orc

# Tolerance for the bf16 output O against the float64 oracle: the raw
# max-abs error <= 1e-2 and L2-relative <= 5e-3.  How much of the error is the
# bf16 rounding an exact result pays anyway (half an ulp, 2^-9 |O|) is logged
# for information only.
MAX_ABS = 1e-2
L2_REL = 5e-3

# Tolerance for the optional LSE output (natural log; the pages state none).
# The kernel weights each key by exp(logit - m) rounded to bf16, the operand
# its P V product needs, and sums the same rounded weights, so the row sum l
# carries a relative error of at most 2^-9 (every term positive): ln(1 + 2^-9)
# = 1.95e-3 in LSE.  On top of that come the float32 logits: 128 exact bf16
# products summed in float32 miss by at most 127 * 2^-24 * sum |q_d k_d|
# (about 1.4e-4 nats after the 1/sqrt(128) scale for these inputs), and one
# rounding each in exp2 and log.  5e-4 covers those three times over.
LSE_MAX_ABS = math.log1p(2.0 ** -9) + 5e-4


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers around |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 0.5 * np.exp2(e - 7)


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def gpu_lists_to_mask(idx: np.ndarray, cnt: np.ndarray, NB: int) -> np.ndarray:
    """Mask from the GPU lists; asserts each list is strictly ascending and in range."""
    B, H, _ = cnt.shape
    sel = np.zeros((B, H, NB, NB), bool)
    for b in range(B):
        for h in range(H):
            for i in range(NB):
                c = int(cnt[b, h, i])
                lst = idx[b, h, i, :c].astype(np.int64)
                assert c >= 0 and c <= NB, (b, h, i, c)
                if c:
                    assert np.all(np.diff(lst) > 0), (b, h, i, lst)
                    assert lst[0] >= 0 and lst[-1] < NB
                sel[b, h, i, lst] = True
    return sel


def check_schedule(order, cnt):
    """Each row of the schedule is a permutation of the query blocks with
    non-increasing list length (ties may come in any order)."""
    B, H, NB = cnt.shape
    for b in range(B):
        for h in range(H):
            o = order[b, h].astype(np.int64)
            assert np.array_equal(np.sort(o), np.arange(NB)), (b, h)
            assert np.all(np.diff(cnt[b, h][o]) <= 0), (b, h)


def compare_masks(gpu_sel: np.ndarray, r: orc.Route, what: str = "mask") -> int:
    """Bit-exact mask parity: zero mismatches allowed.  Both sides compute the
    scores in the same float32 order, so even a near-tie (|s - T| within 1e-6
    relative) must select alike; the near-ties are counted and logged so that
    a test shows how close the threshold came.  Returns that count."""
    ties = orc.tie_list(r.scores, r.thresh, r.geom)
    diff = np.argwhere(gpu_sel != r.sel)
    tie_set = {tuple(x) for x in ties.tolist()}
    on_ties = sum(tuple(x) in tie_set for x in diff.tolist())
    log(f"{what}: {int(r.sel.sum())} selected pairs, {len(ties)} near-ties listed, "
        f"{len(diff)} mismatches ({on_ties} of them on a near-tie)")
    assert len(diff) == 0, f"{len(diff)} mask mismatches, first {diff[:5].tolist()}"
    return len(ties)


def errors(got: np.ndarray, ref: np.ndarray) -> dict:
    d = np.abs(got.astype(np.float64) - ref)
    return {"max_abs": float(d.max()), "mean_abs": float(d.mean()),
            "max_abs_beyond_rounding": float(np.maximum(d - bf16_half_ulp(ref), 0).max()),
            "l2_rel": float(np.linalg.norm(got.astype(np.float64) - ref)
                            / max(np.linalg.norm(ref), 1e-300))}


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = "") -> dict:
    assert np.isfinite(got).all(), f"{what}: non-finite GPU output"
    e = errors(got, ref)
    log(f"{what}: {e}")
    assert e["max_abs"] <= MAX_ABS and e["l2_rel"] <= L2_REL, f"{what}: {e}"
    return e


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def sample_blocks(g: orc.Geometry, B: int, H: int, n: int, seed: int = 0):
    """Seeded (b, h, i) sample that always holds the first, straddle and last blocks."""
    rng = np.random.default_rng(seed)
    must = {0, g.NB - 1, min(g.S // 64, g.NB - 1), min(g.S // 64 + 1, g.NB - 1)}
    out = set()
    for i in must:
        out.add((int(rng.integers(B)), int(rng.integers(H)), int(i)))
    while len(out) < n:
        out.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(g.NB))))
    return sorted(out)


def workload_inputs(w: synth.Workload):
    q, k, v = synth.make_qkv(w)
    return q, k, v, synth.bf16_bits_to_f32(q), synth.bf16_bits_to_f32(k), synth.bf16_bits_to_f32(v)


def scale_of(D: int) -> float:
    return 1.0 / math.sqrt(D)
