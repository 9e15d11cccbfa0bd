"""Calibrate the routing threshold tau of each synthetic workload on the oracle.

Test infrastructure: prints, for each workload, the tau (4 significant digits)
whose routed density is nearest the target, and the exact density it gives.
The frozen values live in synth.WORKLOADS.  Calls only oracle/ and synth/.

    python -m oracle.calibrate_tau [tiny mid page page_fused varlen]
"""

from __future__ import annotations

import math
import sys

import numpy as np

import synth
from oracle import oracle as orc

TARGET = {"tiny": 0.25, "mid": 0.20, "page": 0.19, "page_fused": 0.19}


def scores_for(w: synth.Workload):
    q, k, _ = synth.make_qkv(w)
    if w.producer:
        gq, gk = synth.norm_weights(w.D)
        cos, sin = synth.rope_tables(w.N, w.D)
        q = orc.qk_norm_rope(q, gq, synth.NORM_EPS, cos, sin)
        k = orc.qk_norm_rope(k, gk, synth.NORM_EPS, cos, sin)
    q32, k32 = synth.bf16_bits_to_f32(q), synth.bf16_bits_to_f32(k)
    g = orc.geometry(w.N, w.sink)
    s = orc.block_scores(orc.pool_queries(q32, g), orc.pool_keys(k32, g), g,
                         orc.default_scale32(w.D))
    return g, s


def density(s, g, tau: float) -> tuple[int, int]:
    sel, _ = orc.select_blocks(s, g, tau)
    B, H = s.shape[:2]
    return int(sel.sum()), B * H * g.NB * g.ncand


def calibrate(name: str) -> None:
    w = synth.WORKLOADS[name]
    g, s = scores_for(w)
    target = TARGET[name]
    lo, hi = 0.0, 64.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        n, d = density(s, g, mid)
        lo, hi = (mid, hi) if n / d < target else (lo, mid)
    tau = float(f"{0.5 * (lo + hi):.4g}")
    n, d = density(s, g, tau)
    print(f"{name}: tau={tau}  routed density {n}/{d} = {n / d:.4%} (target {target:.0%})")


def check_varlen() -> None:
    for w in synth.varlen_calls():
        g, s = scores_for(w)
        n, d = density(s, g, w.tau)
        print(f"{w.name}: N={w.N} tau={w.tau} routed density {n}/{d} = {n / d:.4%}")


if __name__ == "__main__":
    names = sys.argv[1:] or ["tiny", "mid", "page", "varlen"]
    for nm in names:
        if nm == "varlen":
            check_varlen()
        else:
            calibrate(nm)
