"""Seeded synthetic Q/K/V for the block-sparse attention workloads.

This module only draws random tensors and rounds them to bf16.  It holds no
step of the attention method (no pooling, scoring, selection or softmax), so it
can feed both the CPU oracle and the GPU path without tying them together.

Tensors are [B, N, H, D] bf16, returned as their raw uint16 bit patterns
(round-to-nearest-even from float32).  Every draw comes from a numpy
``default_rng`` stream keyed by (seed, tensor, batch, head), so any head can be
regenerated alone and the result does not depend on thread scheduling.

Workload shapes follow the MiniMax-H3 Sol-Attn pages: one packed sequence of
38,247 tokens per attention layer with 56 heads of width 128 and a
951-token multimodal prefix (the clawpit.io article on the single-4090 run,
paragraph on the Sol-Attn settings; the nvlabs Sol-Engine H3 page, policy
paragraph), 124 video frames after the prefix (nvlabs page, opening
paragraph), and 64-token blocks (tokenfactory.fast post, "The benchmark was
not the product").  No real activations are available, so structure stands in
for them:

* ``tiny``   iid N(0,1) plus a per-(64-token block, head) shared N(0,1) vector
             scaled by 0.8, drawn independently for Q, K and V.
* ``field``  a smooth random field along tokens, per head: a per-64-token-block
             vector that is itself AR(1) across blocks (rho 0.95, amplitude
             0.5: nearby blocks look alike, a band in the mask), plus a
             token-level AR(1) process (rho 0.9, unit stationary variance);
             after the prefix the tokens are cut into frame-like groups and
             position p inside a group adds beta * E[p] from a spatial basis E
             that is smooth in p (AR(1), rho 0.98) and shared by all frames (a
             query attends to the same place in other frames: stripes).  K is
             alpha * (field + N(0, 0.5)); Q is alpha * (0.2 field + sqrt(0.96)
             field' + N(0, 0.5)) with field' an independent draw, so Q and K
             are related but the diagonal block is not always the best one.  V
             is another independent draw, scaled to unit variance.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np
from scipy.signal import lfilter

BLOCK = 64

_TENSOR_TAG = {"q": 1, "k": 2, "v": 3}


# --------------------------------------------------------------------------- bf16
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    out = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    out[np.isnan(x)] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- workloads
@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    H: int
    D: int
    sink: int          # exact prefix length S
    tau: float         # routing threshold (inf = route everything)
    kind: str          # "tiny" or "field"
    frames: int = 0    # frame-like groups after the prefix (field only)
    alpha: float = 1.0  # Q/K amplitude (field only)
    beta: float = 0.0  # spatial-basis amplitude (field only)
    seed: int = 0
    dense: bool = False  # routing disabled (full attention)
    producer: bool = False  # Q, K pass through QK-norm + RoPE before routing (norm_weights, rope_tables)

    @property
    def n_blocks(self) -> int:
        return -(-self.N // BLOCK)

    @property
    def n_padded(self) -> int:
        return BLOCK * self.n_blocks


# tau values were calibrated on the oracle's routing so that the routed
# density lands near the stated target; ``oracle/calibrate_tau.py`` recomputes
# them and prints the exact densities they give.
# eps of the synthetic QK-norm (a model hyperparameter; 1e-6 is common)
NORM_EPS = 1e-6

WORKLOADS = {
    # ~25% routed density
    "tiny": Workload("tiny", B=1, N=1024, H=4, D=64, sink=64, tau=0.5019, kind="tiny"),
    # ~20% routed density
    "mid": Workload("mid", B=1, N=8192, H=16, D=128, sink=256, tau=0.8176, kind="field",
                    alpha=1.0),
    # the pages' shape, ~19% routed density
    "page": Workload("page", B=1, N=38247, H=56, D=128, sink=951, tau=1.951, kind="field",
                     frames=124, alpha=1.0, beta=1.0),
    # the pages' shape with routing disabled
    "page_dense": Workload("page_dense", B=1, N=38247, H=56, D=128, sink=951,
                           tau=math.inf, kind="field", frames=124, alpha=1.0, beta=1.0,
                           dense=True),
    # the pages' shape with the QK-norm + RoPE producer in front of routing
    # (the same raw tensors as "page"; tau recalibrated on the producer's outputs)
    "page_fused": Workload("page_fused", B=1, N=38247, H=56, D=128, sink=951, tau=0.7832,
                           kind="field", frames=124, alpha=1.0, beta=1.0, producer=True),
    # one GPU's share of a 4-way head split; N varies per call (see varlen_calls)
    "varlen": Workload("varlen", B=1, N=38000, H=14, D=128, sink=951, tau=1.951,
                       kind="field", frames=124, alpha=1.0, beta=1.0),
}


def varlen_calls(n_calls: int = 16) -> list[Workload]:
    """The variable-length sequence: N_k ~ U{36000..40000} from default_rng(0), seed k."""
    ns = np.random.default_rng(0).integers(36000, 40001, size=n_calls)
    base = WORKLOADS["varlen"]
    return [replace(base, name=f"varlen{k}", N=int(n), seed=k) for k, n in enumerate(ns)]


# --------------------------------------------------------------------------- drawing
def _rng(seed: int, tensor: str, b: int, h: int, part: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, _TENSOR_TAG[tensor], b, h, part])


def _frame_position(N: int, sink: int, frames: int) -> np.ndarray:
    """Position of each token inside its frame group (-1 for prefix tokens)."""
    pos = np.full(N, -1, dtype=np.int64)
    if frames <= 0 or N <= sink:
        return pos
    span = N - sink
    starts = sink + (np.arange(frames + 1) * span) // frames
    for g in range(frames):
        a, e = starts[g], starts[g + 1]
        pos[a:e] = np.arange(e - a)
    return pos


# constants of the "field" recipe
FIELD_BLOCK_AMP = 0.5
FIELD_BLOCK_RHO = 0.95
FIELD_TOKEN_RHO = 0.9
FIELD_FRAME_RHO = 0.98
FIELD_QK_SHARE = 0.2
FIELD_NOISE = 0.5


def _ar1(rng: np.random.Generator, n: int, rho: float, D: int) -> np.ndarray:
    """n steps of a D-dimensional AR(1) process with unit stationary variance."""
    e = rng.standard_normal((n, D))
    e[1:] *= math.sqrt(1.0 - rho * rho)
    return lfilter([1.0], [1.0, -rho], e, axis=0)


def _field(rng: np.random.Generator, N: int, D: int, fpos: np.ndarray, beta: float) -> np.ndarray:
    nb = -(-N // BLOCK)
    f = FIELD_BLOCK_AMP * _ar1(rng, nb, FIELD_BLOCK_RHO, D)[np.arange(N) // BLOCK]
    f += _ar1(rng, N, FIELD_TOKEN_RHO, D)
    sel = fpos >= 0
    if beta != 0.0 and sel.any():
        basis = _ar1(rng, int(fpos.max()) + 1, FIELD_FRAME_RHO, D)
        f[sel] += beta * basis[fpos[sel]]
    return f


def _head(w: Workload, b: int, h: int, N: int, fpos: np.ndarray):
    D = w.D
    if w.kind == "tiny":
        out = []
        for t in ("q", "k", "v"):
            r = _rng(w.seed, t, b, h)
            blockvec = r.standard_normal((-(-N // BLOCK), D), dtype=np.float32)
            x = r.standard_normal((N, D), dtype=np.float32) + 0.8 * blockvec[np.arange(N) // BLOCK]
            out.append(x)
        return out
    fk = _field(_rng(w.seed, "k", b, h, 0), N, D, fpos, w.beta)
    fq = _field(_rng(w.seed, "q", b, h, 0), N, D, fpos, w.beta)
    c = FIELD_QK_SHARE
    fq = c * fk + math.sqrt(1.0 - c * c) * fq
    q = w.alpha * (fq + FIELD_NOISE * _rng(w.seed, "q", b, h, 1).standard_normal((N, D)))
    k = w.alpha * (fk + FIELD_NOISE * _rng(w.seed, "k", b, h, 1).standard_normal((N, D)))
    fv = _field(_rng(w.seed, "v", b, h, 0), N, D, fpos, w.beta)
    var_v = FIELD_BLOCK_AMP ** 2 + 1.0 + w.beta ** 2 + FIELD_NOISE ** 2
    v = (fv + FIELD_NOISE * _rng(w.seed, "v", b, h, 1).standard_normal((N, D))) / math.sqrt(var_v)
    return [q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)]


def make_qkv(w: Workload, heads: list[int] | None = None, threads: int = 8):
    """Draw Q, K, V for workload ``w`` as bf16 bit patterns, each [B, N, H', D] uint16.

    ``heads`` restricts the draw to those heads (same values as in the full
    draw); H' = len(heads).
    """
    N, D, B = w.N, w.D, w.B
    heads = list(range(w.H)) if heads is None else list(heads)
    fpos = _frame_position(N, w.sink, w.frames)
    out = [np.empty((B, N, len(heads), D), dtype=np.uint16) for _ in range(3)]

    def one(job):
        b, hi = job
        for t, x in enumerate(_head(w, b, heads[hi], N, fpos)):
            out[t][b, :, hi, :] = f32_to_bf16_bits(x)

    jobs = [(b, hi) for b in range(B) for hi in range(len(heads))]
    if threads > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(max_workers=min(threads, len(jobs))) as ex:
            list(ex.map(one, jobs))
    else:
        for j in jobs:
            one(j)
    return out[0], out[1], out[2]


def packed_batch(calls: list[Workload], threads: int = 8):
    """Several workloads (same H and D, B = 1 each) as one packed batch.

    Returns (q, k, v, cu): bf16 bit patterns [T, H, D] with the samples back to
    back in the order given, and the row offsets cu (int64 [len(calls) + 1]).
    Each sample holds exactly the values make_qkv draws for its workload.
    """
    if not calls or any(c.B != 1 or c.H != calls[0].H or c.D != calls[0].D for c in calls):
        raise ValueError("packed samples need B = 1 and one H and D")
    lengths = [c.N if c.N > 0 else 0 for c in calls]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T, H, D = int(cu[-1]), calls[0].H, calls[0].D
    out = [np.empty((T, H, D), dtype=np.uint16) for _ in range(3)]
    for c, s0, s1 in zip(calls, cu[:-1], cu[1:]):
        if s1 == s0:
            continue
        for t, x in enumerate(make_qkv(c, threads=threads)):
            out[t][s0:s1] = x[0]
    return out[0], out[1], out[2], cu



def norm_weights(D: int, seed: int = 0):
    """Synthetic QK-norm weights (gamma_q, gamma_k), float32 [D] each: 1 + 0.1 N(0, 1)."""
    rng = np.random.default_rng([seed, 0x9A])
    return (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32), \
        (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)


def rope_tables(N: int, D: int, base: float = 10000.0):
    """Cosine and sine tables float32 [N, D/2] of rotary positions 0 .. N-1: pair i of
    position t turns by t * base^(-2i/D) (computed in float64, rounded once)."""
    t = np.arange(N, dtype=np.float64)[:, None]
    inv = base ** (-np.arange(0, D, 2, dtype=np.float64) / D)[None, :]
    ang = t * inv
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
