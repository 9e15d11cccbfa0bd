"""CPU oracle for the Sol-Attn block-sparse attention forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code with
the HIP path (``block_sparse_attention_sol_amd``) and imports nothing from it.

What the forward computes (sources are the five pages on MiniMax-H3
acceleration; "clawpit" = clawpit.io article on the single-4090 run, its
paragraph on the Sol-Attn settings; "nvlabs" = nvlabs.github.io Sol-Engine
H3-DataCenter page, policy paragraph; "tokenfactory" = tokenfactory.fast post;
"blog" = ty-yang3015 "MiniAcc" post, section "What is Sol attention?"):

1. Tokens are cut into contiguous 64-token blocks in sequence order, with no
   reordering (nvlabs; tokenfactory "The benchmark was not the product" for
   the 64-token alignment).  Blk = 64, NB = ceil(N / 64).
2. An exact prefix sink: every query attends densely to the first S keys
   (S = 951 at the release setting; nvlabs, clawpit).
3. Online routing per head from compressed (block-mean-pooled) queries and
   keys under threshold tau, with the diagonal block always kept (clawpit,
   nvlabs, blog).  Key block j is a routing candidate for j >= j0 = S // 64;
   its routable keys are R(j) = [max(64 j, S), min(64 j + 64, N)).  The
   pages give no selection formula; the reading taken is
       keep j  iff  s_ij >= max_j' s_ij' - tau   or   j == i,
   with s_ij = (mean of query block i) . (mean of R(j)) / sqrt(D).
4. Attention over the sink keys and over the routed keys, merged by
   log-sum-exp (the blog's "correction term" read as the exact sink merge).

Routing (steps 1-3) is mirrored in float32 in one fixed order, so the routed
mask is reproducible bit for bit; attention (step 4) is float64.

Two further parts sit beside the path: packed variable-length batches (each
sample routed and attended on its own; route_packed, attention_packed) and
the QK-norm + RoPE producer whose outputs routing pools (qk_norm_rope, its
float32 definition in score_ref.c, and qk_norm_rope_f64, the same in float64
without rounding).

Parity of the selection rule itself against the published Sol-Attn is
unpinned: the pages print no rule and no worked example.  So is the choice of
QK-norm and RoPE variant (per-head RMS normalisation, rotation of channel
pairs by caller tables): the pages name the fused op and nothing more.
Everything else is pinned by the tests in tests/test_oracle_*.py (closed
forms, brute force on tiny inputs, float64 recomputations with error bounds,
exact selection sets, the defining properties of the normalisation and the
rotation).
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BLOCK = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "score_ref.c")
_LIB = os.path.join(_HERE, "_score_ref.so")


# --------------------------------------------------------------------------- C part
def build_c(force: bool = False) -> str:
    """Compile the float32 scores and producer (plain C, gcc) next to their source."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _clib():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build_c())
        lib.oracle_block_scores.restype = None
        lib.oracle_block_scores.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                            ctypes.c_void_p]
        lib.oracle_qk_norm_rope.restype = None
        lib.oracle_qk_norm_rope.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


# --------------------------------------------------------------------------- geometry
@dataclass(frozen=True)
class Geometry:
    N: int       # true sequence length
    S: int       # sink length as given
    NB: int      # number of 64-token blocks
    Ssink: int   # keys in the sink: min(S, N)
    j0: int      # first candidate key block (NB when there is none)

    @property
    def ncand(self) -> int:
        return self.NB - self.j0

    def q_rows(self, i: int) -> range:
        return range(BLOCK * i, min(BLOCK * i + BLOCK, self.N))

    def r_keys(self, j: int) -> range:
        """Routable keys of block j: [max(64 j, S), min(64 j + 64, N))."""
        return range(max(BLOCK * j, self.S), min(BLOCK * j + BLOCK, self.N))


def geometry(N: int, S: int) -> Geometry:
    if N < 1 or S < 0:
        raise ValueError("need N >= 1 and S >= 0")
    NB = -(-N // BLOCK)
    # a block is a candidate when it holds at least one non-sink key
    j0 = NB if S >= N else S // BLOCK
    return Geometry(N=N, S=S, NB=NB, Ssink=min(S, N), j0=j0)


def default_scale32(D: int) -> np.float32:
    """Softmax scale 1/sqrt(D), rounded once to float32 (used by routing)."""
    return np.float32(1.0 / math.sqrt(D))


# --------------------------------------------------------------------------- routing
def pool_queries(q32: np.ndarray, g: Geometry) -> np.ndarray:
    """Block means of the queries, float32, [B, H, NB, D].

    For every (b, h, block, d): acc = +0; add the block's valid rows one by one
    in ascending token order (float32 adds); mean = acc / row count (one
    correctly rounded float32 divide).  Rows past N do not exist.
    """
    B, N, H, D = q32.shape
    assert N == g.N and q32.dtype == np.float32
    acc = np.zeros((B, g.NB, H, D), np.float32)
    base = BLOCK * np.arange(g.NB)
    for t in range(BLOCK):
        rows = base + t
        ok = rows < N
        acc[:, ok] += q32[:, rows[ok]]
    cnt = np.array([len(g.q_rows(i)) for i in range(g.NB)], np.float32)
    return np.ascontiguousarray((acc / cnt[None, :, None, None]).transpose(0, 2, 1, 3))


def pool_keys(k32: np.ndarray, g: Geometry) -> np.ndarray:
    """Means of the routable keys R(j) of each candidate block, float32, [B, H, NB, D].

    Same order as pool_queries, over R(j) only; blocks j < j0 hold NaN (they
    are never candidates).
    """
    B, N, H, D = k32.shape
    assert N == g.N and k32.dtype == np.float32
    acc = np.zeros((B, g.NB, H, D), np.float32)
    base = BLOCK * np.arange(g.NB)
    for t in range(BLOCK):
        rows = base + t
        ok = (rows < N) & (rows >= g.S)
        acc[:, ok] += k32[:, rows[ok]]
    cnt = np.array([max(len(g.r_keys(j)), 1) for j in range(g.NB)], np.float32)
    kbar = acc / cnt[None, :, None, None]
    kbar[:, : g.j0] = np.nan
    return np.ascontiguousarray(kbar.transpose(0, 2, 1, 3))


def block_scores(qbar: np.ndarray, kbar: np.ndarray, g: Geometry, scale32: np.float32,
                 threads: int | None = None) -> np.ndarray:
    """Pooled scores s[b, h, i, j] (float32) for j in [j0, NB); NaN for j < j0.

    Each score is the float32 FMA chain over d ascending, then times scale32
    (see score_ref.c).
    """
    B, H, NB, D = qbar.shape
    out = np.full((B, H, NB, NB), np.nan, np.float32)
    if g.ncand == 0:
        return out
    lib = _clib()
    scale32 = np.float32(scale32)

    def one(bh):
        b, h = bh
        qa = np.ascontiguousarray(qbar[b, h], np.float32)
        ka = np.ascontiguousarray(kbar[b, h, g.j0:], np.float32)
        sa = np.empty((NB, g.ncand), np.float32)
        lib.oracle_block_scores(qa.ctypes.data, ka.ctypes.data, NB, g.ncand, D,
                                ctypes.c_float(scale32), sa.ctypes.data)
        out[b, h, :, g.j0:] = sa

    jobs = [(b, h) for b in range(B) for h in range(H)]
    threads = threads or min(8, os.cpu_count() or 1)
    if threads > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, jobs))
    else:
        for j in jobs:
            one(j)
    return out


def select_blocks(s: np.ndarray, g: Geometry, tau: float):
    """Threshold selection with the forced diagonal.

    m_i = max over candidates of s_ij; T_i = float32(m_i - tau);
    keep j iff s_ij >= T_i, and always keep j == i when i is a candidate.
    Returns (sel bool [B, H, NB, NB], T float32 [B, H, NB]).
    """
    B, H, NB, _ = s.shape
    sel = np.zeros((B, H, NB, NB), bool)
    T = np.full((B, H, NB), np.nan, np.float32)
    if g.ncand == 0:
        return sel, T
    cand = s[..., g.j0:]
    m = cand.max(axis=-1)
    T = (m - np.float32(tau)).astype(np.float32)
    sel[..., g.j0:] = cand >= T[..., None]
    diag = np.arange(g.j0, NB)
    sel[:, :, diag, diag] = True
    return sel, T


def tie_list(s: np.ndarray, T: np.ndarray, g: Geometry, rel: float = 1e-6):
    """(b, h, i, j) candidates whose score is within rel of the threshold."""
    if g.ncand == 0:
        return np.zeros((0, 4), np.int64)
    cand = s[..., g.j0:].astype(np.float64)
    t = T.astype(np.float64)[..., None]
    near = np.abs(cand - t) <= rel * np.maximum(np.abs(cand), np.abs(t))
    idx = np.argwhere(near)
    idx[:, 3] += g.j0
    return idx


def block_lists(sel: np.ndarray):
    """Ascending key-block lists and counts from the mask: (idx [B,H,NB,NB] int32 padded -1, cnt)."""
    B, H, NB, _ = sel.shape
    cnt = sel.sum(axis=-1).astype(np.int32)
    idx = np.full((B, H, NB, NB), -1, np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(NB):
                js = np.nonzero(sel[b, h, i])[0]
                idx[b, h, i, : len(js)] = js
    return idx, cnt


@dataclass
class Route:
    geom: Geometry
    qbar: np.ndarray
    kbar: np.ndarray
    scores: np.ndarray
    thresh: np.ndarray
    sel: np.ndarray
    cnt: np.ndarray
    routed_pairs: int      # sum of list lengths
    attended_pairs: int    # attended (query, key) pairs, sink included


def attended_pairs(sel: np.ndarray, g: Geometry) -> int:
    """Sum over (b, h, query rows) of (sink keys + routed keys)."""
    rk = np.array([len(g.r_keys(j)) for j in range(g.NB)], np.int64)
    rows = np.array([len(g.q_rows(i)) for i in range(g.NB)], np.int64)
    per_block = g.Ssink + sel.astype(np.int64) @ rk          # [B, H, NB]
    return int((per_block * rows).sum())


def route(q32: np.ndarray, k32: np.ndarray, N: int, S: int, tau: float,
          scale32: np.float32 | None = None, dense: bool = False) -> Route:
    """Full routing: pool, score, select.  ``dense`` selects every candidate."""
    B, _, H, D = q32.shape
    g = geometry(N, S)
    scale32 = default_scale32(D) if scale32 is None else np.float32(scale32)
    qbar = pool_queries(q32, g)
    kbar = pool_keys(k32, g)
    s = block_scores(qbar, kbar, g, scale32)
    sel, T = select_blocks(s, g, math.inf if dense else tau)
    cnt = sel.sum(axis=-1).astype(np.int32)
    return Route(geom=g, qbar=qbar, kbar=kbar, scores=s, thresh=T, sel=sel, cnt=cnt,
                 routed_pairs=int(cnt.sum()), attended_pairs=attended_pairs(sel, g))


def densities(r: Route, B: int, H: int) -> dict:
    """Exact densities as (numerator, denominator) integer pairs."""
    g = r.geom
    nsink_blocks = -(-g.Ssink // BLOCK)
    extra = r.sel[..., nsink_blocks:].sum() if nsink_blocks < g.NB else 0
    return {
        "route": (r.routed_pairs, B * H * g.NB * g.ncand),
        "block": (int(B * H * g.NB * nsink_blocks + extra), B * H * g.NB * g.NB),
        "pair": (r.attended_pairs, B * H * g.N * g.N),
    }


# --------------------------------------------------------------------------- attention
def _softmax_attend(qr: np.ndarray, kc: np.ndarray, vc: np.ndarray, scale: float):
    """Softmax attention of rows qr over keys kc / values vc (float64).

    Returns (O, L) with O = softmax(qr kc^T scale) vc and L the natural
    log-sum-exp of the logits, or None when there are no keys.
    """
    if kc.shape[0] == 0:
        return None
    z = (qr @ kc.T) * scale
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ vc) / l, (m + np.log(l))[:, 0]


def attend_block(q: np.ndarray, k: np.ndarray, v: np.ndarray, b: int, h: int, i: int,
                 sel_row: np.ndarray, g: Geometry, scale: float):
    """Output rows of query block i for (b, h): sink part and routed part merged by LSE.

    q, k, v are [B, N, H, D] arrays of the bf16 values; math is float64.
    Returns (O [rows, D] float64, L [rows] float64).
    """
    rows = g.q_rows(i)
    qr = q[b, rows.start:rows.stop, h, :].astype(np.float64)
    parts = []
    if g.Ssink > 0:
        parts.append(_softmax_attend(qr, k[b, : g.Ssink, h, :].astype(np.float64),
                                     v[b, : g.Ssink, h, :].astype(np.float64), scale))
    keys = [np.arange(g.r_keys(j).start, g.r_keys(j).stop) for j in np.nonzero(sel_row)[0]]
    if keys:
        kk = np.concatenate(keys)
        parts.append(_softmax_attend(qr, k[b, kk, h, :].astype(np.float64),
                                     v[b, kk, h, :].astype(np.float64), scale))
    parts = [p for p in parts if p is not None]
    if len(parts) == 1:
        return parts[0]
    (o1, l1), (o2, l2) = parts
    L = np.logaddexp(l1, l2)
    return np.exp(l1 - L)[:, None] * o1 + np.exp(l2 - L)[:, None] * o2, L


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel: np.ndarray, g: Geometry,
              scale: float | None = None, blocks=None):
    """Sink + routed attention, float64.

    Returns (O [B, N, H, D], LSE [B, H, N]); rows of blocks not listed in
    ``blocks`` (a list of (b, h, i)) stay NaN.  ``blocks=None`` computes all.
    """
    B, N, H, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    O = np.full((B, N, H, D), np.nan)
    L = np.full((B, H, N), np.nan)
    if blocks is None:
        blocks = [(b, h, i) for b in range(B) for h in range(H) for i in range(g.NB)]
    for b, h, i in blocks:
        o, l = attend_block(q, k, v, b, h, i, sel[b, h, i], g, scale)
        rows = g.q_rows(i)
        O[b, rows.start:rows.stop, h, :] = o
        L[b, h, rows.start:rows.stop] = l
    return O, L


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None,
                    blocks=None):
    """Full softmax attention (routing disabled), float64, same return form as attention()."""
    B, N, H, D = q.shape
    g = geometry(N, N)                   # everything is sink: one dense softmax
    sel = np.zeros((B, H, g.NB, g.NB), bool)
    return attention(q, k, v, sel, g, scale, blocks)


# --------------------------------------------------------------------------- packed batches
# Several prompts of different lengths in one call (tokenfactory.fast post,
# "The benchmark was not the product": served traffic mixes prompt lengths).
# The pages run one prompt per forward, so the reading taken for a batch is
# the plainest one: its samples are independent sequences.  Each has its own
# 64-token blocks, its own sink (its first S tokens), its own candidates and
# routing, and no query attends to another sample's keys.  The samples lie back
# to back in [T, H, D] arrays; sample b is rows cu[b] .. cu[b + 1] - 1.

def split_packed(x: np.ndarray, cu) -> list[np.ndarray]:
    """The samples of a packed [T, H, D] array as [1, n_b, H, D] arrays."""
    cu = [int(c) for c in cu]
    return [x[None, cu[b]:cu[b + 1]] for b in range(len(cu) - 1)]


def route_packed(q32: np.ndarray, k32: np.ndarray, cu, S: int, tau: float,
                 scale32: np.float32 | None = None) -> list[Route | None]:
    """Routing of each sample on its own (None for an empty sample)."""
    out = []
    for qs, ks in zip(split_packed(q32, cu), split_packed(k32, cu)):
        n = qs.shape[1]
        out.append(route(qs, ks, n, S, tau, scale32) if n > 0 else None)
    return out


def attention_packed(q: np.ndarray, k: np.ndarray, v: np.ndarray, routes, cu,
                     scale: float | None = None, dense: bool = False):
    """Sink + routed (or, with ``dense``, full) attention of each sample, float64.

    Returns (O [T, H, D] with NaN on rows outside every sample, [L_b [H, n_b]]).
    """
    T, H, D = q.shape
    O = np.full((T, H, D), np.nan)
    Ls = []
    cu = [int(c) for c in cu]
    for b, (qs, ks, vs) in enumerate(zip(split_packed(q, cu), split_packed(k, cu),
                                         split_packed(v, cu))):
        n = qs.shape[1]
        if n == 0:
            Ls.append(np.zeros((H, 0)))
            continue
        if dense:
            o, lse = dense_attention(qs, ks, vs, scale)
        else:
            o, lse = attention(qs, ks, vs, routes[b].sel, routes[b].geom, scale)
        O[cu[b]:cu[b + 1]] = o[0]
        Ls.append(lse[0])
    return O, Ls


# --------------------------------------------------------------------------- producer
# QK-norm plus RoPE, the op the tokenfactory.fast post ("Custom kernels") fuses
# right before attention.  The pages define neither part; the reading taken:
# per-head RMS normalisation over the D channels with a weight per channel and
# a small eps, then RoPE rotating channel pairs (2i, 2i + 1) by the angle whose
# cosine and sine tables give for the row's position in its sample.  Routing
# then pools the producer's bf16 outputs exactly as it pools Q and K.

def qk_norm_rope_f64(x: np.ndarray, gamma: np.ndarray, eps: float, cos=None, sin=None):
    """The definition in float64, no rounding: x [..., N, H, D] (any float), cos/sin
    [N, D/2] for the row positions (or None).  Returns float64 of x's shape."""
    x = np.asarray(x, np.float64)
    ms = (x * x).mean(axis=-1, keepdims=True)
    y = x / np.sqrt(ms + float(eps)) * np.asarray(gamma, np.float64)
    if cos is None:
        return y
    c = np.asarray(cos, np.float64)[:, None, :]           # [N, 1, D/2], broadcast over heads
    s = np.asarray(sin, np.float64)[:, None, :]
    a, b = y[..., 0::2], y[..., 1::2]
    out = np.empty_like(y)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def qk_norm_rope(x_bits: np.ndarray, gamma: np.ndarray, eps: float, cos=None, sin=None):
    """The float32 definition (score_ref.c: one ascending running sum of squares,
    then the normalisation and rotation, each step one float32 rounding):
    [B, N, H, D] bf16 bits -> bf16 bits."""
    B, N, H, D = x_bits.shape
    lib = _clib()
    g = np.ascontiguousarray(gamma, np.float32)
    cs = None if cos is None else np.ascontiguousarray(cos[:N], np.float32)
    sn = None if sin is None else np.ascontiguousarray(sin[:N], np.float32)
    out = np.empty_like(x_bits)
    for b in range(B):
        for h in range(H):
            xi = np.ascontiguousarray(x_bits[b, :, h, :], np.uint16)
            oi = np.empty_like(xi)
            lib.oracle_qk_norm_rope(xi.ctypes.data, N, D, g.ctypes.data, ctypes.c_float(eps),
                                    None if cs is None else cs.ctypes.data,
                                    None if sn is None else sn.ctypes.data, oi.ctypes.data)
            out[b, :, h, :] = oi
    return out


def qk_norm_rope_packed(x_bits: np.ndarray, cu, gamma, eps: float, cos=None, sin=None):
    """qk_norm_rope on a packed [T, H, D] batch: positions restart at 0 in every sample;
    rows outside the samples are returned unchanged."""
    out = x_bits.copy()
    cu = [int(c) for c in cu]
    for b in range(len(cu) - 1):
        if cu[b + 1] > cu[b]:
            out[cu[b]:cu[b + 1]] = qk_norm_rope(x_bits[None, cu[b]:cu[b + 1]], gamma, eps,
                                                cos, sin)[0]
    return out
