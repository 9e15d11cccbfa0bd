#!/usr/bin/env python3
"""Benchmark of the Sol-Attn block-sparse attention forward on one MI355X.

One step = one forward over one batch of synthetic input: sol_route (block
pooling, pooled scores, selection) followed by sol_attn_fwd (exact 951-token
prefix sink plus the routed 64-token key blocks) at the pages' shape
[1, 38247, 56, 128] bf16 with ~19% routed density.  Inputs are resident in
HBM before the timed region.  Prints one JSON line on stdout; diagnostics go
to stderr.

The K timed steps run back to back (the headline value).  Then K more
forwards each follow a 512 MiB scratch write that evicts L2 and the MALL, and
both sets are reported as median, p10 and p90 per forward.  Other workloads:
page_dense, mid, varlen_packed (16 prompts in one packed call) and page_fused
(QK-norm + RoPE producer, routing from its block means, attention).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--workload page|page_dense|mid|varlen_packed|page_fused]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_page_sparse_traffic.json")
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_sol_amd", "csrc", "attn.hip")


def err(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter runs,
    or None when the kernel source changed since they were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    t = json.load(open(TRAFFIC_FILE))
    if t.get("attn_src_sha256_16") != src_hash(ATTN_SRC):
        return None
    return t.get("hbm_bytes_per_launch")


def _counter_kib(csv_path: str, kernel_substr: str, counter: str) -> list:
    """Per-dispatch values (KiB) of one counter for kernels whose name contains kernel_substr."""
    import csv
    vals = []
    for r in csv.DictReader(open(csv_path)):
        if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
            vals.append(float(r["Counter_Value"]))
    return vals


def record_traffic(fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str,
                   copy_bytes: int) -> dict:
    """HBM traffic of one sparse attention launch at the pages' shape from rocprofv3
    counter collections: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the attention
    kernel, each scaled by what the same counter reads for a plain device copy of
    copy_bytes bytes (the copy reads and writes copy_bytes each)."""
    import numpy as np
    fetch = np.mean(_counter_kib(fetch_csv, "attn_fwd_kernel<128, false>", "FETCH_SIZE"))
    write = np.mean(_counter_kib(write_csv, "attn_fwd_kernel<128, false>", "WRITE_SIZE"))
    cf = np.mean(_counter_kib(copy_fetch_csv, "copyBuffer", "FETCH_SIZE"))
    cw = np.mean(_counter_kib(copy_write_csv, "copyBuffer", "WRITE_SIZE"))
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    rec = {
        "attn_src_sha256_16": src_hash(ATTN_SRC),
        "fetch_kib_per_launch": round(float(fetch), 1),
        "write_kib_per_launch": round(float(write), 1),
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": round(float(cf), 1),
        "copy_write_kib": round(float(cw), 1),
        "fetch_scale": round(float(f_scale), 4),
        "write_scale": round(float(w_scale), 4),
        "hbm_bytes_per_launch": int(fetch * 1024.0 * f_scale + write * 1024.0 * w_scale),
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def cpu_baseline(w, q_bits, k_bits, v_bits, n_heads: int):
    """Time the oracle (as it stands) on a whole, stated slice of the same
    workload: the complete forward -- routing (float32 pool, score, select) and
    float64 sink + routed attention of every query block -- of the first
    n_heads heads.  The value is that slice's effective FLOP over its measured
    wall time; nothing is extrapolated."""
    import numpy as np

    import synth
    from oracle import oracle as orc

    heads = list(range(n_heads))
    qh, kh, vh = (synth.bf16_bits_to_f32(x[:, :, heads]) for x in (q_bits, k_bits, v_bits))
    t0 = time.perf_counter()
    r = orc.route(qh, kh, w.N, w.sink, w.tau)
    t_route = time.perf_counter() - t0
    t0 = time.perf_counter()
    orc.attention(qh, kh, vh, r.sel, r.geom)
    t_attn = time.perf_counter() - t0
    flops = 4.0 * w.D * r.attended_pairs
    t_all = t_route + t_attn
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"] or threadpool_info()
        blas_threads = max((p.get("num_threads", 1) for p in pools), default=1)
        blas_name = ",".join(sorted({str(p.get("internal_api", "?")) for p in pools})) or "?"
    except Exception:
        blas_threads, blas_name = os.cpu_count() or 1, "unknown"
    score_threads = min(8, os.cpu_count() or 1)
    return {
        "value": flops / t_all / 1e12,
        "unit": "TFLOP/s",
        "cores": int(max(blas_threads, score_threads)),
        "kind": "oracle",
        "sample": (f"the whole forward of heads {heads[0]}-{heads[-1]} ({n_heads} of {w.H}) of "
                   f"the same workload, measured: routing of those heads in {t_route:.2f} s, "
                   f"float64 attention of all {n_heads * r.geom.NB} of their query blocks "
                   f"({flops / 1e9:.1f} effective GFLOP) in {t_attn:.2f} s; value = effective "
                   f"FLOP / measured time ({t_all:.1f} s), no extrapolation; host cpu_count "
                   f"{os.cpu_count()}, BLAS {blas_name} with {blas_threads} threads, routing "
                   f"scores in {score_threads} threads"),
        "seconds": round(t_all, 2),
        "effective_flop": flops,
    }


def block_pairs(cnt, first, lengths, sink: int) -> int:
    """Block pairs (i, j) that hold at least one attended key, sink or routed,
    summed over the batch and heads: the 64 x 64 tiles the attention kernel
    computes.  Every query block of sample b sees its sink blocks
    ceil(min(S, n_b) / 64), plus its listed blocks, except that a listed
    straddle block (the block holding key S when S is not a multiple of 64)
    is already one of the sink blocks.  cnt and first are the routing counts
    and the first list entries, [B, H, NB] each; lengths the sample lengths."""
    import numpy as np
    cnt = np.asarray(cnt, np.int64)
    first = np.asarray(first, np.int64)
    H = cnt.shape[1]
    total = 0
    for b, n in enumerate(lengths):
        nb = (n + 63) // 64
        nsink = (min(sink, n) + 63) // 64
        c = cnt[b, :, :nb]
        total += H * nb * nsink + int(c.sum())
        if sink % 64 and sink < n:
            total -= int(((c > 0) & (first[b, :, :nb] == sink // 64)).sum())
    return total


def locality_lists(cnt, nb: int, j0: int, kind: str, seed: int = 5):
    """Routed lists with the same per-block counts as cnt ([B, H, NB] int, on the
    host) but another key locality, as int16 [B, H, NB, nb] on the host: row
    (b, h, i) holds cnt[b, h, i] ascending candidates of [j0, nb).  "prefix"
    gives every row the first candidates j0, j0 + 1, ... (every walk touches
    the same tiles: the most L2 reuse any schedule could get); "random" a
    seeded uniform subset (no structure at all).  They are valid inputs of the
    attention kernel with its work per block unchanged, for measuring what
    the key locality of the routed lists costs."""
    import torch
    B, H, nbr = cnt.shape
    ncand = nb - j0
    rows = B * H * nbr
    c = cnt.reshape(rows, 1).to(torch.int64)
    if int(c.min()) < 0 or int(c.max()) > ncand:
        raise ValueError("counts must lie in [0, NB - j0]")
    keep = torch.arange(ncand)[None, :] < c
    if kind == "prefix":
        vals = j0 + torch.arange(ncand)[None, :].expand(rows, ncand)
    elif kind == "random":
        g = torch.Generator().manual_seed(seed)
        perm = torch.rand(rows, ncand, generator=g).argsort(dim=1)
        vals = torch.where(keep, perm, torch.full_like(perm, ncand)).sort(dim=1).values + j0
    else:
        raise ValueError(f"unknown list kind {kind!r}")
    out = torch.zeros(rows, nb, dtype=torch.int16)
    out[:, :ncand] = torch.where(keep, vals, torch.zeros_like(vals)).to(torch.int16)
    return out.reshape(B, H, nbr, nb)


def trace_summary(csv_path: str, warmup: int, steps: int) -> dict:
    """Per-kernel durations from a rocprofv3 --kernel-trace CSV of one bench run.

    Each forward launches each of its kernels once, so the n-th dispatch of a
    kernel (in start order) belongs to forward n: the first `warmup` are the
    warm-ups, the next `steps` the timed back-to-back forwards of the bench
    line, the next `steps` the cold-cache forwards, and any later dispatches the
    rest of the run (the separate calls of the packed workload)."""
    import csv
    import statistics
    per = {}
    for r in csv.DictReader(open(csv_path)):
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    out = {}
    for name, d in per.items():
        d.sort()
        us = [(e - b) / 1e3 for b, e in d]
        warm = us[warmup:warmup + steps]
        cold = us[warmup + steps:warmup + 2 * steps]
        rest = us[warmup + 2 * steps:]
        out[name] = {"calls": len(us), "mean_all_us": round(statistics.mean(us), 2),
                     "calls_rest": len(rest),
                     "mean_rest_us": round(statistics.mean(rest), 2) if rest else None,
                     "mean_timed_us": round(statistics.mean(warm), 2) if warm else None,
                     "median_timed_us": round(statistics.median(warm), 2) if warm else None,
                     "mean_cold_us": round(statistics.mean(cold), 2) if cold else None,
                     "min_us": round(min(us), 2), "max_us": round(max(us), 2)}
    return out


def _median_ms(fn, reps: int):
    import torch
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(reps):
        ev0.record()
        fn()
        ev1.record()
        torch.cuda.synchronize()
        ts.append(ev0.elapsed_time(ev1))
    ts.sort()
    return {"median_ms": round(ts[len(ts) // 2], 4), "min_ms": round(ts[0], 4),
            "max_ms": round(ts[-1], 4)}


def list_locality(args, sol, w, q, k, v, o, idx, cnt, order) -> int:
    """The attention kernel on list sets of equal counts and different key
    locality (locality_lists), round robin, --steps launches each."""
    import torch
    kinds = args.list_locality.split(",")
    B, H, NB, _ = idx.shape
    j0 = w.sink // 64 if w.sink < w.N else NB
    cnt_h = cnt.cpu()
    sets = {}
    for kind in kinds:
        if kind == "routed":
            sets[kind] = idx
        else:
            sets[kind] = locality_lists(cnt_h, NB, j0, kind).to(q.device)
    times = {kind: [] for kind in kinds}
    for kind in kinds:
        sol.attn(q, k, v, sets[kind], cnt, w.sink, out=o, order=order)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        for kind in kinds:
            times[kind].append(_median_ms(
                lambda: sol.attn(q, k, v, sets[kind], cnt, w.sink, out=o, order=order), 1)["median_ms"])
    rec = {"list_locality": {kind: {"median_ms": round(sorted(t)[len(t) // 2], 4),
                                    "min_ms": round(min(t), 4), "max_ms": round(max(t), 4)}
                             for kind, t in times.items()},
           "launches_each": args.steps, "schedule": "routing order (longest list first)",
           "workload": f"[{w.B},{w.N},{w.H},{w.D}] bf16, sink {w.sink}, tau {w.tau}"}
    print(json.dumps(rec), flush=True)
    return 0


def platform_flash(args, sol, q, k, v, o) -> int:
    """torch's scaled_dot_product_attention restricted to its flash backend
    (an unavailable backend raises instead of falling back to the math path)
    against sol_attn_dense_fwd on the same inputs."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    B, N, H, D = q.shape
    flop = 4.0 * B * H * N * N * D
    ours = _median_ms(lambda: sol.attn_dense(q, k, v, out=o), max(args.steps, 3))
    rec = {"ours_dense": {**ours, "tflops": round(flop / ours["median_ms"] / 1e9, 1)}}
    qt, kt, vt = (x.permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
    try:
        rec["torch_fa_library"] = str(torch.backends.cuda.preferred_rocm_fa_library())
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            ot = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
            torch.cuda.synchronize()
            t = _median_ms(lambda: torch.nn.functional.scaled_dot_product_attention(qt, kt, vt),
                           max(args.steps, 3))
        rec["torch_flash"] = {**t, "tflops": round(flop / t["median_ms"] / 1e9, 1)}
        rec["max_abs_diff"] = float((ot.permute(0, 2, 1, 3).float() - o.float()).abs().max())
    except RuntimeError as e:
        rec["torch_flash"] = f"unavailable: {str(e)[:200]}"
    rec["workload"] = f"dense [{B},{N},{H},{D}] bf16"
    print(json.dumps(rec), flush=True)
    return 0


def varlen_calls(args, sol, synth) -> int:
    """One forward (routing + attention) per variable-length prompt, each on its
    own fixed-length call of the one ahead-of-time build; per call the median
    and best of --steps timed forwards after one untimed forward (the first
    call's first forward is reported too: no compile happens at a new length)."""
    import numpy as np
    import torch
    calls = synth.varlen_calls()
    rows, first_ms = [], None
    ev0, evm, ev1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    for n, w in enumerate(calls):
        q, k, v = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda:0")
                   for x in synth.make_qkv(w))
        o = torch.empty_like(q)
        ws = torch.empty(max(sol.route_workspace_bytes(q), 256), dtype=torch.uint8, device=q.device)
        outs = sol.route_outputs(q)
        ts, tr, ta = [], [], []
        for rep in range(args.steps + 1):
            ev0.record()
            sol.route(q, k, w.tau, w.sink, workspace=ws, out=outs)
            evm.record()
            sol.attn(q, k, v, outs[0], outs[1], w.sink, out=o, order=outs[3])
            ev1.record()
            torch.cuda.synchronize()
            t = ev0.elapsed_time(ev1)
            if n == 0 and rep == 0:
                first_ms = t
            if rep > 0:
                ts.append(t)
                tr.append(ev0.elapsed_time(evm))
                ta.append(evm.elapsed_time(ev1))
        tot = outs[2].cpu().numpy()
        nb = sol.num_blocks(w.N)
        ncand = nb - (nb if w.sink >= w.N else w.sink // 64)
        flop = 4.0 * w.D * int(tot[1])
        med, best = float(np.median(ts)), float(min(ts))
        rows.append({"N": w.N, "median_ms": round(med, 4), "best_ms": round(best, 4),
                     "route_ms": round(float(np.median(tr)), 4),
                     "attn_ms": round(float(np.median(ta)), 4),
                     "tflops_median": round(flop / med / 1e9, 1),
                     "attn_tflops": round(flop / float(np.median(ta)) / 1e9, 1),
                     "route_density": round(int(tot[0]) / (w.B * w.H * nb * ncand), 6),
                     "effective_flop": flop})
        err(f"{w.name}: N={w.N} median {med:.3f} ms, best {best:.3f} ms, "
            f"{flop / med / 1e9:.1f} TFLOP/s")
        del q, k, v, o, ws, outs
    per_flop = [r["median_ms"] / r["effective_flop"] for r in rows]
    rec = {"varlen_calls": rows, "steps_each": args.steps,
           "worst_over_median_ms_per_flop": round(max(per_flop) / float(np.median(per_flop)), 4),
           "first_forward_ms": round(first_ms, 3),
           "workload": f"16 prompts, N in [36000, 40000] from the seeded draw, H {calls[0].H}, "
                       f"D {calls[0].D}, sink {calls[0].sink}, tau {calls[0].tau}, bf16"}
    print(json.dumps(rec), flush=True)
    return 0


def gemm_peak(args) -> int:
    """Measured dense bf16 contraction rate of this chip: torch.matmul on square,
    contiguous, seeded operands (float32 accumulation inside the library), the
    median of --steps launches after warm-up, at three sizes."""
    import torch
    g = torch.Generator(device="cuda:0").manual_seed(0)
    rec = {"gemm_bf16": {}}
    for n in (4096, 8192, 16384):
        a = torch.randn(n, n, device="cuda:0", generator=g).to(torch.bfloat16)
        b = torch.randn(n, n, device="cuda:0", generator=g).to(torch.bfloat16)
        c = torch.empty(n, n, device="cuda:0", dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        t = _median_ms(lambda: torch.matmul(a, b, out=c), max(args.steps, 5))
        tf = 2.0 * n ** 3 / t["median_ms"] / 1e9
        rec["gemm_bf16"][str(n)] = {**t, "tflops": round(tf, 1),
                                    "frac_of_spec": round(tf / PEAK_BF16_TFLOPS, 4)}
        del a, b, c
    rec["spec_peak_tflops"] = PEAK_BF16_TFLOPS
    rec["library"] = "torch.matmul (hipBLASLt / rocBLAS), bf16 in and out"
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="page",
                    choices=["page", "page_dense", "mid", "varlen_packed", "page_fused"],
                    help="varlen_packed: the 16 variable-length prompts (N in [36000, 40000], "
                         "H = 14) packed into one call; page_fused: the pages' shape with the "
                         "QK-norm + RoPE producer in front, routing from its block means")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=4,
                    help="heads whose whole forward the oracle baseline times")
    ap.add_argument("--attn-loop", type=float, default=0.0, metavar="SECONDS",
                    help="only run the attention kernel of the workload (sparse for page, dense "
                         "for page_dense) back to back for SECONDS, printing 'start' when the "
                         "loop begins and the mean launch time at the end: a steady load for "
                         "reading the board's power and clock sensors")
    ap.add_argument("--list-locality", metavar="KINDS",
                    help="page workload only: time the attention kernel --steps times on each "
                         "of the comma-separated list sets routed, prefix and random (same "
                         "counts per block, different key locality), print one JSON object "
                         "and exit")
    ap.add_argument("--platform-flash", action="store_true",
                    help="page_dense workload only: time torch's own flash attention "
                         "(scaled_dot_product_attention, flash backend only) against this "
                         "library's dense kernel on the same inputs, print one JSON object "
                         "and exit")
    ap.add_argument("--gemm-peak", action="store_true",
                    help="time torch's bf16 matrix product (the platform's GEMM library) on "
                         "square contiguous operands of 4096, 8192 and 16384, print one JSON "
                         "object with the measured dense bf16 MFMA rate and exit (context for "
                         "the spec peak the roofline uses)")
    ap.add_argument("--varlen-calls", action="store_true",
                    help="the 16 variable-length prompts (N in [36000, 40000], H = 14) as 16 "
                         "separate forwards on the one build: per call the median and best of "
                         "--steps timed forwards, effective TFLOP/s and densities, then the "
                         "worst / median time per FLOP; one JSON object, then exit")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="per-kernel durations (all, timed window, cold window) from a rocprofv3 "
                         "kernel-trace CSV of a bench run with the same --warmup/--steps; no GPU")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (for scaling "
                         "the HBM counters FETCH_SIZE / WRITE_SIZE) and exit")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                         "COPY_WRITE_CSV"),
                    help="write the attention kernel's HBM bytes per launch from rocprofv3 "
                         "counter CSVs (no GPU needed) and exit")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30,
                    help="size of the copy behind COPY_*_CSV (default 1 GiB)")
    args = ap.parse_args()
    if args.trace_summary:
        print(json.dumps(trace_summary(args.trace_summary, args.warmup, args.steps), indent=1))
        return 0
    if args.record_traffic:
        rec = record_traffic(*args.record_traffic, copy_bytes=args.copy_bytes)
        print(json.dumps(rec))
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        err(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}, "
            f"WORLD_SIZE {world}); the path would shard by head across GPUs, but only the "
            "one-GPU path exists")
        return 2

    import numpy as np
    import torch

    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        err(f"copied {args.copy_calibration} bytes 5 times")
        return 0

    if args.gemm_peak:
        return gemm_peak(args)

    import block_sparse_attention_sol_amd as sol
    import synth

    if args.varlen_calls:
        return varlen_calls(args, sol, synth)

    packed = args.workload == "varlen_packed"
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    if packed:
        # one packed batch: the samples back to back in [T, H, D], rows through offsets
        calls = synth.varlen_calls()
        w = calls[0]
        q_bits, k_bits, v_bits, cu_h = synth.packed_batch(calls)
        lengths = [int(n) for n in np.diff(cu_h)]
        B, N, H, D = len(calls), max(lengths), w.H, w.D
    else:
        w = synth.WORKLOADS[args.workload]
        q_bits, k_bits, v_bits = synth.make_qkv(w)
        B, N, H, D = w.B, w.N, w.H, w.D
        lengths = [N] * B
    dense = w.dense
    err(f"generated {args.workload} inputs in {time.perf_counter() - t0:.1f} s")

    def to_dev(b):
        return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    vk = {}
    if packed:
        vk = {"cu_seqlens": torch.tensor(np.asarray(cu_h, np.int32), device=dev), "max_seqlen": N}
    o = torch.empty_like(q)
    ws = torch.empty(max(sol.route_workspace_bytes(q, **vk), 256), dtype=torch.uint8, device=dev)
    outs = sol.route_outputs(q, **vk)
    idx, cnt, totals, order = outs
    producer = w.producer
    qa, ka = q, k                      # what attention reads
    if producer:
        # raw projections in q, k; the producer writes normalised, rotated qa, ka
        gq, gk = synth.norm_weights(D)
        cos, sin = synth.rope_tables(N, D)
        pargs = tuple(torch.from_numpy(x).to(dev) for x in (gq, gk)) + (synth.NORM_EPS,) + \
            tuple(torch.from_numpy(x).to(dev) for x in (cos, sin))
        qa, ka = torch.empty_like(q), torch.empty_like(k)

    def routing_stage(mark=None):
        if producer:
            sol.qk_norm_rope_pool(q, k, *pargs, sink=w.sink, out=(qa, ka), workspace=ws, **vk)
            if mark is not None:
                mark.record()
            sol.route_pooled(q, ws, w.tau, w.sink, out=outs, **vk)
        else:
            if mark is not None:
                mark.record()
            sol.route(q, k, w.tau, w.sink, workspace=ws, out=outs, **vk)

    def step():
        if dense:
            sol.attn_dense(q, k, v, out=o, **vk)
        else:
            routing_stage()
            sol.attn(qa, ka, v, idx, cnt, w.sink, out=o, order=order, **vk)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    if args.list_locality:
        if args.workload != "page":
            err("--list-locality needs --workload page")
            return 2
        return list_locality(args, sol, w, q, k, v, o, idx, cnt, order)
    if args.platform_flash:
        if args.workload != "page_dense":
            err("--platform-flash needs --workload page_dense")
            return 2
        return platform_flash(args, sol, q, k, v, o)

    if args.attn_loop > 0:
        def attn_only():
            if dense:
                sol.attn_dense(q, k, v, out=o, **vk)
            else:
                sol.attn(qa, ka, v, idx, cnt, w.sink, out=o, order=order, **vk)
        err("start")
        t_loop0 = time.perf_counter()
        launches = 0
        while time.perf_counter() - t_loop0 < args.attn_loop:
            for _ in range(4):
                attn_only()
            torch.cuda.synchronize()
            launches += 4
        dt = time.perf_counter() - t_loop0
        err(f"{args.workload} attention loop: {launches} launches in {dt:.2f} s, "
            f"{dt / launches * 1e3:.3f} ms per launch")
        return 0

    # per-kernel events on the stream the kernels run on (torch's current stream)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        ev[s][0].record()
        if not dense:
            routing_stage(ev[s][1])
        else:
            ev[s][1].record()
        ev[s][2].record()
        if dense:
            sol.attn_dense(q, k, v, out=o, **vk)
        else:
            sol.attn(qa, ka, v, idx, cnt, w.sink, out=o, order=order, **vk)
        ev[s][3].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(end) / args.steps
    prod_ms = [e[0].elapsed_time(e[1]) for e in ev]
    route_ms = [e[1].elapsed_time(e[2]) for e in ev]
    attn_ms = [e[2].elapsed_time(e[3]) for e in ev]
    t_prod = float(np.mean(prod_ms)) if producer else 0.0
    t_route = float(np.mean(route_ms)) if not dense else 0.0
    t_attn = float(np.mean(attn_ms))
    step_ms = [e[0].elapsed_time(e[3]) for e in ev]

    # cold-cache repetitions: a 512 MiB scratch write before each forward
    # evicts L2 and the MALL; only the forward itself is timed
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold_ms = []
    for _ in range(args.steps):
        scratch.fill_(1)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        step()
        c1.record()
        torch.cuda.synchronize()
        cold_ms.append(c0.elapsed_time(c1))
    del scratch

    def spread(x):
        return {"median": round(float(np.median(x)), 4), "p10": round(float(np.percentile(x, 10)), 4),
                "p90": round(float(np.percentile(x, 90)), 4)}
    sep_ms = None
    if packed:
        # the same prompts as one fixed-length call each, for comparison
        views = [tuple(x[int(a):int(b)].unsqueeze(0) for x in (q, k, v))
                 for a, b in zip(cu_h[:-1], cu_h[1:])]
        sep_out = [sol.route_outputs(vw[0]) for vw in views]
        sep_o = [torch.empty_like(vw[0]) for vw in views]

        def separate():
            for (qs, ks, vs), so, oo in zip(views, sep_out, sep_o):
                sol.route(qs, ks, w.tau, w.sink, workspace=ws, out=so)
                sol.attn(qs, ks, vs, so[0], so[1], w.sink, out=oo, order=so[3])
        separate()
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(args.steps):
            separate()
        s1.record()
        torch.cuda.synchronize()
        sep_ms = s0.elapsed_time(s1) / args.steps

    NB = sol.num_blocks(N)
    # per-sample blocks and candidates (all equal unless the batch is packed)
    nbs = [sol.num_blocks(n) for n in lengths]
    ncands = [nb - (nb if w.sink >= n else w.sink // 64) for n, nb in zip(lengths, nbs)]
    if dense:
        pairs = H * sum(n * n for n in lengths)
        routed = H * sum(nb * nb for nb in nbs)
        cand_pairs = routed
    else:
        tot = totals.cpu().numpy()
        routed, pairs = int(tot[0]), int(tot[1])
        cand_pairs = H * sum(nb * nc for nb, nc in zip(nbs, ncands))
    flop_eff = 4.0 * D * pairs
    # tile FLOP: what the attention kernel computes, 64 x 64 tiles including
    # their masked parts (sink tiles, then each listed block; a listed
    # straddle block shares the last sink tile)
    if dense:
        tile_pairs = H * sum(nb * nb for nb in nbs)
    else:
        tile_pairs = block_pairs(cnt.cpu().numpy(), idx[..., 0].cpu().numpy(), lengths, w.sink)
    flop_tile = 4.0 * D * 64 * 64 * tile_pairs
    rho_route = routed / cand_pairs
    rho_pair = pairs / (H * sum(n * n for n in lengths))
    # block density: block pairs (i, j) with at least one attended key, sink or
    # routed, over all B H NB^2 block pairs (the straddle block counts once);
    # these are exactly the 64 x 64 tiles the kernel computes
    block_den = H * sum(nb * nb for nb in nbs)
    rho_block = tile_pairs / block_den
    tflops = flop_eff / (ms_step * 1e-3) / 1e12
    attn_tflops = flop_eff / (t_attn * 1e-3) / 1e12
    route_bytes = (sum(n * H * D * 2 + max(n - w.sink, 0) * H * D * 2 for n in lengths)
                   + 2 * routed + 4 * B * H * NB + 16) if not (dense or producer) else 0
    route_gbs = route_bytes / (t_route * 1e-3) / 1e9 if route_bytes else None
    prod_gbs = None
    if producer:
        # Q and K read and written once, the block means written, tables and weights read
        prod_bytes = (4 * sum(lengths) * H * D * 2 + 2 * B * H * NB * D * 4 + 2 * N * (D // 2) * 4
                      + 2 * D * 4)
        prod_gbs = prod_bytes / (t_prod * 1e-3) / 1e9
        err(f"producer (QK-norm + RoPE + block means): {t_prod:.3f} ms, {prod_gbs:.0f} GB/s "
            f"({prod_gbs / PEAK_HBM_GBS:.1%} of HBM peak)")
    err(f"{args.workload}: {ms_step:.3f} ms/forward (route {t_route:.3f} ms, attention {t_attn:.3f} ms), "
        f"effective {tflops:.1f} TFLOP/s, attention {attn_tflops:.1f} TFLOP/s "
        f"({attn_tflops / PEAK_BF16_TFLOPS:.1%} of bf16 peak), routing "
        f"{f'{route_gbs:.0f} GB/s' if route_gbs else ('off' if dense else 'from block means')}; "
        f"route density {rho_route:.4%}, block density {rho_block:.4%}, pair density "
        f"{rho_pair:.4%}; "
        f"wall {wall:.2f} s for {args.steps} steps")

    err(f"per forward: warm median {np.median(step_ms):.3f} ms (p10 {np.percentile(step_ms, 10):.3f}, "
        f"p90 {np.percentile(step_ms, 90):.3f}); cold (L2 and MALL evicted) median "
        f"{np.median(cold_ms):.3f} ms (p10 {np.percentile(cold_ms, 10):.3f}, "
        f"p90 {np.percentile(cold_ms, 90):.3f})")
    # the committed counter runs cover the pages' sparse shape only
    traffic = measured_traffic() if args.workload == "page" else None
    if packed:
        desc = (f"varlen_packed: one Sol-Attn forward (routing + sink/routed attention) of "
                f"{B} prompts with N in [{min(lengths)}, {max(lengths)}] packed in one call "
                f"([{sum(lengths)},{H},{D}] bf16 with row offsets), sink {w.sink}, 64-token "
                f"blocks, tau {w.tau}")
    elif dense:
        desc = f"{w.name}: dense attention (routing disabled) on [{B},{N},{H},{D}] bf16"
    elif producer:
        desc = (f"{w.name}: QK-norm + RoPE producer writing Q, K and their block means, routing "
                f"from the means, then sink/routed attention on [{B},{N},{H},{D}] bf16, sink "
                f"{w.sink}, 64-token blocks, tau {w.tau}")
    else:
        desc = (f"{w.name}: one Sol-Attn forward (routing + sink/routed attention) on "
                f"[{B},{N},{H},{D}] bf16, sink {w.sink}, 64-token blocks, tau {w.tau}")
    rec = {
        "metric": "ms/forward + effective TFLOP/s (MFMA % peak) at [1,38247,56,128], ~19% density",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": desc,
            "B": B, "N": N, "H": H, "D": D, "sink": w.sink, "tau": w.tau,
            "route_density": round(rho_route, 6), "block_density": round(rho_block, 6),
            "pair_density": round(rho_pair, 6),
            "densities_exact": {"route": [routed, cand_pairs], "block": [tile_pairs, block_den],
                                "pair": [pairs, H * sum(n * n for n in lengths)]},
            "routed_block_pairs": routed, "attended_pairs": pairs,
            "tile_flop": flop_tile, "effective_flop": flop_eff,
            "tile_flop_waste": round(1.0 - flop_eff / flop_tile, 5),
            "route_ms": round(t_route, 4), "attn_ms": round(t_attn, 4),
            "warm_ms_per_forward": spread(step_ms), "cold_ms_per_forward": spread(cold_ms),
            **({"producer_ms": round(t_prod, 4), "producer_gbs": round(prod_gbs, 1),
                "producer_hbm_frac": round(prod_gbs / PEAK_HBM_GBS, 4)} if producer else {}),
            "route_gbs": round(route_gbs, 1) if route_gbs else None,
            "route_hbm_frac": round(route_gbs / PEAK_HBM_GBS, 4) if route_gbs else None,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    if (packed or producer) and not args.no_cpu_baseline:
        err("cpu baseline: timed on the default (pages' shape) workload only")
    if not args.no_cpu_baseline and not packed and not producer:
        t0 = time.perf_counter()
        rec["cpu_baseline"] = cpu_baseline(w, q_bits, k_bits, v_bits, args.cpu_heads)
        err(f"cpu baseline took {time.perf_counter() - t0:.1f} s")
    if packed:
        rec["config"]["sample_lengths"] = lengths
        rec["config"]["separate_calls_ms"] = round(sep_ms, 4)
        err(f"the same {B} prompts as separate calls: {sep_ms:.3f} ms per forward")
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
