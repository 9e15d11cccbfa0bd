"""bench.py's command line on the host: a request for more than one GPU is
refused with exit status 2 before any device work (the path runs on one GPU;
sharding by head is described, not built)."""

from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, env=env)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout.strip() == ""            # no JSON line


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4", RANK="0", LOCAL_RANK="0")
    r = _bench("--steps", "1", "--warmup", "0", env=env)
    assert r.returncode == 2
    assert "WORLD_SIZE 4" in r.stderr


def _counter_csv(path, rows):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": value})


def test_traffic_record_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    """roofline.traffic: FETCH_SIZE / WRITE_SIZE of the attention kernel (KiB per
    dispatch, averaged) scaled by what the same counters read for a plain copy
    of known size; the record holds only while the kernel source is unchanged."""
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    attn = "void sol::(anonymous namespace)::attn_fwd_kernel<128, false>(...)"
    other = "void sol::(anonymous namespace)::pool_kernel(...)"
    copy = "__amd_rocclr_copyBuffer"
    f, w, cf, cw = (str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv"))
    _counter_csv(f, [(attn, "FETCH_SIZE", 1000.0), (attn, "FETCH_SIZE", 3000.0),
                     (other, "FETCH_SIZE", 9e9)])
    _counter_csv(w, [(attn, "WRITE_SIZE", 500.0), (other, "WRITE_SIZE", 9e9)])
    copy_bytes = 1 << 20                       # a copy of 1 MiB reads and writes 1 MiB
    _counter_csv(cf, [(copy, "FETCH_SIZE", 512.0)])     # fetch counter reads half: scale 2
    _counter_csv(cw, [(copy, "WRITE_SIZE", 1024.0)])    # write counter exact: scale 1
    rec = bench.record_traffic(f, w, cf, cw, copy_bytes=copy_bytes)
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["hbm_bytes_per_launch"] == int(2000.0 * 1024 * 2 + 500.0 * 1024)
    assert bench.measured_traffic() == rec["hbm_bytes_per_launch"]
    # a record taken on another kernel source is ignored (traffic reported as null)
    import json
    stale = dict(rec, attn_src_sha256_16="0" * 16)
    (tmp_path / "traffic.json").write_text(json.dumps(stale))
    assert bench.measured_traffic() is None


def test_trace_summary_windows(tmp_path):
    """--trace-summary: the n-th dispatch of a kernel (in start order) is forward
    n; the timed window is [warmup, warmup + steps), the cold one follows it."""
    import csv
    sys.path.insert(0, ROOT)
    import bench
    path = tmp_path / "kt.csv"
    W, K = 2, 3
    # attention durations (us): warm-ups 50, 50; timed 10, 12, 14; cold 20, 20, 20
    attn_us = [50, 50, 10, 12, 14, 20, 20, 20]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 1000
        # written out of order: the summary sorts by start time
        rows = []
        for d in attn_us:
            rows.append({"Kernel_Name": "attn", "Start_Timestamp": t, "End_Timestamp": t + d * 1000})
            rows.append({"Kernel_Name": "pool", "Start_Timestamp": t + d * 1000 + 5,
                         "End_Timestamp": t + d * 1000 + 2005})
            t += 10 ** 6
        for r in reversed(rows):
            w.writerow(r)
    out = bench.trace_summary(str(path), W, K)
    a = out["attn"]
    assert a["calls"] == 8 and a["mean_timed_us"] == 12.0 and a["median_timed_us"] == 12.0
    assert a["mean_cold_us"] == 20.0 and a["min_us"] == 10.0 and a["max_us"] == 50.0
    assert out["pool"]["mean_timed_us"] == 2.0


def test_block_pairs_match_the_oracles_block_density():
    """The bench's exact block-density numerator equals the oracle's count of
    block pairs with an attended key, on routed cases with and without a
    straddle block, an empty sink, a sink as long as the sequence, and a
    batch of unequal lengths."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    from oracle import oracle as orc
    for N, S, tau, seed in [(1000, 951, 0.4, 1), (700, 0, 0.3, 2), (640, 128, 0.2, 3),
                            (300, 300, 1.0, 4), (2000, 95, 0.0, 5), (130, 63, 10.0, 6)]:
        rng = np.random.default_rng(seed)
        q = rng.standard_normal((1, N, 3, 64)).astype(np.float32)
        k = rng.standard_normal((1, N, 3, 64)).astype(np.float32)
        r = orc.route(q, k, N, S, tau)
        NB = r.geom.NB
        first = np.where(r.sel.any(-1), r.sel.argmax(-1), -1)
        got = bench.block_pairs(r.cnt, first, [N], S)
        assert got == orc.densities(r, 1, 3)["block"][0], (N, S, tau)
    # a batch of samples of unequal lengths, padded to the longest
    lengths, S, H = [500, 64, 1000], 96, 2
    NBmax = (max(lengths) + 63) // 64
    cnt = np.zeros((3, H, NBmax), np.int64)
    first = np.full((3, H, NBmax), -1, np.int64)
    want = 0
    for b, n in enumerate(lengths):
        rng = np.random.default_rng(10 + b)
        q = rng.standard_normal((1, n, H, 64)).astype(np.float32)
        k = rng.standard_normal((1, n, H, 64)).astype(np.float32)
        r = orc.route(q, k, n, S, 0.3)
        nb = r.geom.NB
        cnt[b, :, :nb] = r.cnt[0]
        first[b, :, :nb] = np.where(r.sel[0].any(-1), r.sel[0].argmax(-1), -1)
        want += orc.densities(r, 1, H)["block"][0]
    assert bench.block_pairs(cnt, first, lengths, S) == want


def test_locality_lists_are_valid_and_keep_the_counts():
    """The list sets of the locality measurement are valid attention inputs
    with the routed counts: every row holds cnt ascending candidates of
    [j0, NB); "prefix" rows are j0, j0 + 1, ...; "random" rows are a seeded
    draw (the same seed gives the same lists, another seed other lists)."""
    import torch
    sys.path.insert(0, ROOT)
    import bench
    B, H, NB, j0 = 2, 3, 40, 14
    g = torch.Generator().manual_seed(0)
    cnt = torch.randint(0, NB - j0 + 1, (B, H, NB), generator=g, dtype=torch.int32)
    cnt[0, 0, 0], cnt[0, 0, 1] = 0, NB - j0          # the empty and the full list
    for kind in ("prefix", "random"):
        L = bench.locality_lists(cnt, NB, j0, kind)
        assert L.dtype == torch.int16 and tuple(L.shape) == (B, H, NB, NB)
        for b in range(B):
            for h in range(H):
                for i in range(NB):
                    c = int(cnt[b, h, i])
                    row = L[b, h, i, :c].to(torch.int64)
                    assert row.numel() == c
                    if c:
                        assert int(row.min()) >= j0 and int(row.max()) < NB
                        assert bool((row[1:] > row[:-1]).all())
                    if kind == "prefix":
                        assert torch.equal(row, torch.arange(j0, j0 + c))
    assert torch.equal(bench.locality_lists(cnt, NB, j0, "random"),
                       bench.locality_lists(cnt, NB, j0, "random"))
    assert not torch.equal(bench.locality_lists(cnt, NB, j0, "random", seed=1),
                           bench.locality_lists(cnt, NB, j0, "random", seed=2))
    try:
        bench.locality_lists(cnt + NB, NB, j0, "prefix")
        raise AssertionError("counts above NB - j0 must be refused")
    except ValueError:
        pass
