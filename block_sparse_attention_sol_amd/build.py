"""Ahead-of-time build of libsol.so for gfx950 with hipcc (in-tree).

One build serves every sequence length: N, B and H are runtime arguments.
Run as ``python block_sparse_attention_sol_amd/build.py`` (by path: importing the
package loads the library this script builds).
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsol.so")
SOURCES = ["api.cpp", "route.hip", "attn.hip", "gate.hip", "qknorm.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed float32 VALU ops stay disabled: plain scalar float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the attention softmax reads every score with VALU
    # ops, and an AGPR destination would cost one copy per score
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


# per-source extra flags: the attention walk never needs NaN semantics (the
# masks are -inf, never NaN), so max() needs no NaN canonicalisation there
EXTRA = {"attn.hip": ["-fno-honor-nans"]}


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    def compile_one(src):
        obj = os.path.join(objdir, src + f".{os.getpid()}.o")
        cmd = [hipcc, *HIPCC_FLAGS, *EXTRA.get(src, []), f"-I{INCLUDE}", f"-I{CSRC}", "-c", "-o",
               obj, os.path.join(CSRC, src)]
        cmd.remove("-shared")
        if verbose:
            print(" ".join(cmd), flush=True)
        return src, obj, subprocess.run(cmd, capture_output=True, text=True)

    # the sources compile independently; at most MAX_JOBS (or the CPU count) at once
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        results = list(pool.map(compile_one, SOURCES))
    objs = [obj for _, obj, _ in results]
    for src, obj, res in results:
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            for o in objs:
                if os.path.exists(o):
                    os.remove(o)
            raise RuntimeError(f"hipcc failed on {src}")
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    for o in objs:
        os.remove(o)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to link libsol.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
