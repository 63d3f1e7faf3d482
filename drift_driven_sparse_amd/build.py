"""Build libpolestar.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m drift_driven_sparse_amd.build [-j N] [--incremental]
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libpolestar.so")
BUILD = os.path.join(PKG, "_build")
SOURCES = ["api.hip", "gemm.hip", "gemm_dl.hip", "gemm_dl_narrow.hip", "gemm_dl_n192.hip", "gemm_dl_n96.hip",
           "gemm_dl_wide.hip", "gemm_dl_mid.hip", "gemm_dl_w192.hip", "gemm_dl_mid8.hip", "gemm_dl_p96.hip", "gemm_dl_p160.hip", "gemm_dl_x512.hip", "attn.hip", "cluster.hip", "commit.hip", "staleness.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _stale(obj: str, src: str) -> bool:
    """True when obj is missing or older than its source or any header of the package."""
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    deps.append(os.path.join(os.path.dirname(PKG), "include", "polestar.h"))
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps if os.path.exists(d))


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    if incremental and not _stale(obj, src):
        return obj
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        msg = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    return obj


def build(jobs: int = 8, verbose: bool = True, incremental: bool = False) -> str:
    """Compiles every source (incremental: only those older than their inputs) and links."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda f: _compile(f, incremental), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--incremental", action="store_true", help="skip objects newer than their sources")
    a = ap.parse_args()
    try:
        build(a.j, incremental=a.incremental)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
