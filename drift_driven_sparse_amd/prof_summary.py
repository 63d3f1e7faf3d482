"""Summarise a rocprofv3 results database (kernel trace) as a markdown table.

Usage: python -m drift_driven_sparse_amd.prof_summary <results.db> [--title T] [--command C]
Kernels of this library are listed first; other kernels (e.g. input generation)
are aggregated in one line.  The top_kernels view stores durations in
microseconds.
"""
from __future__ import annotations

import argparse
import re
import sqlite3


def short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    m = re.match(r"(?:void )?([A-Za-z0-9_]+(?:<[^()]*>)?)", name)
    return m.group(1) if m else name[:80]


def summarise(db_path: str):
    db = sqlite3.connect(db_path)
    rows = list(db.execute("select name, total_calls, total_duration, average, percentage from top_kernels"))
    ours, other = [], [0, 0.0]
    for name, calls, total, avg, pct in rows:
        n = short(name)
        if n.split("<")[0] in ("gemm_bf16_kernel", "gemm_f32_kernel", "attn_kernel", "topk_kernel",
                               "window_update_kernel", "kmeans_entry_kernel", "prep_qkv_kernel", "row_reduce_kernel",
                               "lm_prep_kernel", "decide_kernel", "pack_bf16_kernel", "pack_f32_kernel",
                               "nvfp4_pack_kernel", "nvfp4_unpack_kernel"):
            ours.append((n, calls, total, avg))
        else:
            other[0] += calls
            other[1] += total
    return ours, other


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--title", default="rocprofv3 kernel trace")
    ap.add_argument("--command", default="")
    a = ap.parse_args()
    ours, other = summarise(a.db)
    print(f"# {a.title}\n")
    if a.command:
        print(f"Command (from the repository root on the GPU box):\n\n```\n{a.command}\n```\n")
    print("| kernel | calls | total ms | avg us |")
    print("|---|---:|---:|---:|")
    for n, calls, total, avg in ours:
        print(f"| `{n}` | {calls} | {total / 1e3:.3f} | {avg:.2f} |")
    print(f"| (other kernels: input generation, copies) | {other[0]} | {other[1] / 1e3:.3f} | |")


if __name__ == "__main__":
    main()
