"""Summaries of rocprofv3 output as short markdown.

  python -m drift_driven_sparse_amd.prof_summary trace <results.db> [--title T] [--command C]
      kernel-trace statistics (the top_kernels view stores durations in microseconds);
      this library's kernels one per line, everything else (input generation, copies)
      aggregated.
  python -m drift_driven_sparse_amd.prof_summary pmc --fetch <fetch.csv> --write <write.csv>
      --kernels NAME [NAME ...] --probe-bytes B [--title T] [--command C]
      per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the named kernels from two counter
      runs, each scaled by the counter's reading for an element-wise copy kernel that
      reads and writes B bytes (the run's last float add kernel); ends with a JSON line
      of the figures and a hash of the projection sources they were taken from.
      --pick every:offset selects dispatches of a kernel that serves several units.
  python -m drift_driven_sparse_amd.prof_summary mfma <counters.csv> --kernels NAME [NAME ...]
      [--pick every:offset ...] [--labels L ...]
      MfmaUtil (MFMA busy %) and bf16 MFMA FLOPs per dispatch of the named kernels.
  python -m drift_driven_sparse_amd.prof_summary stall <counters.csv> [<counters.csv> ...]
      --kernels NAME [NAME ...] [--pick every:offset ...] [--labels L ...]
      where the waves of the named kernels spend their time (SQ wait and issue counters),
      LDS bank conflicts, average vector-memory latency and MFMA busy cycles per SIMD, from
      counter runs that together hold the counters listed in STALL_COUNTERS.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sqlite3

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["csrc/gemm_dl.hip", "csrc/gemm_dl_impl.h", "csrc/kernels.h", "csrc/common.h"]


def short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    m = re.match(r"(?:void )?([A-Za-z0-9_:]+(?:<[^()]*>)?)", name)
    return m.group(1) if m else name[:80]


def foreign(name: str) -> bool:
    return name.startswith("at::") or "at::native" in name or "rocclr" in name or name.startswith("__amd")


def source_hash() -> str:
    """Hash of the projection sources' code: comments and whitespace are dropped, so that a
    comment edit keeps the counters that describe the same code."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(PKG, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def trace(a):
    db = sqlite3.connect(a.db)
    rows = list(db.execute("select name, total_calls, total_duration, average, percentage from top_kernels"))
    print(f"# {a.title}\n")
    if a.command:
        print(f"Command (from the repository root on the MI355X machine):\n\n```\n{a.command}\n```\n")
    print("| kernel | calls | total ms | avg us |")
    print("|---|---:|---:|---:|")
    other = [0, 0.0]
    for name, calls, total, avg, _ in rows:
        n = short(name)
        if foreign(n):
            other[0] += calls
            other[1] += total
        else:
            print(f"| `{n}` | {calls} | {total / 1e3:.3f} | {avg:.2f} |")
    print(f"| (other kernels: input generation, copies) | {other[0]} | {other[1] / 1e3:.3f} | |")


def _per_kernel(path, counter=None):
    """Per kernel name, the counter values of its dispatches in dispatch order (rows of other
    counters skipped when ``counter`` is given), and the copy probe's value."""
    rows = list(csv.DictReader(open(path)))
    key = "Dispatch_Id" if rows and "Dispatch_Id" in rows[0] else None
    if key:
        rows.sort(key=lambda r: int(r[key]))
    agg = collections.defaultdict(list)
    probe = None
    for r in rows:
        if counter and r.get("Counter_Name") != counter:
            continue
        n = short(r["Kernel_Name"])
        v = float(r["Counter_Value"])
        agg[n].append(v)
        if "CUDAFunctorOnSelf_add<float>" in n:
            probe = v
    return agg, probe


def _pick(vals, spec):
    """Dispatches selected by 'every:offset' (e.g. 2:1 = the odd ones), or all."""
    if not spec:
        return vals
    every, off = (int(x) for x in spec.split(":"))
    return vals[off::every]


def pmc(a):
    fetch, pf = _per_kernel(a.fetch)
    write, pw = _per_kernel(a.write)
    kib = 1024.0
    f_scale = a.probe_bytes / (pf * kib)
    w_scale = a.probe_bytes / (pw * kib)
    print(f"# {a.title}\n")
    if a.command:
        print(f"Commands (from the repository root on the MI355X machine, one counter per run):\n\n```\n{a.command}\n```\n")
    print(f"Calibration: the element-wise copy reads and writes {a.probe_bytes} B; FETCH_SIZE reads "
          f"{pf:.0f} KiB (scale {f_scale:.3f}), WRITE_SIZE reads {pw:.0f} KiB (scale {w_scale:.3f}).\n")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | written MB (scaled) |")
    print("|---|---:|---:|---:|---:|---:|")
    total = 0.0
    picks = a.pick or [""] * len(a.kernels)
    for k, pk in zip(a.kernels, picks):
        fv, wv = _pick(fetch.get(k, []), pk), _pick(write.get(k, []), pk)
        if not fv or not wv:
            raise SystemExit(f"kernel {k} not in both runs")
        fa, wa = sum(fv) / len(fv), sum(wv) / len(wv)
        rd, wr = fa * kib * f_scale / 1e6, wa * kib * w_scale / 1e6
        total += rd + wr
        print(f"| `{k}` | {len(fv)} | {fa:.1f} | {wa:.1f} | {rd:.2f} | {wr:.2f} |")
    print(f"\nHBM bytes per launch of the whole unit: {total:.2f} MB.\n")
    print("```json")
    print(json.dumps({"traffic_bytes": round(total * 1e6), "kernels": a.kernels, "source_hash": source_hash()}))
    print("```")


def mfma(a):
    """Per kernel: mean MfmaUtil (% of the MFMA units' cycles busy while the GPU was active) and
    bf16 MFMA FLOPs per dispatch, from one counter run."""
    util, _ = _per_kernel(a.csv, "MfmaUtil")
    flops, _ = _per_kernel(a.csv, "MfmaFlopsBF16")
    print(f"# {a.title}\n")
    if a.command:
        print(f"Command (from the repository root on the MI355X machine):\n\n```\n{a.command}\n```\n")
    print("| unit | kernel | dispatches | MFMA busy % | bf16 MFMA GFLOP per dispatch |")
    print("|---|---|---:|---:|---:|")
    picks = a.pick or [""] * len(a.kernels)
    labels = a.labels or a.kernels
    for k, pk, lab in zip(a.kernels, picks, labels):
        u, f = _pick(util.get(k, []), pk), _pick(flops.get(k, []), pk)
        if not u:
            raise SystemExit(f"kernel {k} not in the run")
        fl = sum(f) / len(f) / 1e9 if f else float("nan")
        print(f"| {lab} | `{k}` | {len(u)} | {sum(u) / len(u):.1f} | {fl:.2f} |")


STALL_COUNTERS = ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
                  "SQ_WAIT_INST_LDS", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "VmemLatency",
                  "SQ_VALU_MFMA_BUSY_CYCLES", "TA_TA_BUSY", "TA_ADDR_STALLED_BY_TC_CYCLES"]


def stall(a):
    """Per kernel, means over its dispatches.  SQ_WAVE_CYCLES, SQ_WAIT_ANY and SQ_WAIT_INST_ANY
    count wave-cycles in units of 4 cycles; SQ_BUSY_CYCLES counts, per shader engine, the cycles
    with a wave present (32 shader engines, 4 SIMDs per compute unit, 8 compute units per engine);
    SQ_VALU_MFMA_BUSY_CYCLES is summed over the 1024 SIMDs, TA_* over the 256 texture-address
    units; VmemLatency is the average cycles from issue to return of a vector-memory instruction."""
    vals = {}
    for path in a.csv:
        for c in STALL_COUNTERS:
            per, _ = _per_kernel(path, c)
            for k, v in per.items():
                if v:
                    vals[(k, c)] = v
    print(f"# {a.title}\n")
    if a.command:
        print(f"Commands (from the repository root on the MI355X machine, one counter set per run):\n\n```\n{a.command}\n```\n")
    print("| unit | kernel | waves | cycles per wave | waiting (waitcnt, barrier) % | waiting for issue % | "
          "LDS-issue wait % | LDS bank-conflict cycles per LDS cycle | vector-memory latency (cycles) | "
          "MFMA busy % of SIMD time | TA stalled by L1 % of TA busy |")
    print("|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
    picks = a.pick or [""] * len(a.kernels)
    labels = a.labels or a.kernels
    for k, pk, lab in zip(a.kernels, picks, labels):
        def m(c):
            v = _pick(vals.get((k, c), []), pk)
            if not v:
                raise SystemExit(f"counter {c} of kernel {k} not in the runs")
            return sum(v) / len(v)
        waves, wc = m("SQ_WAVES"), m("SQ_WAVE_CYCLES")
        se_cycles = m("SQ_BUSY_CYCLES") / 32
        print(f"| {lab} | `{k}` | {waves:.0f} | {4 * wc / waves:.0f} | {100 * m('SQ_WAIT_ANY') / wc:.0f} | "
              f"{100 * m('SQ_WAIT_INST_ANY') / wc:.0f} | {100 * m('SQ_WAIT_INST_LDS') / wc:.1f} | "
              f"{m('SQ_LDS_BANK_CONFLICT') / max(m('SQ_LDS_IDX_ACTIVE'), 1):.3f} | {m('VmemLatency'):.0f} | "
              f"{100 * m('SQ_VALU_MFMA_BUSY_CYCLES') / 1024 / se_cycles:.0f} | "
              f"{100 * m('TA_ADDR_STALLED_BY_TC_CYCLES') / max(m('TA_TA_BUSY'), 1):.0f} |")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--title", default="rocprofv3 kernel trace")
    t.add_argument("--command", default="")
    p = sub.add_parser("pmc")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--kernels", nargs="+", required=True)
    p.add_argument("--probe-bytes", type=int, required=True)
    p.add_argument("--pick", nargs="*", default=None,
                   help="per kernel, 'every:offset' to select dispatches (kernels launched for several units)")
    p.add_argument("--title", default="rocprofv3 memory counters")
    p.add_argument("--command", default="")
    m = sub.add_parser("mfma")
    m.add_argument("csv")
    m.add_argument("--kernels", nargs="+", required=True)
    m.add_argument("--pick", nargs="*", default=None)
    m.add_argument("--labels", nargs="*", default=None)
    m.add_argument("--title", default="rocprofv3 MFMA counters")
    m.add_argument("--command", default="")
    st = sub.add_parser("stall")
    st.add_argument("csv", nargs="+")
    st.add_argument("--kernels", nargs="+", required=True)
    st.add_argument("--pick", nargs="*", default=None)
    st.add_argument("--labels", nargs="*", default=None)
    st.add_argument("--title", default="rocprofv3 wave-state counters")
    st.add_argument("--command", default="")
    a = ap.parse_args()
    {"trace": trace, "pmc": pmc, "mfma": mfma, "stall": stall}[a.cmd](a)


if __name__ == "__main__":
    main()
