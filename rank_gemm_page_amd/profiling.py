"""Summaries of rocprofv3 runs of bench.py, for the committed profiles.

Three runs of the same bench command feed one summary:
  * ``--kernel-trace --stats --output-format csv``: per-kernel call counts and
    average durations (``*_kernel_stats.csv``);
  * ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` (``*_counter_collection.csv``):
    per-dispatch KiB read and written between the L2 and the memory fabric.

The counters are scaled by what they read for a copy kernel of known size in
the same run: the bench's last-level-cache flush, a device copy that reads
flush_mib/2 MiB and writes flush_mib/2 MiB per step.

Usage:
  python -m rank_gemm_page_amd.profiling --config decode7b --trace DIR --fetch DIR \
      --write DIR --command "..." [--flush-mib 1024] [--out profiles]
writes ``<out>/fused_kernel_<config>.txt`` (the figures and the commands) and
``<out>/traffic_<config>.json`` (bytes per launch, read by bench.py while the
kernel sources are unchanged).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_source_hash(kind: str = "fused") -> str:
    """Hash of the sources the measured kernel depends on: every host and
    device source except the bandwidth probes and the no-allocation wrapper,
    and for the delta's kernels ("fused") not the base-plus-delta kernel's
    own file either."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rank_gemm_page_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if not name.endswith((".hip", ".cpp", ".h")):
            continue            # build by-products are not sources
        if name in ("slora_probe.hip", "slora_noalloc.hip"):
            continue            # measurement probes and a wrapper: no kernel of the delta
        if kind == "fused" and name == "slora_forward.hip":
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def _one(pattern: str) -> str:
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def short_name(name: str) -> str:
    if "forward_kernel" in name:       # one entry per tile shape
        m = re.search(r"forward_kernel<(\d+), ?(\d+)", name) or re.search(r"forward_kernelILi(\d+)ELi(\d+)E", name)
        return f"forward_kernel<{m.group(1)},{m.group(2)}>" if m else "forward_kernel"
    for key in ("fused_kernel", "shrink_kernel", "combine_kernel", "expand_kernel", "scatter_pages_kernel"):
        if key in name:
            return key
    return name.split("(")[0][:60]


def kernel_stats(trace_dir: str):
    rows = list(csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_stats.csv")))))
    out = []
    for r in rows:
        out.append({"name": r["Name"], "short": short_name(r["Name"]), "calls": int(r["Calls"]),
                    "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                    "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return out


def counter_values(run_dir: str, counter: str):
    """{(kernel name, grid size): [KiB per dispatch, ...]} for one counter."""
    path = _one(os.path.join(run_dir, "**", "*counter_collection.csv"))
    by = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            by[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return by


def traffic(fetch_dir: str, write_dir: str, flush_mib: int):
    """Bytes per dispatch of each slora kernel, scaled by the flush copy."""
    fetch = counter_values(fetch_dir, "FETCH_SIZE")
    write = counter_values(write_dir, "WRITE_SIZE")
    known_kib = flush_mib * 1024 / 2          # the flush reads and writes half of flush_mib each

    def calib(by):
        copies = [(g, v) for (n, g), v in by.items() if n == COPY_KERNEL]
        g, v = max(copies, key=lambda gv: gv[0])   # the largest copy is the flush
        return statistics.median(v) / known_kib, len(v)

    f_fac, f_n = calib(fetch)
    w_fac, w_n = calib(write)
    kernels = {}
    for (name, grid), vals in fetch.items():
        if "slora" not in name or "scatter" in name:
            continue
        wv = write.get((name, grid), [])
        k = short_name(name)
        kernels[k] = {"fetch_bytes": statistics.median(vals) * 1024 / f_fac,
                      "write_bytes": (statistics.median(wv) * 1024 / w_fac) if wv else 0.0,
                      "dispatches": len(vals), "grid": grid,
                      "fetch_kib_raw": statistics.median(vals),
                      "write_kib_raw": statistics.median(wv) if wv else 0.0}
    return {"fetch_factor": f_fac, "write_factor": w_fac, "calibration_dispatches": [f_n, w_n],
            "kernels": kernels}


def write_summary(config, trace_dir, fetch_dir, write_dir, command, flush_mib, out_dir,
                  algorithmic_bytes=None, event_us=None, kind="fused"):
    """kind "fused": the delta's fused kernel (profiles/fused_kernel_<config>.txt,
    traffic_<config>.json); "forward": the base-plus-delta kernel
    (forward_kernel_<config>.txt, traffic_forward_<config>.json)."""
    dom = f"{kind}_kernel"
    tname = f"traffic_{config}.json" if kind == "fused" else f"traffic_{kind}_{config}.json"
    stats = kernel_stats(trace_dir)
    tr = traffic(fetch_dir, write_dir, flush_mib)
    for s in stats:            # the kernel trace's average duration beside the bytes
        if s["short"] in tr["kernels"]:
            tr["kernels"][s["short"]]["trace_avg_us"] = s["avg_us"]
    tr["kernel_source_hash"] = kernel_source_hash(kind)
    tr["config"] = config
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, tname), "w") as f:
        json.dump(tr, f, indent=1)
    lines = [f"# rocprofv3 summary: slora kernels, workload {config}", "",
             "Commands (run from the repository root on one MI355X, TMPDIR=/tmp):"]
    lines += [f"  {c}" for c in command]
    lines += ["", "Kernel trace (--kernel-trace --stats):",
              f"  {'kernel':24s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s}"]
    for s in stats:
        lines.append(f"  {s['short']:24s} {s['calls']:6d} {s['avg_us']:9.3f} {s['min_us']:9.3f} "
                     f"{s['max_us']:9.3f}")
    lines += ["", f"PMC (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), calibrated on the "
                  f"{flush_mib} MiB flush copy:",
              f"  FETCH_SIZE reads {tr['fetch_factor']:.4f} x the copy's bytes read, "
              f"WRITE_SIZE {tr['write_factor']:.4f} x its bytes written"]
    for k, v in tr["kernels"].items():
        lines.append(f"  {k}: fetch {v['fetch_kib_raw']:.1f} KiB raw -> {v['fetch_bytes'] / 1e6:.2f} MB, "
                     f"write {v['write_kib_raw']:.1f} KiB raw -> {v['write_bytes'] / 1e6:.2f} MB "
                     f"({v['dispatches']} dispatches)")
    mine = [v for k, v in tr["kernels"].items() if k.startswith(dom)]
    if algorithmic_bytes and mine:
        # per call: one dispatch of each of the measured kernel's launches
        tot = sum(v["fetch_bytes"] + v["write_bytes"] for v in mine)
        lines.append(f"  {dom} per call: traffic / algorithmic bytes = {tot / 1e6:.2f} / "
                     f"{algorithmic_bytes / 1e6:.2f} MB = {tot / algorithmic_bytes:.3f}")
    if event_us is not None:
        lines += ["", f"bench.py dispatch-event average for the same kernel: {event_us:.3f} us"]
    lines.append(f"kernel source hash: {tr['kernel_source_hash']}")
    path = os.path.join(out_dir, f"{dom}_{config}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--flush-mib", type=int, default=1024)
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--algorithmic-bytes", type=float, default=None)
    ap.add_argument("--event-us", type=float, default=None)
    ap.add_argument("--kind", choices=["fused", "forward"], default="fused")
    a = ap.parse_args()
    print(write_summary(a.config, a.trace, a.fetch, a.write, a.command, a.flush_mib, a.out,
                        a.algorithmic_bytes, a.event_us, a.kind))


if __name__ == "__main__":
    main()
