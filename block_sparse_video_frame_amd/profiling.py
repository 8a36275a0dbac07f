"""Summaries of rocprofv3 output for the attention kernels.

Reads the CSV files rocprofv3 writes with ``--output-format csv`` and turns
them into the short text/JSON summaries kept with the project:

* ``stats``: per-kernel call count and average duration from a
  ``--kernel-trace --stats`` run (``*_kernel_stats.csv``);
* ``counters``: per-kernel mean of each hardware counter per dispatch from a
  ``--pmc`` run (``*_counter_collection.csv``);
* ``traffic``: HBM bytes per call of a kernel (attn_fwd by default, or
  ``--kernel attn_qk_prep``) from a FETCH_SIZE run and a
  WRITE_SIZE run, each scaled by what the same counter reads for a plain copy
  of known size recorded in the same process (``bench.py --calibrate-copy``).

Usage::

    python -m block_sparse_video_frame_amd.profiling stats DIR
    python -m block_sparse_video_frame_amd.profiling counters DIR
    python -m block_sparse_video_frame_amd.profiling traffic FETCH_DIR WRITE_DIR --copy-bytes N \\
        --workload 720p --mode 1 --source-hash H --command "..."
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
from collections import defaultdict


def short_name(kernel: str) -> str:
    # fwd_persistent<D, NQB, NW, MASK, BOTH, CHECK>: one workgroup per CU,
    # each item on its own softmax path (BOTH), or the online path alone; the
    # CHECK kernels run mode 5
    m = re.search(r"fwd_persistent<([^>]*)>", kernel)
    if m:
        args = [x.strip() for x in m.group(1).split(",")]
        masked = len(args) > 3 and args[3] == "true"
        online = len(args) > 4 and args[4] == "false"
        checked = len(args) > 5 and args[5] == "true"
        return (f"attn_fwd[persistent{',online' if online else ''}{',masked' if masked else ''}"
                f"{',checked' if checked else ''}]")
    # fwd_kernel<D, NQB, NW, BOUND, MASK, CHECK>: one workgroup per item,
    # reported under the path it runs
    m = re.search(r"fwd_kernel<([^>]*)>", kernel)
    if m:
        args = [x.strip() for x in m.group(1).split(",")]
        path = "bound" if len(args) > 3 and args[3] == "true" else "online"
        masked = len(args) > 4 and args[4] == "true"
        checked = len(args) > 5 and args[5] == "true"
        return f"attn_fwd[{path}{',masked' if masked else ''}{',checked' if checked else ''}]"
    m = re.search(r"prep_kernel<([^>]*)>", kernel)
    if m:
        args = [x.strip() for x in m.group(1).split(",")]
        return "attn_qk_prep[norms]" if len(args) > 1 and args[1] == "true" else "attn_qk_prep"
    if "head_max_kernel" in kernel:
        return "attn_norms[head_max]"
    if "norms_kernel" in kernel:
        return "attn_norms"
    if "zero_head_max" in kernel:
        return "attn_norms[init]"
    if "copyBuffer" in kernel or "elementwise" in kernel.lower() or "copy" in kernel.lower():
        return "copy"
    return kernel[:60]


def _one(pattern: str) -> str:
    files = glob.glob(pattern, recursive=True)
    if not files:
        raise FileNotFoundError(pattern)
    return sorted(files)[0]


def stats(directory: str):
    """[(kernel, calls, avg_us, total_us)] from a --kernel-trace --stats run."""
    path = _one(os.path.join(directory, "**", "*kernel_stats.csv"))
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            out.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                        float(r["TotalDurationNs"]) / 1e3))
    return out


def dispatches(directory: str):
    """{kernel: {counter: [value per dispatch]}} from a --pmc run."""
    path = _one(os.path.join(directory, "**", "*counter_collection.csv"))
    acc = defaultdict(lambda: defaultdict(list))
    with open(path) as f:
        for r in csv.DictReader(f):
            acc[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return acc


def counters(directory: str):
    """{kernel: {counter: mean value per dispatch}} from a --pmc run."""
    return {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in dispatches(directory).items()}


def traffic(fetch_dir: str, write_dir: str, copy_bytes: float, kernel: str = "attn_fwd"):
    """HBM bytes per call of ``kernel`` (all kernels whose short name starts
    with it: every launch of one attn_fwd call, say)."""
    fc = counters(fetch_dir)
    wc = counters(write_dir)
    # the calibration copy is by far the largest copy dispatch of the run
    f_copy = max(dispatches(fetch_dir)["copy"]["FETCH_SIZE"]) * 1024.0
    w_copy = max(dispatches(write_dir)["copy"]["WRITE_SIZE"]) * 1024.0
    f_scale = copy_bytes / f_copy
    w_scale = copy_bytes / w_copy
    fetch = sum(fc[k]["FETCH_SIZE"] for k in fc if k.startswith(kernel)) * 1024.0 * f_scale
    write = sum(wc[k]["WRITE_SIZE"] for k in wc if k.startswith(kernel)) * 1024.0 * w_scale
    return {"fetch_bytes": fetch, "write_bytes": write, "bytes_per_launch": fetch + write,
            "fetch_scale": f_scale, "write_scale": w_scale,
            "copy_fetch_kib": f_copy / 1024.0, "copy_write_kib": w_copy / 1024.0}


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats"); s.add_argument("dir")
    c = sub.add_parser("counters"); c.add_argument("dir")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir"); t.add_argument("write_dir")
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--workload", required=True); t.add_argument("--mode", type=int, required=True)
    t.add_argument("--source-hash", required=True); t.add_argument("--command", required=True)
    t.add_argument("--kernel", default="attn_fwd")
    a = ap.parse_args()
    if a.cmd == "stats":
        for name, calls, avg, tot in stats(a.dir):
            print(f"{name:24s} calls {calls:5d}  avg {avg:10.2f} us  total {tot:12.2f} us")
    elif a.cmd == "counters":
        for k, d in counters(a.dir).items():
            print(k)
            for cn, v in sorted(d.items()):
                print(f"    {cn:32s} {v:.6g}")
    else:
        d = traffic(a.fetch_dir, a.write_dir, a.copy_bytes, a.kernel)
        d.update({"workload": a.workload, "mode": a.mode, "source_hash": a.source_hash, "command": a.command})
        print(json.dumps(d, indent=1))


if __name__ == "__main__":
    main()
