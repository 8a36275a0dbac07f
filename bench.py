#!/usr/bin/env python3
"""Throughput of the frame-aligned block-sparse attention forward on one MI355X.

One step = the whole hot path over one batch of resident synthetic input:
attn_norms (per-row |q|, per-16-key max |k|, per-head maxima) followed by
attn_fwd (bound softmax with per-head online fallback, or the online softmax
for --mode 0).  The block list is built once per pattern (host, integer) and
uploaded before timing; its host time is reported as ``setup_ms``.

Metric: useful TFLOP/s = 4 * D * (unmasked query-key pairs) * B * H / time.
Prints one JSON line.  Default workload: the 720p chunk (1 x 8 heads x 128,
13 frames x 3600 tokens, +-1 frame window + frame 0 global).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
COPY_BYTES = 512 * 1024 * 1024


def _code_only(text: str) -> bytes:
    """C/C++ source with comments and blank space removed (so that a change of
    comments alone does not mark the committed counters as stale)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split()).encode()


# The device sources each kernel is built from (host-side declarations in the
# headers are not part of it): counters taken on a kernel stay valid while
# these are unchanged.
KERNEL_SOURCES = {
    "attn_fwd": ["attn_fwd.hip", "bsvf_device.h"],
    "attn_qk_prep": ["attn_qk_prep.hip", "attn_norms.hip", "bsvf_device.h"],
}


def source_hash(kernel: str = "attn_fwd") -> str:
    """Hash of the code (not the comments) of one kernel's sources."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_video_frame_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), encoding="utf-8") as fh:
            h.update(name.encode() + _code_only(fh.read()))
    return h.hexdigest()[:16]


def load_traffic(workload: str, mode: int):
    """HBM bytes per attn_fwd launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != source_hash() or int(d.get("mode", -1)) != mode:
        return None
    return d.get("bytes_per_launch")


def load_producer_traffic(workload: str):
    """HBM bytes per attn_qk_prep launch (with norms) from committed counter
    runs on the current kernel sources, else None."""
    path = os.path.join(ROOT, "profiles", f"attn_qk_prep_{workload}_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    return d.get("bytes_per_launch") if d.get("source_hash") == source_hash("attn_qk_prep") else None


def time_producer(bs, wl, q, k, dev, steps: int, warmup: int):
    """attn_qk_prep with the norms in its epilogue, against the same producer
    without them followed by attn_norms over its output (the unfused order).
    Pre-norm Q and K are the workload's seeded tensors; weights and rotary
    tables come from the seeded generators.  Outputs go to separate buffers."""
    import torch
    from synth import FRAME_GRID, norm_weights, rope_tables
    B, H, N, D = wl.batch, wl.heads, wl.seq_len, wl.head_dim
    gq, gk = (torch.from_numpy(x).to(dev) for x in norm_weights(D))
    cos, sin = (torch.from_numpy(x).to(dev) for x in rope_tables(wl.pattern, D, FRAME_GRID[wl.name]))
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    nm = (torch.empty(B, H, N, dtype=torch.float32, device=dev),
          torch.empty(B, H, N // 16, dtype=torch.float32, device=dev),
          torch.empty(B, H, 2, dtype=torch.float32, device=dev))

    def fused():
        bs.qk_prep(q, k, gq, gk, cos, sin, 1e-6, q_out=qo, k_out=ko, norms_out=nm)

    def plain():
        bs.qk_prep(q, k, gq, gk, cos, sin, 1e-6, q_out=qo, k_out=ko, norms=False)

    def norms():
        bs.norms(qo, ko, out=nm)

    for _ in range(warmup):
        fused(); plain(); norms()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in evs:
        e[0].record(); fused(); e[1].record(); plain(); e[2].record(); norms(); e[3].record()
    torch.cuda.synchronize()
    t_fused = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    t_plain = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    t_norms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    # algorithmic bytes: Q, K read and written once, the rotary tables and
    # weights read once, the norms written once
    qk = 2 * B * H * N * D * 2
    nbytes = 2 * qk + 2 * N * (D // 2) * 4 + 2 * D * 4 + 4 * B * H * (N + N // 16 + 2)
    gbs = nbytes / (t_fused * 1e-3) / 1e9
    print(f"[bench] attn_qk_prep {t_fused * 1e3:.1f} us with norms; {t_plain * 1e3:.1f} us without + "
          f"attn_norms {t_norms * 1e3:.1f} us", file=sys.stderr, flush=True)
    return {"fused_us": round(t_fused * 1e3, 2), "plain_us": round(t_plain * 1e3, 2),
            "attn_norms_us": round(t_norms * 1e3, 2), "unfused_us": round((t_plain + t_norms) * 1e3, 2),
            "saved_us": round((t_plain + t_norms - t_fused) * 1e3, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": load_producer_traffic(wl.name),
                         "kernel": "attn_qk_prep", "per_launch_bytes": nbytes},
            "source_hash": source_hash("attn_qk_prep")}


def time_modes(bs, wl, dev, steps: int, warmup: int, modes=(0, 1), tensors=None):
    """attn_fwd per softmax mode on one workload, each timed by events on the
    launch stream over about `steps` calls (interleaved with the other modes,
    in 4 rounds) after `warmup` each; the bound modes also time attn_norms,
    which their step includes.  Returns {mode: (fwd_ms, norms_ms)}
    and the head paths of the mode-1 call."""
    import torch
    from synth import make_qkv
    B, H, N, D = wl.batch, wl.heads, wl.seq_len, wl.head_dim
    if tensors is None:
        def up(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
        q, k, v = (up(x) for x in make_qkv(wl))
    else:
        q, k, v = tensors
    blocks = bs.build_blocks_for(wl.pattern, bs.MAX_BLOCK_Q)
    dblk = blocks.to_device(dev, B, H)
    nm = (torch.empty(B, H, N, dtype=torch.float32, device=dev),
          torch.empty(B, H, N // 16, dtype=torch.float32, device=dev),
          torch.empty(B, H, 2, dtype=torch.float32, device=dev))
    o = torch.empty(B, H, N, D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    hp = torch.zeros(B, H, dtype=torch.int32, device=dev)
    out, paths = {}, None

    def run(mode, ev=None):
        bound = mode != bs.SOFTMAX_ONLINE
        if bound:
            if ev:
                ev[0].record()
            bs.norms(q, k, out=nm)
        if ev:
            ev[1].record()
        bs.attention(q, k, v, dblk, wl.scale, mode, norms=nm if bound else None, out=o, lse=lse,
                     head_path=hp)
        if ev:
            ev[2].record()

    # The modes are timed interleaved, in rounds, so that a clock that is
    # still rising after the input upload (or falling with heat) weighs on
    # all of them alike rather than on the first.
    for mode in modes:
        for _ in range(warmup):
            run(mode)
    rounds = 4
    per = max(1, steps // rounds)
    evs = {mode: [] for mode in modes}
    torch.cuda.synchronize()
    for _ in range(rounds):
        for mode in modes:
            for _ in range(per):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                run(mode, e)
                evs[mode].append(e)
    torch.cuda.synchronize()
    if bs.SOFTMAX_BOUND in modes:
        run(bs.SOFTMAX_BOUND)
        paths = hp.cpu().tolist()
    for mode in modes:
        fwd = float(np.mean([e[1].elapsed_time(e[2]) for e in evs[mode]]))
        nms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs[mode]])) if mode != bs.SOFTMAX_ONLINE else 0.0
        out[mode] = (fwd, nms)
    return out, paths, 4.0 * D * blocks.useful_pairs * B * H


# Modes timed on a companion workload besides 0 and 1: the per-tile and the
# checked per-tile test where heads fail the per-head test on part of their
# tiles (hotframe) or on every certificate while their rows stay close to the
# bound (spread).
EXTRA_MODES = {"hotframe": (3, 5), "spread": (3, 5)}


def companions(bs, wl_main, tensors, dev, steps: int, warmup: int, others):
    """The bound-vs-online comparison on the headline workload (same run, same
    tensors) and on the other workloads: per workload, attn_fwd in mode 0 and
    mode 1, attn_norms, and the ratios mode-0 time / mode-1 time for the
    kernel alone and for the step (mode 1 with its norms pass); modes 4 (the
    headline workload) and 3 and 5 (EXTRA_MODES) with their kernel ratios
    against mode 0."""
    import torch
    from synth import WORKLOADS
    res = {}
    # the headline workload last, after the others have settled the clock
    for name in [n for n in others if n != wl_main.name] + [wl_main.name]:
        wl = WORKLOADS[name]
        main = name == wl_main.name
        modes = (0, 1, 4) if main else (0, 1) + EXTRA_MODES.get(name, ())
        t, paths, flop = time_modes(bs, wl, dev, steps, warmup, modes=modes, tensors=tensors if main else None)
        (f0, _), (f1, n1) = t[0], t[1]
        res[name] = {"mode0_fwd_ms": round(f0, 4), "mode1_fwd_ms": round(f1, 4), "mode1_norms_ms": round(n1, 4),
                     "kernel_ratio": round(f0 / f1, 4), "step_ratio": round(f0 / (f1 + n1), 4),
                     "mode1_fwd_tflops": round(flop / (f1 * 1e-3) / 1e12, 2),
                     "mode1_fwd_frac": round(flop / (f1 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "mode1_bound_heads": int(sum(sum(r) for r in paths)), "heads": wl.batch * wl.heads}
        for m in (3, 4, 5):
            # 4: the bound with Q never rounded; 3: the per-tile test; 5: the checked per-tile test
            if m in t:
                res[name][f"mode{m}_fwd_ms"] = round(t[m][0], 4)
                res[name][f"mode{m}_kernel_ratio"] = round(f0 / t[m][0], 4)
        print(f"[bench] {name}: attn_fwd mode 0 {f0:.3f} ms, mode 1 {f1:.3f} ms (+ norms {n1:.3f}); "
              f"kernel ratio {f0 / f1:.3f}, step ratio {f0 / (f1 + n1):.3f}", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    return res


def cpu_baseline(wl, q, k, v, target_s: float):
    """The fp64 oracle, timed on a bounded sample of query rows of the workload:
    a pool of one worker thread per host core, each evaluating one (head,
    512-row chunk) task at a time with its BLAS held to one thread (numpy
    releases the interpreter lock inside its array loops and BLAS calls)."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import attention as OA
    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:
        host_cores = os.cpu_count() or 1
    T = wl.pattern.tokens_per_frame
    F = wl.pattern.num_frames
    H = wl.heads
    rng = np.random.default_rng(1)

    def keys_of(row):
        f = row // T
        frames = [g for g in range(F) if -wl.pattern.win_before <= g - f <= wl.pattern.win_after
                  or g in wl.pattern.global_frames]
        return len(frames) * T

    chunk = min(512, wl.seq_len)

    def task(h, rows):
        OA.attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], wl.pattern, wl.scale, rows=rows, chunk=chunk)

    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1, user_api="blas")
        blas = 1
    except Exception:  # threadpoolctl missing: BLAS keeps its own threads
        import contextlib
        limit, blas = contextlib.nullcontext(), None
    spent, useful, rows_done, tasks = 0.0, 0.0, 0, 0
    with limit, ThreadPoolExecutor(max_workers=host_cores) as ex:
        while spent < target_s:
            batch = []
            for _ in range(host_cores):
                h = tasks % H
                rows = np.sort(rng.choice(wl.seq_len, size=chunk, replace=False))
                batch.append((h, rows))
                tasks += 1
            t0 = time.perf_counter()
            for f in [ex.submit(task, h, r) for h, r in batch]:
                f.result()
            spent += time.perf_counter() - t0
            for _, r in batch:
                rows_done += len(r)
                useful += sum(4.0 * wl.head_dim * keys_of(int(x)) for x in r)
    return {"value": useful / spent / 1e12, "unit": "TFLOP/s", "cores": int(host_cores), "kind": "oracle",
            "host_cores": int(host_cores), "blas_threads": blas, "workers": int(host_cores),
            "sample": f"{rows_done} random query rows ({tasks} tasks of {chunk} rows, heads in turn) of the "
                      f"{wl.name} workload, fp64 dense masked attention over all {wl.seq_len} keys, "
                      f"{host_cores} worker threads with one BLAS thread each, {spent:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="720p")
    ap.add_argument("--mode", type=int, default=1, help="0 online, 1 bound with per-head fallback, 2 forced bound, "
                    "3 bound per query tile, 4 as 1 with Q never rounded, 5 as 3 with the checked test")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layout", default="aligned16", choices=["aligned16", "granular128"],
                    help="block layout: frame-aligned 16-token blocks (the method), or fixed 128-token "
                         "blocks that ignore frame edges with a per-element frame mask (ablation)")
    ap.add_argument("--producer", action="store_true",
                    help="also time attn_qk_prep (QK RMS norm + rotary, norms in its epilogue) against the "
                         "same producer without norms followed by attn_norms")
    ap.add_argument("--companions", default="1080p,sr,stress,hotframe,spread",
                    help="after the headline, time modes 0 and 1 on the headline workload and on these "
                         "workloads (comma list; 'none' to skip) for the bound-vs-online ratios")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 512 MiB device copy (reference for the byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU form (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_video_frame_amd as bs
    from synth import WORKLOADS, make_qkv

    wl = WORKLOADS[args.workload]
    B, H, N, D = wl.batch, wl.heads, wl.seq_len, wl.head_dim
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload {wl.name}: B{B} H{H} N{N} D{D} mode {args.mode} layout {args.layout}", file=sys.stderr, flush=True)
    qb, kb, vb = make_qkv(wl)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(qb), up(kb), up(vb)
    t0 = time.perf_counter()
    if args.layout == "aligned16":
        blocks = bs.build_blocks_for(wl.pattern, bs.MAX_BLOCK_Q)
    else:
        blocks = bs.build_blocks_granular(wl.pattern, 128, bs.MAX_BLOCK_Q)
    setup_ms = (time.perf_counter() - t0) * 1e3
    dblk = blocks.to_device(dev, B, H)
    useful_flop = 4.0 * D * blocks.useful_pairs * B * H
    qn = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    kg = torch.empty(B, H, N // 16, dtype=torch.float32, device=dev)
    hm = torch.empty(B, H, 2, dtype=torch.float32, device=dev)
    o = torch.empty(B, H, N, D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    hp = torch.empty(B, H, dtype=torch.int32, device=dev)
    need_norms = args.mode != bs.SOFTMAX_ONLINE

    def step(ev=None):
        if need_norms:
            if ev:
                ev[0].record()
            bs.norms(q, k, out=(qn, kg, hm))
        if ev:
            ev[1].record()
        bs.attention(q, k, v, dblk, wl.scale, args.mode, norms=(qn, kg, hm) if need_norms else None,
                     out=o, lse=lse, head_path=hp)
        if ev:
            ev[2].record()

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # The companion timings run first: the GPU's clock climbs for about the
    # first 30 ms of work after the input upload (the first steps take up to
    # 20% longer), and seconds of other launches before the warm-up put the
    # timed steps at the settled clock of a job that runs continuously.
    comp = None
    if args.companions != "none" and args.layout == "aligned16":
        others = [x for x in args.companions.split(",") if x]
        comp = companions(bs, wl, (q, k, v), dev, max(5, min(args.steps, 10)), max(2, min(args.warmup, 3)),
                          others)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # Timed region: K steps, each bracketed by events on the stream the kernels
    # are launched on (torch's current stream), so the per-kernel means come
    # from the same launches as the step time.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3 / args.steps
    first = 0 if need_norms else 1
    ms_step = evs[0][first].elapsed_time(evs[-1][2]) / args.steps
    fwd = np.array([e[1].elapsed_time(e[2]) for e in evs])
    fwd_ms = float(fwd.mean())
    norms_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) if need_norms else 0.0
    paths = hp.cpu().tolist()
    print(f"[bench] step {ms_step:.3f} ms (host wall {wall_ms:.3f}), attn_fwd {fwd_ms:.3f} ms "
          f"(min {fwd.min():.3f}, max {fwd.max():.3f}), attn_norms {norms_ms:.3f} ms",
          file=sys.stderr, flush=True)

    value = useful_flop / (ms_step * 1e-3) / 1e12
    fwd_tflops = useful_flop / (fwd_ms * 1e-3) / 1e12
    norms_bytes = 2 * B * H * N * D * 2 + 4 * B * H * (N + N // 16 + 2)
    traffic = load_traffic(wl.name, args.mode) if args.layout == "aligned16" else None
    res = {
        "metric": "useful TFLOP/s (unmasked blocks) block-sparse attn fwd; % bf16 MFMA peak",
        "value": round(value, 2),
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
        "config": {"workload": f"{wl.name} chunk: B{B} H{H} D{D}, {wl.pattern.num_frames} frames x "
                               f"{wl.pattern.tokens_per_frame} tokens (N {N}), window -{wl.pattern.win_before}/"
                               f"+{wl.pattern.win_after}, global {list(wl.pattern.global_frames)}"
                               + (f", Q and K rows of frame {wl.hot_frame[0]} x{wl.hot_frame[1]:g}" if wl.hot_frame else ""),
                   "softmax_mode": args.mode, "block_q": bs.MAX_BLOCK_Q, "layout": args.layout,
                   "useful_flop": useful_flop, "useful_pairs_per_head": blocks.useful_pairs},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "attn_fwd_ms": round(fwd_ms, 4),
        "attn_fwd_ms_min": round(float(fwd.min()), 4),
        "attn_norms_ms": round(norms_ms, 4),
        "attn_norms_GBs": round(norms_bytes / (norms_ms * 1e-3) / 1e9, 1) if norms_ms else None,
        "head_paths": paths,
        "setup_ms": round(setup_ms, 3),
        "roofline": {"bound": "mfma", "achieved": round(fwd_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "attn_fwd",
                     "per_launch_flop": useful_flop},
        "source_hash": source_hash(),
    }
    if args.producer:
        res["qk_prep"] = time_producer(bs, wl, q, k, dev, args.steps, args.warmup)
    if comp is not None:
        res["bound_vs_online"] = comp[wl.name]
        res["workloads"] = {n: c for n, c in comp.items() if n != wl.name}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, qb, kb, vb, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
