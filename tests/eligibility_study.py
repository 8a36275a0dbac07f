#!/usr/bin/env python3
"""Eligibility and slack of the bound softmax across norm distributions.

CPU only (the fp64 oracle); reproduces the table in the design notes:

    python tests/eligibility_study.py [--heads 2] [--rows 256]

For the 720p shape (13 frames x 3600 tokens, window -1/+1, global frame 0,
D = 128) and seeded inputs whose rows are scaled by exp(sigma z) with a
fraction `rate` of the keys scaled by 8 more (the stress construction with
swept parameters), or whose rows in one frame are scaled by c ("local"), it
reports per setting:

* the head-wide slack bound 2 scale max|q| max|k| (nats) and the fraction of
  heads the per-head test (<= 60 nats) puts on the bound path;
* the fraction of 256-row query tiles the per-tile test puts on the bound
  path (softmax mode 3);
* the fraction of tiles the checked per-tile test keeps on the bound (softmax
  mode 5: certificate up to 60 nats, or up to 256 nats and every row's
  l >= 2^-100 under the bound shift), over every 4th tile of each head (all
  rows of those tiles);
* percentiles of the actual slack m_i - max_j s_ij (nats) of sampled rows
  under the bound shift m_i = scale |q_i| max_{j attended} |k_j|.
"""
import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import attention as OA   # noqa: E402
from oracle import blocks as BL      # noqa: E402
from oracle import norms as ON       # noqa: E402
from synth import WORKLOADS, f32_to_bf16_bits, random_qkv  # noqa: E402


def local_inputs(q, k, T, frame, c):
    out = []
    for x in (q, k):
        f = OA.widen(x).astype(np.float32)
        f[:, :, frame * T:(frame + 1) * T] *= np.float32(c)
        out.append(f32_to_bf16_bits(f))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--heads", type=int, default=2)
    ap.add_argument("--rows", type=int, default=256)
    ap.add_argument("--tile-step", type=int, default=4)
    args = ap.parse_args()
    wl = WORKLOADS["720p"]
    p, N, D, scale = wl.pattern, wl.seq_len, wl.head_dim, wl.scale
    tiles = [tuple(t) for t in BL.derive_blocks(p, 256)["q_tiles"]]
    # a tile's rows share one frame, so its keys are those of its first row
    tile_rows = [(qs, nr) for qs, nr in tiles]
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(N, size=args.rows, replace=False))
    settings = [("lognormal", s, r) for s in (0.0, 0.25, 0.5, 0.75, 1.0) for r in (0.0, 0.001, 0.01)]
    settings += [("local", c, 6) for c in (1.5, 2.0, 3.0)]
    print("| inputs | head slack bound (nats) | heads on bound | tiles on bound | tiles on bound, checked "
          "| slack p50 / p95 / p99 (nats) |")
    print("|---|---|---|---|---|---|")
    some = tile_rows[::args.tile_step]
    for kind, a, b in settings:
        if kind == "lognormal":
            q, k, _ = random_qkv(1, args.heads, N, D, seed=0, stress=(a > 0 or b > 0), stress_params=(a, b, 8.0))
            label = f"sigma {a}, {b * 100:g}% keys x8"
        else:
            q, k, _ = random_qkv(1, args.heads, N, D, seed=0)
            q, k = local_inputs(q, k, p.tokens_per_frame, b, a)
            label = f"frame {b} rows x{a}"
        hb = ON.slack_bound(ON.head_max(ON.row_norms(q), ON.row_norms(k)), scale)[0]
        tb = ON.tile_slack_bound(q, k, p, scale, tile_rows)[0]
        v = np.zeros_like(q)   # the path does not depend on V
        cp, _ = ON.checked_tile_paths(q, k, v, p, scale, some)
        mx = OA.scores_max(q, k, p, scale, rows=rows)[0]
        bd = ON.row_bound(q, k, p, scale, rows=rows)[0]
        slack = (bd - mx).ravel()
        pc = np.percentile(slack, [50, 95, 99])
        print(f"| {label} | {hb.min():.1f} – {hb.max():.1f} | {np.mean(hb <= ON.ELIGIBLE_NATS) * 100:.0f}% "
              f"| {np.mean(tb <= ON.ELIGIBLE_NATS) * 100:.0f}% | {np.mean(cp[0] > 0) * 100:.0f}% "
              f"| {pc[0]:.1f} / {pc[1]:.1f} / {pc[2]:.1f} |",
              flush=True)


if __name__ == "__main__":
    main()
