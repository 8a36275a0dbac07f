"""Pins of the oracle's block-list derivation (CPU).

* closed-form counts for the five video-chunk workloads, from their definitions
  (frame pairs x tokens per frame squared; tiles per frame = T // BQ plus a tail);
* a brute-force enumeration over frames on random small patterns, written with
  plain loops and no mask array.
"""
import random

import numpy as np
import pytest

from oracle import blocks as BL
from synth import WORKLOADS, Pattern


def ceil_div(a, b):
    return -(-a // b)


# (workload, frame pairs, intervals per tile summed over frames)
# 720p / stress: 13 frames, +-1 window + frame 0 global. Frames 0, 1, 2 see one
# contiguous run (0-1, 0-2, 0-3); frames 3..12 see frame 0 plus a separate run.
# 1080p: 7 frames, same pattern: frames 0-2 one run, frames 3..6 two runs.
# tiny: 4 frames, +-1: one run each.  sr: frame-local, one run each.
CLOSED = {
    "tiny": (2 + 3 + 3 + 2, 4 * 1),
    "720p": (2 + 3 + 4 * 10 + 3, 3 * 1 + 10 * 2),
    "1080p": (2 + 3 + 4 * 4 + 3, 3 * 1 + 4 * 2),
    "stress": (2 + 3 + 4 * 10 + 3, 3 * 1 + 10 * 2),
    "sr": (5, 5),
}


@pytest.mark.parametrize("name", list(CLOSED))
@pytest.mark.parametrize("bq", [128, 256])
def test_closed_form_counts(name, bq):
    wl = WORKLOADS[name]
    p = wl.pattern
    pairs, iv_per_tile_sum = CLOSED[name]
    assert BL.frame_pairs(p) == pairs
    blk = BL.derive_blocks(p, bq)
    T = p.tokens_per_frame
    tiles_per_frame = ceil_div(T, bq)
    assert blk["n_qt"] == p.num_frames * tiles_per_frame
    assert blk["nnz"] == tiles_per_frame * iv_per_tile_sum
    assert blk["useful_pairs"] == pairs * T * T
    # every value in the list is a multiple of 16 (frame-aligned 16-token blocks)
    assert all(s % 16 == 0 and n % 16 == 0 for s, n in blk["q_tiles"])
    assert all(s % 16 == 0 and n % 16 == 0 for s, n in blk["kv_iv"])


def test_published_useful_pairs():
    # useful (query, key) pairs per head, from frame pairs x T^2
    want = {"tiny": 23_040, "720p": 622_080_000, "1080p": 1_598_054_400,
            "stress": 622_080_000, "sr": 1_036_800_000}
    for name, n in want.items():
        assert BL.derive_blocks(WORKLOADS[name].pattern, 256)["useful_pairs"] == n


def enumerate_blocks(p, bq):
    """Brute force: walk frames in order, merge adjacent attended frames."""
    T, F = p.tokens_per_frame, p.num_frames
    q_tiles, kv_ptr, kv_iv, useful = [], [0], [], 0
    for f in range(F):
        seen = []
        for g in range(F):
            if -p.win_before <= g - f <= p.win_after or g in p.global_frames:
                seen.append(g)
        runs = []
        for g in seen:
            if runs and runs[-1][1] == g:
                runs[-1][1] = g + 1
            else:
                runs.append([g, g + 1])
        r = 0
        while r < T:
            nr = min(bq, T - r)
            q_tiles.append((f * T + r, nr))
            for a, b in runs:
                kv_iv.append((a * T, (b - a) * T))
                useful += nr * (b - a) * T
            kv_ptr.append(len(kv_iv))
            r += nr
    return q_tiles, kv_ptr, kv_iv, useful


def test_random_patterns_brute_force():
    rnd = random.Random(7)
    for _ in range(60):
        F = rnd.randint(1, 9)
        T = 16 * rnd.randint(1, 12)
        p = Pattern(F, T, rnd.randint(0, 3), rnd.randint(0, 3),
                    tuple(sorted(rnd.sample(range(F), rnd.randint(0, min(2, F))))))
        bq = 16 * rnd.randint(1, 16)
        blk = BL.derive_blocks(p, bq, check_rows="all")
        qt, kp, kv, u = enumerate_blocks(p, bq)
        assert blk["q_tiles"] == qt and blk["kv_ptr"] == kp and blk["kv_iv"] == kv
        assert blk["useful_pairs"] == u


def test_alignment_assertions_fire():
    with pytest.raises(ValueError):
        BL.derive_blocks(Pattern(2, 40, 1, 1), 32)   # T not a multiple of 16
    with pytest.raises(ValueError):
        BL.derive_blocks(Pattern(2, 48, 1, 1), 24)   # block_q not a multiple of 16


def granular_by_pairs(p, granule, block_q):
    """The frame-unaware block list by plain loops over every (row, key) pair:
    tiles of block_q rows and key blocks of `granule` keys cut from token 0;
    a block is absent when no pair attends, full when every pair does, partial
    otherwise; a tile's intervals are the maximal runs of present blocks of one
    kind (full or partial), ascending."""
    T = p.tokens_per_frame
    N = p.num_frames * T

    def sees(i, j):
        d = j // T - i // T
        return -p.win_before <= d <= p.win_after or (j // T) in p.global_frames

    q_tiles, kv_ptr, kv_iv, kv_flag = [], [0], [], []
    for qs in range(0, N, block_q):
        qe = min(qs + block_q, N)
        kinds = []
        for ks in range(0, N, granule):
            ke = min(ks + granule, N)
            hit = sum(1 for i in range(qs, qe) for j in range(ks, ke) if sees(i, j))
            kinds.append((ks, ke, "none" if hit == 0 else "full" if hit == (qe - qs) * (ke - ks) else "part"))
        run = None
        for ks, ke, kind in kinds + [(N, N, "none")]:
            if run is not None and kind != run[2]:
                kv_iv.append((run[0], run[1] - run[0]))
                kv_flag.append(1 if run[2] == "part" else 0)
                run = None
            if kind != "none":
                run = [run[0], ke, kind] if run is not None else [ks, ke, kind]
        q_tiles.append((qs, qe - qs))
        kv_ptr.append(len(kv_iv))
    return q_tiles, kv_ptr, kv_iv, kv_flag


def test_granular_derivation_brute_force():
    """derive_blocks_granular against the per-pair enumeration on random small
    patterns (vatt-ghern section 把 block 縮到 16; bytechap "How it works": the
    frame-unaware layout keeps partly masked blocks and marks them).  The
    enumeration fixes coverage (no attended pair outside the runs, no block
    without an attended pair inside them) and the flags; maximality is checked
    on its own: neighbouring runs of a tile leave a gap or change flag."""
    rnd = random.Random(31)
    for _ in range(25):
        F = rnd.randint(1, 5)
        T = 16 * rnd.randint(4, 8)
        gl = tuple(sorted(set(rnd.randint(0, F - 1) for _ in range(rnd.randint(0, 2)))))
        p = Pattern(F, T, rnd.randint(0, 2), rnd.randint(0, 2), gl)
        granule = rnd.choice([64, 128])
        bq = 16 * rnd.randint(1, 10)
        qt, kp, kv, fl = granular_by_pairs(p, granule, bq)
        got = BL.derive_blocks_granular(p, granule, bq, check_rows="all")
        assert got["q_tiles"] == qt and got["kv_ptr"] == kp, p
        assert got["kv_iv"] == kv and got["kv_flag"] == fl, p
        for t in range(len(qt)):
            runs = list(zip(kv[kp[t]:kp[t + 1]], fl[kp[t]:kp[t + 1]]))
            for ((a0, l0), f0), ((a1, _), f1) in zip(runs, runs[1:]):
                assert a0 + l0 < a1 or f0 != f1
