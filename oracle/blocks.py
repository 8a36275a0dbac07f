"""Block list derived from the dense boolean frame mask.

TEST INFRASTRUCTURE (see the package header): never imported by the product.

The block granularity is 16 tokens and every block edge lies on a frame edge,
so no block is ever partly masked and no padding exists (vatt-ghern
"deep-heygen-avatar-iv-trillium-tpu", section 把 block 縮到 16; bytechap "How
it works"; cloudcurated Wall 2).  This module re-derives the block list from
the explicit mask rather than from the pattern's arithmetic, and asserts the
alignment invariants on the way.

Canonical form (both sides produce exactly this; it is the bit-exact contract):

* Query tiles, frame-major: frame f is cut into ``T // block_q`` tiles of
  ``block_q`` rows starting at ``f*T``, then one tail tile of ``T % block_q``
  rows when that is non-zero.
* For each tile, its key intervals: maximal runs of consecutive attended keys,
  in ascending order, as ``(start token, length)``.
* ``kv_ptr`` is the CSR row pointer of tiles into intervals.
* ``useful_pairs`` = number of unmasked (query, key) pairs, per head.
"""
from __future__ import annotations

import numpy as np

from .attention import frame_mask

GRANULE = 16


def derive_blocks(pattern, block_q, check_rows="ends"):
    """Block list of ``pattern`` at query tile size ``block_q`` (canonical form).

    ``check_rows="all"`` evaluates the mask for every row of every tile and
    asserts the rows are identical; ``"ends"`` (default, for full-size
    workloads) evaluates the first and last row of each tile and asserts that
    they lie in the same frame and see the same keys.  Mask rows depend on the
    query only through its frame and frames grow with the token index, so
    equal ends imply equal rows in between.
    """
    T = pattern.tokens_per_frame
    F = pattern.num_frames
    N = F * T
    if T % GRANULE or block_q % GRANULE or block_q <= 0:
        raise ValueError("tokens_per_frame and block_q must be positive multiples of 16")
    q_tiles, kv_ptr, kv_iv = [], [0], []
    useful = 0
    for f in range(F):
        starts = [(f * T + t * block_q, block_q) for t in range(T // block_q)]
        if T % block_q:
            starts.append((f * T + (T // block_q) * block_q, T % block_q))
        for qs, nr in starts:
            if check_rows == "all":
                M = frame_mask(pattern, np.arange(qs, qs + nr), N)
            else:
                M = frame_mask(pattern, np.array([qs, qs + nr - 1]), N)
                assert qs // T == (qs + nr - 1) // T, "tile crosses a frame edge"
            row = M[0]
            # every row of the tile sees the same keys: the tile never straddles a frame
            assert (M == row[None, :]).all(), "tile rows differ: tile crosses a frame edge"
            g = row.reshape(N // GRANULE, GRANULE)
            # every 16-key granule is fully attended or fully masked: no partial block
            assert (g.all(axis=1) | ~g.any(axis=1)).all(), "partially masked 16-key granule"
            if not row.any():
                raise ValueError("a query tile attends no key")
            gr = g.all(axis=1)
            j = 0
            ng = len(gr)
            while j < ng:
                if gr[j]:
                    j0 = j
                    while j < ng and gr[j]:
                        j += 1
                    kv_iv.append((j0 * GRANULE, (j - j0) * GRANULE))
                else:
                    j += 1
            q_tiles.append((qs, nr))
            kv_ptr.append(len(kv_iv))
            useful += nr * int(row.sum())
    return {
        "q_tiles": q_tiles,
        "kv_ptr": kv_ptr,
        "kv_iv": kv_iv,
        "useful_pairs": useful,
        "n_qt": len(q_tiles),
        "nnz": len(kv_iv),
    }


def derive_blocks_granular(pattern, granule, block_q, check_rows="frames"):
    """Block list of the frame-unaware layout: query tiles of ``block_q``
    consecutive rows and key blocks of ``granule`` consecutive keys over the
    whole sequence, with no regard to frame edges (the layout the pages moved
    away from; vatt-ghern section 把 block 縮到 16, bytechap "How it works").

    A key block is kept when some (row, key) pair of the tile attends it and
    is flagged partial (1) unless every pair does.  Intervals are maximal runs
    of kept blocks with equal flags, ascending.  ``useful_pairs`` is the same
    count as for the aligned layout (the mask does not change).

    ``check_rows="all"`` evaluates the dense mask for every row of a tile;
    ``"frames"`` evaluates one row per frame present in the tile (rows of one
    frame have identical mask rows by the mask's definition).
    """
    T = pattern.tokens_per_frame
    N = pattern.num_frames * T
    if granule <= 0 or granule % 64 or block_q <= 0 or block_q % 16 or T % 16:
        raise ValueError("granule must be a multiple of 64, block_q and T multiples of 16")
    q_tiles, kv_ptr, kv_iv, kv_flag = [], [0], [], []
    for qs in range(0, N, block_q):
        qe = min(qs + block_q, N)
        if check_rows == "all":
            rows = np.arange(qs, qe)
        else:
            rows = np.unique(np.clip(np.arange(qs // T, (qe - 1) // T + 1) * T, qs, qe - 1))
        M = frame_mask(pattern, rows, N)
        if not M.any():
            raise ValueError("a query tile attends no key")
        run = None  # [start, flag]
        for ks in range(0, N, granule):
            ke = min(ks + granule, N)
            sub = M[:, ks:ke]
            kind = 0 if not sub.any() else (1 if sub.all() else 2)
            if run is not None and (kind == 0 or kind != run[1]):
                kv_iv.append((run[0], ks - run[0]))
                kv_flag.append(1 if run[1] == 2 else 0)
                run = None
            if kind and run is None:
                run = [ks, kind]
        if run is not None:
            kv_iv.append((run[0], N - run[0]))
            kv_flag.append(1 if run[1] == 2 else 0)
        q_tiles.append((qs, qe - qs))
        kv_ptr.append(len(kv_iv))
    return {"q_tiles": q_tiles, "kv_ptr": kv_ptr, "kv_iv": kv_iv, "kv_flag": kv_flag,
            "n_qt": len(q_tiles), "nnz": len(kv_iv)}


def frame_pairs(pattern):
    """Number of (query frame, key frame) pairs the mask allows."""
    T = pattern.tokens_per_frame
    M = frame_mask(pattern, np.arange(pattern.num_frames) * T, pattern.num_frames * T)
    return int(M[:, ::T].sum())
