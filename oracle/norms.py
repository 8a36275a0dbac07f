"""Norms, the Cauchy-Schwarz row bound and per-head eligibility, in fp64.

TEST INFRASTRUCTURE (see the package header): never imported by the product.

Source: vatt-ghern "deep-heygen-avatar-iv-trillium-tpu", section
拿掉 softmax 的序列相依.  A logit q.k can never exceed |q| |k| (Cauchy-Schwarz),
so ``m_i = scale * |q_i| * max over attended keys |k_j|`` bounds every score of
row i before any score is computed; precomputed norms are handed to the kernel
so each row knows its bound up front.  The bound is not tight for every head:
eligibility is decided per head, and ineligible heads use the online max.

Readings where the pages leave the step open (each listed in the design notes):

* The maximum key norm is taken over all keys the row attends (one fixed
  shift per row).  A per-block maximum would change the shift from block to
  block and bring the rescaling back.
* Eligibility is a norm-only sufficient condition: since
  ``-m_i <= max_j s_ij <= m_i``, the slack ``m_i - max_j s_ij`` is at most
  ``2 m_i <= 2 * scale * max_n |q_n| * max_n |k_n|``.  A head is eligible when
  that head-wide quantity is at most 60 (nats), inclusive: then the largest
  term ``exp(s - m)`` is at least ``e^-60``, 27 nats above the smallest normal
  float32/bf16 value ``e^-87.3``.
* The checked per-tile test (``checked_tile_paths``) is a widening of that
  check, not a step the pages give: where the norm certificate fails, the
  shift is checked after the fact on the row sums it produced.
"""
from __future__ import annotations

import numpy as np

from .attention import attention, frame_mask, widen

GRANULE = 16
ELIGIBLE_NATS = 60.0
CHECK_NATS = 256.0
CHECK_LOG2_L = -100.0
CHECK_SHIFT_NATS = 40.0


def row_norms(x):
    """``|x_n|_2`` per row, fp64, ``[B, H, N]``."""
    x = widen(x)
    return np.sqrt((x * x).sum(axis=-1))


def granule_max(knorm):
    """Max key norm over each 16-key granule: ``[B, H, N] -> [B, H, N/16]``."""
    B, H, N = knorm.shape
    return knorm.reshape(B, H, N // GRANULE, GRANULE).max(axis=-1)


def head_max(qnorm, knorm):
    """``[B, H, 2]``: (max_n |q_n|, max_n |k_n|)."""
    return np.stack([qnorm.max(axis=-1), knorm.max(axis=-1)], axis=-1)


def row_bound(q, k, pattern, scale, rows=None):
    """``m_i = scale |q_i| max_{j attended by i} |k_j|`` in fp64, ``[B, H, R]``."""
    qn = row_norms(q)
    kn = row_norms(k)
    B, H, N = qn.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    M = frame_mask(pattern, rows, N)
    out = np.empty((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            kmax = np.where(M, kn[b, h][None, :], -np.inf).max(axis=1)
            out[b, h] = scale * qn[b, h, rows] * kmax
    return out


def slack_bound(hmax, scale):
    """Head-wide upper bound on the slack: ``2 scale max|q| max|k|`` (nats), ``[B, H]``."""
    return 2.0 * scale * hmax[..., 0] * hmax[..., 1]


def eligible(hmax, scale, limit=ELIGIBLE_NATS):
    """Per-head eligibility for the bound softmax, ``[B, H]`` bool (inclusive)."""
    return slack_bound(hmax, scale) <= limit


def tile_slack_bound(q, k, pattern, scale, tiles):
    """Per query tile, ``2 scale max_{rows of the tile} |q| max_{keys the tile
    attends} |k|`` (nats), ``[B, H, n_tiles]``: the head-wide slack bound
    restricted to one tile's rows and keys (finer-grained eligibility; the
    pages check the bound per head, vatt-ghern section 拿掉 softmax 的序列相依).
    ``tiles`` is a sequence of ``(first row, rows)``; a tile's keys are the keys
    any of its rows attends (read from the dense mask)."""
    qn = row_norms(q)
    kn = row_norms(k)
    B, H, N = qn.shape
    out = np.empty((B, H, len(tiles)))
    for t, (qs, nr) in enumerate(tiles):
        keys = frame_mask(pattern, np.arange(qs, qs + nr), N).any(axis=0)
        for b in range(B):
            for h in range(H):
                out[b, h, t] = 2.0 * scale * qn[b, h, qs:qs + nr].max() * kn[b, h, keys].max()
    return out


def checked_tile_paths(q, k, v, pattern, scale, tiles):
    """The checked per-tile test (softmax mode 5), per query tile: the path it
    takes and the smallest ``ln l_i`` over the tile's rows under the shift it
    tries.

    The pages certify the fixed shift from norms alone (vatt-ghern
    "deep-heygen-avatar-iv-trillium-tpu", section 拿掉 softmax 的序列相依); the
    certificate charges every row the worst case ``2 m_i``.  This test keeps
    the certificate where it is cheap and otherwise checks a shift after the
    fact, which the identity the method rests on allows (any per-row shift
    gives the same softmax as long as nothing underflows or overflows):

    * tile slack bound (``tile_slack_bound``) <= ELIGIBLE_NATS: the bound,
      certified (path 1);
    * bound in (ELIGIBLE_NATS, CHECK_NATS]: the tile is evaluated with the
      shift ``m_i - CHECK_SHIFT_NATS`` (``m_i = row_bound``: every term is then
      at most e^CHECK_SHIFT_NATS, so nothing can overflow); it keeps that
      result when every row has ``l_i = sum_j exp(s_ij - m_i + CHECK_SHIFT_NATS)``
      of at least ``2^CHECK_LOG2_L`` and finite (path 2); otherwise it is
      evaluated again with the running max (path 0);
    * beyond CHECK_NATS: running max (path 0).

    ``ln l_i`` is ``LSE_i - m_i + CHECK_SHIFT_NATS`` with the fp64 LSE of
    ``attention``.  Returns ``(paths [B, H, n_tiles] int, min_ln_l [B, H,
    n_tiles])``, the latter NaN for tiles the test does not evaluate."""
    cert = tile_slack_bound(q, k, pattern, scale, tiles)
    B, H, nt = cert.shape
    paths = np.zeros((B, H, nt), dtype=np.int64)
    min_ln_l = np.full((B, H, nt), np.nan)
    paths[cert <= ELIGIBLE_NATS] = 1
    top = np.log(np.finfo(np.float32).max)
    for t, (qs, nr) in enumerate(tiles):
        todo = (cert[:, :, t] > ELIGIBLE_NATS) & (cert[:, :, t] <= CHECK_NATS)
        if not todo.any():
            continue
        rows = np.arange(qs, qs + nr)
        _, lse = attention(q, k, v, pattern, scale, rows=rows)
        m = row_bound(q, k, pattern, scale, rows=rows) - CHECK_SHIFT_NATS
        ln_l = lse - m
        for b in range(B):
            for h in range(H):
                if todo[b, h]:
                    lo, hi = ln_l[b, h].min(), ln_l[b, h].max()
                    min_ln_l[b, h, t] = lo
                    paths[b, h, t] = 2 if lo >= CHECK_LOG2_L * np.log(2.0) and hi < top else 0
    return paths, min_ln_l
