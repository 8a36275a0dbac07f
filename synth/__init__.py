"""Seeded synthetic inputs shaped like the video-chunk attention workloads.

This module only *creates inputs*: workload shapes, frame-window patterns and
seeded bf16 Q/K/V tensors. It holds none of the attention arithmetic, so both
the CPU oracle (``oracle/``) and the HIP path (``block_sparse_video_frame_amd``)
may import it without sharing any of the method's code.

Workloads (token layout is frame by frame: token ``n = f*T + t``):

=========  ======  =====  ====  ==================  ==========================
name       batch   heads  D     frames x tokens     pattern
=========  ======  =====  ====  ==================  ==========================
tiny       1       2      64    4 x 48   (N 192)    +-1 frame
720p       1       8      128   13 x 3600 (N 46800) +-1 frame + frame 0 global
1080p      1       8      128   7 x 8160 (N 57120)  +-1 frame + frame 0 global
stress     as 720p, rows scaled by log-normal(0, 0.75) norms, 1% of keys x8
spread     as 720p, rows scaled by log-normal(0, 0.25) norms, no outliers
hotframe   as 720p, the Q and K rows of frame 6 doubled
sr         1       16     64    5 x 14400 (N 72000) frame-local
=========  ======  =====  ====  ==================  ==========================

Recipe: ``numpy.random.default_rng(seed)``; draw ``standard_normal`` float32 in
the order Q, K, V, each ``[B, H, N, D]`` C-order; round float32 -> bf16 with
round-to-nearest-even on the bit pattern.  The stress workload draws the same
Q, K, V first, then ``z_q``, ``z_k`` (``[B, H, N]`` standard normal) and an
outlier uniform ``[B, H, N]``; each Q row is multiplied by ``exp(0.75 z_q)``,
each K row by ``exp(0.75 z_k)`` and, where the uniform is below 0.01, by 8;
all in float32, rounded to bf16 once at the end.  V is left unscaled.  The
spread workload is the same construction with sigma 0.25 and no outliers:
every head's norm certificate exceeds the eligibility limit, while the true
slack of its rows stays far below it.  The
hotframe workload takes the 720p Q and K and doubles every row of frame 6
(exact in bf16): per-head eligibility then fails on every head, while the
tiles whose keys avoid frame 6 stay eligible.

The Q/K producer (per-head RMS norm, then rotary embedding) takes the same
Q and K as its pre-norm input, RMS-norm weights from ``norm_weights`` and
rotary tables from ``rope_tables`` on the frame grids of ``FRAME_GRID``.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Pattern", "Workload", "WORKLOADS", "FRAME_GRID", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "make_qkv", "random_qkv", "rope_tables", "norm_weights", "sha256",
]


@dataclass(frozen=True)
class Pattern:
    """Frame-window attention pattern over a frame-major token sequence."""
    num_frames: int
    tokens_per_frame: int
    win_before: int
    win_after: int
    global_frames: tuple = field(default_factory=tuple)

    @property
    def seq_len(self) -> int:
        return self.num_frames * self.tokens_per_frame


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    pattern: Pattern
    stress: bool = False
    seed: int = 0
    stress_params: tuple = (0.75, 0.01, 8.0)   # (sigma, outlier rate, outlier scale)
    hot_frame: tuple = ()   # (frame, factor): Q and K rows of that frame scaled

    @property
    def seq_len(self) -> int:
        return self.pattern.seq_len

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(D), as the float32 value both sides use."""
        return float(np.float32(1.0) / np.sqrt(np.float32(self.head_dim)))


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, Pattern(4, 48, 1, 1)),
    "720p": Workload("720p", 1, 8, 128, Pattern(13, 3600, 1, 1, (0,))),
    "1080p": Workload("1080p", 1, 8, 128, Pattern(7, 8160, 1, 1, (0,))),
    "stress": Workload("stress", 1, 8, 128, Pattern(13, 3600, 1, 1, (0,)), stress=True),
    "sr": Workload("sr", 1, 16, 64, Pattern(5, 14400, 0, 0)),
    "hotframe": Workload("hotframe", 1, 8, 128, Pattern(13, 3600, 1, 1, (0,)), hot_frame=(6, 2.0)),
    "spread": Workload("spread", 1, 8, 128, Pattern(13, 3600, 1, 1, (0,)), stress=True,
                       stress_params=(0.25, 0.0, 8.0)),
}


# Latent grid (rows, columns) of one frame: tokens_per_frame = rows * columns,
# token t of a frame sits at row t // columns, column t % columns.
FRAME_GRID = {
    "tiny": (6, 8),
    "720p": (45, 80),
    "1080p": (68, 120),
    "stress": (45, 80),
    "sr": (90, 160),
    "hotframe": (45, 80),
    "spread": (45, 80),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits.

    NaN is kept quiet NaN; the generators never produce one.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    r = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def random_qkv(batch, heads, seq_len, head_dim, seed=0, stress=False, stress_params=(0.75, 0.01, 8.0)):
    """Seeded bf16 Q, K, V (uint16 bit arrays, ``[B, H, N, D]``).

    ``stress``: every Q and K row is scaled by exp(sigma * z), z ~ N(0, 1)
    independently per row, and a fraction ``rate`` of the K rows (independent
    uniforms) by ``scale`` more; ``stress_params = (sigma, rate, scale)``."""
    rng = np.random.default_rng(seed)
    shape = (batch, heads, seq_len, head_dim)
    q = _draw(rng, shape)
    k = _draw(rng, shape)
    v = _draw(rng, shape)
    if stress:
        sigma, rate, scale = (np.float32(x) for x in stress_params)
        rows = (batch, heads, seq_len)
        zq = _draw(rng, rows)
        zk = _draw(rng, rows)
        u = rng.random(size=rows, dtype=np.float32)
        q *= np.exp(sigma * zq)[..., None]
        ks = np.exp(sigma * zk)
        ks = np.where(u < rate, ks * scale, ks).astype(np.float32)
        k *= ks[..., None]
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def make_qkv(wl: Workload, seed: int | None = None):
    """Q, K, V bf16 bit arrays for a named workload."""
    q, k, v = random_qkv(wl.batch, wl.heads, wl.seq_len, wl.head_dim,
                         wl.seed if seed is None else seed, wl.stress, wl.stress_params)
    if wl.hot_frame:
        f, c = wl.hot_frame
        T = wl.pattern.tokens_per_frame
        q, k = (x.copy() for x in (q, k))
        for x in (q, k):
            rows = bf16_bits_to_f32(x[:, :, f * T:(f + 1) * T]) * np.float32(c)
            x[:, :, f * T:(f + 1) * T] = f32_to_bf16_bits(rows)
    return q, k, v


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def rope_tables(pattern: Pattern, head_dim: int, grid, theta: float = 10000.0):
    """Rotary angle tables ``cos, sin`` (float32 ``[N, D/2]``) for 3-D video
    positions: token ``n`` of frame ``f = n // T`` at in-frame index ``t`` has
    position ``(f, t // W, t % W)`` on a ``grid = (rows, W)`` latent grid.  The
    ``D/2`` adjacent-element pairs are split into a frame group of
    ``D/2 - 2 * (D/2 // 3)`` pairs and a row and a column group of ``D/2 // 3``
    pairs each; pair ``j`` of a group of ``n_a`` pairs turns by
    ``position * theta ** (-j / n_a)``.  Angles and their cos/sin are taken in
    float64 and stored as float32."""
    T, N = pattern.tokens_per_frame, pattern.seq_len
    rows, W = grid
    if rows * W != T:
        raise ValueError("grid must cover the frame exactly")
    half = head_dim // 2
    n_hw = half // 3
    groups = (half - 2 * n_hw, n_hw, n_hw)
    n = np.arange(N, dtype=np.int64)
    t = n % T
    pos = (n // T, t // W, t % W)
    ang = np.empty((N, half), dtype=np.float64)
    col = 0
    for p, na in zip(pos, groups):
        freq = theta ** (-np.arange(na, dtype=np.float64) / na)
        ang[:, col:col + na] = p[:, None].astype(np.float64) * freq[None, :]
        col += na
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def norm_weights(head_dim: int, seed: int = 1, sigma: float = 0.25):
    """RMS-norm weights for Q and K: float32 ``[D]`` each, ``exp(sigma * z)``
    with ``z`` standard normal from ``default_rng(seed)`` (Q's first)."""
    rng = np.random.default_rng(seed)
    gq = np.exp(np.float32(sigma) * _draw(rng, (head_dim,))).astype(np.float32)
    gk = np.exp(np.float32(sigma) * _draw(rng, (head_dim,))).astype(np.float32)
    return gq, gk
