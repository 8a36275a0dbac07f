"""The Q/K producer with the norms in its epilogue, in fp64.

TEST INFRASTRUCTURE (see the package header): never imported by the product.

The pages hand the attention kernel "a small set of precomputed norms"
(vatt-ghern "deep-heygen-avatar-iv-trillium-tpu", section
拿掉 softmax 的序列相依) and fuse producer stages so that one stage's output is
already in the next stage's layout (cloudcurated "How is HeyGen optimizing AI
video on Google Cloud TPUs", the explicit layout contracts after Wall 3;
bytechap "Optimizing HeyGen's Avatar IV ...", What you can do).  They name no
producer.  The reading used here is the step that writes Q and K right before
attention in a video diffusion transformer: a per-head RMS normalisation over
D with a learned weight (QK-norm), then a rotary position embedding, one
rounding to bf16 at the end; the producer also emits the norms of the rows it
wrote, so no separate pass over Q and K is needed.

Per row x (D values) of one head, with weight g (D values) and eps:

    r     = 1 / sqrt(mean_e x_e^2 + eps)
    y_e   = x_e * r * g_e
    (z_2i, z_2i+1) = (y_2i cos t_ni - y_2i+1 sin t_ni,  y_2i sin t_ni + y_2i+1 cos t_ni)
    out   = bf16(z)   (round to nearest, ties to even, straight from fp64)

Pairs are adjacent elements (2i, 2i+1): as a complex number y_2i + j y_2i+1
each pair is multiplied by exp(j t_ni).  ``cos`` and ``sin`` are per-token
tables ``[N, D/2]``: the angles t are the caller's (any 1-D or 3-D position
scheme).  The norms are those of ``attn_norms`` taken over the rounded rows.
"""
from __future__ import annotations

import numpy as np

from .attention import widen
from . import norms as _norms


def round_bf16(x) -> np.ndarray:
    """fp64 -> bf16 bit patterns (uint16), round to nearest, ties to even, in
    one step (no intermediate float32, so no double rounding).  Finite inputs
    only; results beyond the largest bf16 become +-inf.

    In the normal range the fp64 pattern is rounded to bf16's 7 stored
    fraction bits (a carry out of the fraction moves to the next binade);
    below 2^-126 bf16's quantum is fixed at 2^-133 and the value is rounded
    to a multiple of it."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    if not np.isfinite(x).all():
        raise ValueError("round_bf16 takes finite values")
    u = x.view(np.uint64)
    drop = np.uint64(45)                           # 52 - 7 fraction bits go
    lsb = (u >> drop) & np.uint64(1)
    r = ((u + np.uint64((1 << 44) - 1) + lsb) >> drop) << drop
    rv = r.view(np.float64)
    small = np.abs(x) < 2.0 ** -126
    if small.any():
        rv = np.where(small, np.rint(x * 2.0 ** 133) * 2.0 ** -133, rv)   # rint: ties to even
    big = np.abs(rv) >= 2.0 ** 128
    with np.errstate(over="ignore"):
        r32 = np.where(big, 0.0, rv).astype(np.float32)   # exact: <= 8 significant bits
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(big, np.uint16(0x7F80), bits)
    sign = np.where(np.signbit(x), np.uint16(0x8000), np.uint16(0))
    return (bits & np.uint16(0x7FFF)) | sign


def rms_normalize(x, gamma, eps):
    """``x * g / sqrt(mean(x^2) + eps)`` over the last axis, fp64."""
    x = widen(x)
    g = np.asarray(gamma, dtype=np.float64)
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(np.float32(eps))) * g


def rotate_pairs(y, cos, sin):
    """Rotary embedding of adjacent pairs by the per-token angle tables
    ``cos, sin [N, D/2]`` (broadcast over leading axes of ``y [..., N, D]``)."""
    y = np.asarray(y, dtype=np.float64)
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    a, b = y[..., 0::2], y[..., 1::2]
    z = np.empty_like(y)
    z[..., 0::2] = a * c - b * s
    z[..., 1::2] = a * s + b * c
    return z


def qk_norm_rope(x, gamma, eps, cos, sin):
    """One tensor through the producer: fp64 values before rounding, ``[B, H, N, D]``."""
    return rotate_pairs(rms_normalize(x, gamma, eps), cos, sin)


def qk_prep(q, k, q_gamma, k_gamma, eps, cos, sin, chunk=4096):
    """Q and K through the producer, rounded to bf16, plus their norms.

    Returns ``(q_out bits, k_out bits, q_norm [B,H,N], k_gmax [B,H,N/16],
    head_max [B,H,2])``; the norms are fp64 over the rounded rows.  Rows are
    independent, so they are taken ``chunk`` at a time (bounded memory)."""
    q, k = np.asarray(q), np.asarray(k)
    B, H, N, _ = q.shape
    outs = []
    for x, g in ((q, q_gamma), (k, k_gamma)):
        o = np.empty(x.shape, dtype=np.uint16)
        n = np.empty((B, H, N))
        for b in range(B):
            for h in range(H):
                for r0 in range(0, N, chunk):
                    r1 = min(N, r0 + chunk)
                    o[b, h, r0:r1] = round_bf16(qk_norm_rope(x[b, h, r0:r1], g, eps, cos[r0:r1], sin[r0:r1]))
                    n[b, h, r0:r1] = _norms.row_norms(o[b, h, r0:r1])
        outs.append((o, n))
    (qo, qn), (ko, kn) = outs
    return qo, ko, qn, _norms.granule_max(kn), _norms.head_max(qn, kn)
