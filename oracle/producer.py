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
    only; results beyond the largest bf16 become +-inf."""
    x = np.asarray(x, dtype=np.float64)
    if not np.isfinite(x).all():
        raise ValueError("round_bf16 takes finite values")
    sign = np.where(np.signbit(x), np.uint16(0x8000), np.uint16(0))
    a = np.abs(x)
    _, e = np.frexp(a)                 # a = m * 2^e, m in [0.5, 1)
    # bf16 keeps 8 significant bits: quantum 2^(e-8); below the normal range
    # (a < 2^-126, e <= -126) the quantum stays 2^-133
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(a, -q)), q)   # rint: ties to even
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)     # exact below 2^128: r has <= 8 significant bits
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(r >= 2.0 ** 128, np.uint16(0x7F80), bits)
    return bits | sign


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


def qk_prep(q, k, q_gamma, k_gamma, eps, cos, sin):
    """Q and K through the producer, rounded to bf16, plus their norms.

    Returns ``(q_out bits, k_out bits, q_norm [B,H,N], k_gmax [B,H,N/16],
    head_max [B,H,2])``; the norms are fp64 over the rounded rows."""
    qo = round_bf16(qk_norm_rope(q, q_gamma, eps, cos, sin))
    ko = round_bf16(qk_norm_rope(k, k_gamma, eps, cos, sin))
    qn = _norms.row_norms(qo)
    kn = _norms.row_norms(ko)
    return qo, ko, qn, _norms.granule_max(kn), _norms.head_max(qn, kn)
