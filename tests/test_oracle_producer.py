"""Pins of the fp64 Q/K producer oracle (RMS norm, rotary embedding, bf16
rounding, norms of the written rows) and of its synthetic inputs.

Each check ties the oracle to something other than itself: an independent
rounding routine, a library routine (torch's RMS norm, numpy's complex
product), a closed form, or an invariant of rotations.
"""
import math

import numpy as np
import pytest
import torch

from oracle import norms as NM
from oracle import producer as P
from synth import FRAME_GRID, WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, norm_weights, random_qkv, rope_tables


# ---------------------------------------------------------------- rounding

def test_round_bf16_agrees_with_the_float32_rounding_on_float32_values():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(200_000).astype(np.float32)
    x = np.concatenate([x, x * np.float32(1e-39), x * np.float32(1e30), x * np.float32(3e-45),
                        np.float32([0.0, -0.0, 3.3e38, -3.3e38, 1.17549435e-38])])
    assert np.array_equal(P.round_bf16(x.astype(np.float64)), f32_to_bf16_bits(x))


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                 # tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),    # just above a tie: up (float32 would tie)
    (-(1.0 + 2.0 ** -8), 0xBF80),
    (1.5 * 2.0 ** -133, 0x0002),               # subnormal tie -> even
    (0.5 * 2.0 ** -133, 0x0000),
    (0.75 * 2.0 ** -133, 0x0001),
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),    # largest finite
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),    # tie above it -> infinity
    (-(2 - 2.0 ** -8) * 2.0 ** 127, 0xFF80),
])
def test_round_bf16_special_values(value, bits):
    assert int(P.round_bf16(np.array([value]))[0]) == bits


def test_round_bf16_rejects_non_finite():
    with pytest.raises(ValueError):
        P.round_bf16(np.array([np.inf]))


# ---------------------------------------------------------------- RMS norm

def test_rms_normalize_matches_torch_rms_norm():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 3, 40, 64)) * 3.0
    g = rng.standard_normal(64)
    for eps in (0.0, 1e-6, 0.5):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), weight=torch.from_numpy(g),
                                           eps=float(np.float32(eps))).numpy()
        assert np.abs(P.rms_normalize(x, g, eps) - ref).max() < 1e-12


def test_rms_normalize_closed_forms():
    D = 128
    g = np.linspace(0.5, 2.0, D)
    # a constant row c: every element becomes c / sqrt(c^2 + eps) * g_e
    for c in (-3.0, 0.25, 7.0):
        eps = 1e-3
        y = P.rms_normalize(np.full((1, D), c), g, eps)
        e32 = float(np.float32(eps))
        assert np.abs(y[0] - c / math.sqrt(c * c + e32) * g).max() < 1e-14
    # eps = 0, unit weight: every row has norm sqrt(D), whatever its scale
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, D)) * np.exp(rng.standard_normal((50, 1)) * 3)
    y = P.rms_normalize(x, np.ones(D), 0.0)
    assert np.abs(np.linalg.norm(y, axis=1) - math.sqrt(D)).max() < 1e-12
    assert np.abs(P.rms_normalize(17.0 * x, np.ones(D), 0.0) - y).max() < 1e-12


# ---------------------------------------------------------------- rotation

def _angles(N, half, seed=4):
    return np.random.default_rng(seed).uniform(-50, 50, size=(N, half))


def test_rotate_pairs_is_the_complex_product():
    rng = np.random.default_rng(6)
    y = rng.standard_normal((2, 2, 30, 64))
    t = _angles(30, 32)
    z = P.rotate_pairs(y, np.cos(t), np.sin(t))
    ref = (y[..., 0::2] + 1j * y[..., 1::2]) * np.exp(1j * t)
    assert np.abs(z[..., 0::2] - ref.real).max() < 1e-12
    assert np.abs(z[..., 1::2] - ref.imag).max() < 1e-12


def test_rotate_pairs_quarter_turn_and_identity():
    y = np.arange(1.0, 9.0).reshape(1, 8)
    assert np.array_equal(P.rotate_pairs(y, np.zeros((1, 4)), np.ones((1, 4)))[0],
                          np.array([-2, 1, -4, 3, -6, 5, -8, 7], dtype=np.float64))
    assert np.array_equal(P.rotate_pairs(y, np.ones((1, 4)), np.zeros((1, 4))), y)


def test_rotate_pairs_keeps_pair_norms_and_relative_positions():
    rng = np.random.default_rng(8)
    D, N = 64, 24
    y = rng.standard_normal((N, D))
    t = _angles(N, D // 2)
    z = P.rotate_pairs(y, np.cos(t), np.sin(t))
    pn = lambda a: np.hypot(a[..., 0::2], a[..., 1::2])
    assert np.abs(pn(z) - pn(y)).max() < 1e-12
    # with angles linear in the position, <R_m q, R_n k> = <q, R_(n-m) k>
    omega = rng.uniform(0.01, 1.0, size=D // 2)
    pos = np.arange(N)[:, None] * omega[None, :]
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for m, n in ((3, 17), (20, 5), (7, 7)):
        lhs = P.rotate_pairs(q[None], np.cos(pos[m:m + 1]), np.sin(pos[m:m + 1]))[0] @ \
            P.rotate_pairs(k[None], np.cos(pos[n:n + 1]), np.sin(pos[n:n + 1]))[0]
        d = (n - m) * omega[None, :]
        rhs = q @ P.rotate_pairs(k[None], np.cos(d), np.sin(d))[0]
        assert abs(lhs - rhs) < 1e-12


# ---------------------------------------------------------------- the producer

def _small(D=64, N=96, seed=0):
    from synth import Pattern
    pat = Pattern(2, N // 2, 1, 1)
    q, k, _ = random_qkv(1, 2, N, D, seed=seed)
    gq, gk = norm_weights(D)
    cos, sin = rope_tables(pat, D, (6, N // 12))
    return q, k, gq, gk, cos, sin


def test_qk_prep_composition_and_norms():
    q, k, gq, gk, cos, sin = _small()
    eps = 1e-6
    qo, ko, qn, kg, hm = P.qk_prep(q, k, gq, gk, eps, cos, sin)
    assert qo.dtype == np.uint16 and qo.shape == q.shape
    zq = P.rotate_pairs(P.rms_normalize(q, gq, eps), cos, sin)
    assert np.array_equal(qo, P.round_bf16(zq))
    # rounding moves each value by at most half a bf16 step (2^-8 relative)
    assert np.all(np.abs(bf16_bits_to_f32(qo) - zq) <= np.abs(zq) * 2.0 ** -8)
    # the rows' norms: a rotation keeps them, so before rounding each is
    # |x * g| / sqrt(mean x^2 + eps), which is at most sqrt(D) max|g|
    x = bf16_bits_to_f32(q).astype(np.float64)
    D = x.shape[-1]
    pre = np.linalg.norm(x * gq, axis=-1) / np.sqrt((x * x).mean(axis=-1) + float(np.float32(eps)))
    assert np.abs(qn - pre).max() <= pre.max() * 2.0 ** -8
    assert qn.max() <= math.sqrt(D) * np.abs(gq).max() * (1 + 2.0 ** -8)
    kn = NM.row_norms(ko)
    assert np.array_equal(kg, kn.reshape(1, 2, -1, 16).max(axis=-1))
    assert np.array_equal(hm[..., 0], qn.max(axis=-1)) and np.array_equal(hm[..., 1], kn.max(axis=-1))


# ---------------------------------------------------------------- inputs

@pytest.mark.parametrize("name", ["tiny", "720p", "sr"])
def test_rope_tables(name):
    wl = WORKLOADS[name]
    pat, D = wl.pattern, wl.head_dim
    cos, sin = rope_tables(pat, D, FRAME_GRID[name])
    assert cos.shape == (pat.seq_len, D // 2) and cos.dtype == np.float32
    assert np.abs(cos.astype(np.float64) ** 2 + sin.astype(np.float64) ** 2 - 1).max() < 1e-6
    T, (rows, W) = pat.tokens_per_frame, FRAME_GRID[name]
    half, n_hw = D // 2, D // 2 // 3
    nt = half - 2 * n_hw
    for n in (0, T - 1, T + W + 3, pat.seq_len - 1):
        f, t = divmod(n, T)
        # the first pair of each group turns by the position itself (frequency 1)
        for col, p in ((0, f), (nt, t // W), (nt + n_hw, t % W)):
            assert abs(cos[n, col] - math.cos(p)) < 1e-7 and abs(sin[n, col] - math.sin(p)) < 1e-7
    with pytest.raises(ValueError):
        rope_tables(pat, D, (rows + 1, W))


def test_norm_weights_are_seeded_and_positive():
    a, b = norm_weights(128)
    assert a.dtype == np.float32 and a.shape == (128,) and (a > 0).all() and (b > 0).all()
    assert np.array_equal(norm_weights(128)[0], a) and not np.array_equal(a, b)
