"""Pins of the CPU fp64 oracle to things other than itself (runs on CPU).

* brute force: pure-Python loops with math.fsum on the tiny workload;
* a library routine: torch's scaled_dot_product_attention (fp64, CPU) on the
  key set gathered by slicing frames, for every pattern kind (window, global
  frame, frame-local, all frames);
* closed forms: uniform softmax (LSE = ln of the attended count);
* invariants: rows of P/l sum to one, the block-by-block evaluation over the
  attended intervals equals the dense masked one (online and bound shift), the
  Cauchy-Schwarz bound is never below the true row max.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import blocks as BL
from oracle import norms as NM
from synth import WORKLOADS, Pattern, bf16_bits_to_f32, random_qkv

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def small(pattern, B=1, H=2, D=32, seed=3, stress=False):
    return random_qkv(B, H, pattern.seq_len, D, seed=seed, stress=stress)


def keys_by_slicing(pattern, f):
    """Attended key tokens of query frame f, built by slicing whole frames."""
    T = pattern.tokens_per_frame
    frames = [g for g in range(pattern.num_frames)
              if -pattern.win_before <= g - f <= pattern.win_after or g in pattern.global_frames]
    return np.concatenate([np.arange(g * T, (g + 1) * T) for g in frames])


def sdpa_reference(q, k, v, pattern, scale):
    """Per query frame, torch SDPA (fp64, CPU) on the gathered keys; LSE by torch.logsumexp."""
    qf = torch.from_numpy(bf16_bits_to_f32(q).astype(np.float64))
    kf = torch.from_numpy(bf16_bits_to_f32(k).astype(np.float64))
    vf = torch.from_numpy(bf16_bits_to_f32(v).astype(np.float64))
    B, H, N, D = qf.shape
    T = pattern.tokens_per_frame
    out = torch.empty_like(qf)
    lse = torch.empty(B, H, N, dtype=torch.float64)
    for f in range(pattern.num_frames):
        ks = torch.from_numpy(keys_by_slicing(pattern, f))
        qs = qf[:, :, f * T:(f + 1) * T]
        kk = kf[:, :, ks].contiguous()
        vv = vf[:, :, ks].contiguous()
        out[:, :, f * T:(f + 1) * T] = torch.nn.functional.scaled_dot_product_attention(qs, kk, vv, scale=scale)
        lse[:, :, f * T:(f + 1) * T] = torch.logsumexp(scale * qs @ kk.transpose(-1, -2), dim=-1)
    return out.numpy(), lse.numpy()


def test_brute_force_tiny():
    wl = WORKLOADS["tiny"]
    q, k, v = random_qkv(wl.batch, wl.heads, wl.seq_len, wl.head_dim, seed=0)
    O, L = A.attention(q, k, v, wl.pattern, wl.scale)
    Ob, Lb = A.brute_force(q, k, v, wl.pattern, wl.scale)
    assert np.abs(O - np.array(Ob)).max() <= 1e-12
    assert np.abs(L - np.array(Lb)).max() <= 1e-12


@pytest.mark.parametrize("pattern", [
    Pattern(4, 48, 1, 1),            # +-1 window (tiny)
    Pattern(6, 32, 1, 1, (0,)),      # +-1 window + global frame 0
    Pattern(5, 32, 0, 0),            # frame-local (block diagonal)
    Pattern(4, 32, 4, 4),            # every frame sees every frame: plain dense attention
    Pattern(7, 16, 2, 0, (3, 6)),    # lopsided window, two global frames
])
def test_against_sdpa(pattern):
    q, k, v = small(pattern)
    scale = 1.0 / math.sqrt(32)
    O, L = A.attention(q, k, v, pattern, scale, chunk=40)
    Or, Lr = sdpa_reference(q, k, v, pattern, scale)
    assert np.abs(O - Or).max() <= 1e-12
    assert np.abs(L - Lr).max() <= 1e-12


def test_dense_whole_sequence_is_sdpa():
    pattern = Pattern(3, 48, 2, 2)
    q, k, v = small(pattern, D=64)
    qf, kf, vf = (torch.from_numpy(bf16_bits_to_f32(x).astype(np.float64)) for x in (q, k, v))
    O, L = A.attention(q, k, v, pattern, 0.125)
    Or = torch.nn.functional.scaled_dot_product_attention(qf, kf, vf, scale=0.125).numpy()
    assert np.abs(O - Or).max() <= 1e-12


def test_uniform_softmax_closed_form():
    """Q = 0: every attended score is 0, so softmax is uniform over the attended set."""
    gold = json.load(open(os.path.join(GOLD, "uniform_lse.json")))
    wl = WORKLOADS["tiny"]
    _, k, v = random_qkv(1, 2, wl.seq_len, 64, seed=0)
    q = np.zeros_like(k)
    O, L = A.attention(q, k, v, wl.pattern, wl.scale)
    T = gold["tokens_per_frame"]
    vf = bf16_bits_to_f32(v).astype(np.float64)
    for f, (nk, lse) in enumerate(zip(gold["attended_keys_per_frame"], gold["lse_per_frame"])):
        assert np.abs(L[:, :, f * T:(f + 1) * T] - lse).max() <= 1e-12
        lo, hi = max(0, f - 1) * T, min(4, f + 2) * T
        assert hi - lo == nk
        mean = vf[:, :, lo:hi].mean(axis=2)
        assert np.abs(O[:, :, f * T:(f + 1) * T] - mean[:, :, None, :]).max() <= 1e-12


def test_identical_keys_uniform():
    """All keys equal: scores of a row are all equal, LSE = s + ln(count)."""
    pattern = Pattern(5, 32, 1, 1, (0,))
    q, k, v = small(pattern)
    k[:] = k[:, :, :1, :]
    scale = 0.25
    O, L = A.attention(q, k, v, pattern, scale)
    qf = bf16_bits_to_f32(q).astype(np.float64)
    kf = bf16_bits_to_f32(k).astype(np.float64)
    s = scale * (qf * kf[:, :, :1, :]).sum(-1)
    counts = np.array([2, 3, 4, 4, 3]).repeat(32) * 32
    assert np.abs(L - (s + np.log(counts))).max() <= 1e-12


def test_rows_sum_to_one():
    pattern = Pattern(6, 32, 1, 1, (0,))
    q, k, _ = small(pattern, stress=True)
    ones = np.ones(q.shape)
    O, _ = A.attention(q, k, ones, pattern, 0.2)
    assert np.abs(O - 1.0).max() <= 1e-12


@pytest.mark.parametrize("pattern,bq", [
    (Pattern(4, 48, 1, 1), 32),
    (Pattern(6, 80, 1, 1, (0,)), 64),
    (Pattern(5, 64, 0, 0), 48),
    (Pattern(7, 48, 2, 1, (2, 6)), 16),
])
def test_blockwise_equals_dense(pattern, bq):
    q, k, v = small(pattern)
    scale = 1.0 / math.sqrt(32)
    blk = BL.derive_blocks(pattern, bq)
    O, L = A.attention(q, k, v, pattern, scale)
    Oo, Lo = A.blockwise(q, k, v, blk, scale, "online", block_k=32)
    assert np.abs(O - Oo).max() <= 1e-12 and np.abs(L - Lo).max() <= 1e-12
    bound = NM.row_bound(q, k, pattern, scale)
    Ob, Lb = A.blockwise(q, k, v, blk, scale, "bound", bound=bound, block_k=48)
    assert np.abs(O - Ob).max() <= 1e-12 and np.abs(L - Lb).max() <= 1e-12


def test_bound_shift_equals_online_and_dominates_max():
    pattern = Pattern(6, 32, 1, 1, (0,))
    for stress in (False, True):
        q, k, v = small(pattern, D=64, stress=stress)
        scale = 0.125
        bound = NM.row_bound(q, k, pattern, scale)
        mx = A.scores_max(q, k, pattern, scale)
        assert (bound >= mx).all()
        O, L = A.attention(q, k, v, pattern, scale)
        Ob, Lb, _ = A.attention_shifted(q, k, v, pattern, scale, bound)
        ok = (bound - mx) < 600.0
        assert ok.mean() > 0.5
        assert np.abs(O - Ob)[ok].max() <= 1e-12
        assert np.abs(L - Lb)[ok].max() <= 1e-12


def test_norms_against_definition_by_loops():
    pattern = Pattern(2, 32, 0, 0)
    q, k, _ = small(pattern, D=16)
    qf = bf16_bits_to_f32(q).astype(np.float64)
    kn = NM.row_norms(k)
    qn = NM.row_norms(q)
    for b in range(1):
        for h in range(2):
            for n in range(0, 64, 7):
                assert abs(qn[b, h, n] - math.sqrt(math.fsum(x * x for x in qf[b, h, n]))) <= 1e-13
    g = NM.granule_max(kn)
    assert g.shape == (1, 2, 4)
    assert g[0, 1, 2] == max(kn[0, 1, 32:48])
    hm = NM.head_max(qn, kn)
    assert hm[0, 0, 0] == qn[0, 0].max() and hm[0, 1, 1] == kn[0, 1].max()


def test_eligibility_threshold_is_inclusive():
    hm = np.array([[[6.0, 5.0], [6.0, 5.0000001]]])
    e = NM.eligible(hm, 0.5)  # 2 * 0.5 * 6 * 5 = 30
    assert e.all()
    e = NM.eligible(hm, 1.0)  # 60 exactly, then just above 60
    assert e[0, 0] and not e[0, 1]


def test_eligibility_on_workload_heads():
    """The N(0,1) workloads sit far below 60 nats; the stress workload far above."""
    for name, want in [("tiny", True), ("stress", False)]:
        wl = WORKLOADS[name]
        if name == "stress":
            q, k, _ = random_qkv(1, 1, 3600 * 4, 128, seed=0, stress=True)
        else:
            q, k, _ = random_qkv(1, wl.heads, wl.seq_len, wl.head_dim, seed=0)
        hm = NM.head_max(NM.row_norms(q), NM.row_norms(k))
        sl = NM.slack_bound(hm, wl.scale)
        assert (NM.eligible(hm, wl.scale) == want).all(), sl
        if want:
            assert (sl < 40.0).all()
        else:
            assert (sl > 1000.0).all()


def test_tile_slack_bound_pins():
    """The per-tile slack bound: by explicit loops on a tiny case, never above the
    head-wide bound, and equal to it when one tile covers every row."""
    p = Pattern(3, 32, 1, 0)
    q, k, _ = random_qkv(1, 2, p.seq_len, 16, seed=4)
    scale = 0.25
    tiles = [(0, 32), (32, 32), (64, 32)]
    got = NM.tile_slack_bound(q, k, p, scale, tiles)
    qf, kf = A.widen(q), A.widen(k)
    for h in range(2):
        for t, (qs, nr) in enumerate(tiles):
            f = qs // 32
            key_frames = [g for g in range(3) if -1 <= g - f <= 0]
            qmax = max(math.sqrt(sum(x * x for x in qf[0, h, r])) for r in range(qs, qs + nr))
            kmax = max(math.sqrt(sum(x * x for x in kf[0, h, j])) for g in key_frames for j in range(32 * g, 32 * g + 32))
            assert abs(got[0, h, t] - 2 * scale * qmax * kmax) <= 1e-12 * got[0, h, t]
    head = NM.slack_bound(NM.head_max(NM.row_norms(q), NM.row_norms(k)), scale)
    assert (got <= head[..., None] * (1 + 1e-15)).all()
    whole = NM.tile_slack_bound(q, k, Pattern(3, 32, 2, 2), scale, [(0, 96)])
    head2 = NM.slack_bound(NM.head_max(NM.row_norms(q), NM.row_norms(k)), scale)
    assert np.allclose(whole[..., 0], head2, rtol=1e-14)


def test_hot_frame_recipe():
    """The hotframe input is the 720p input with the Q and K rows of frame 6
    doubled, exactly (a power of two in bf16), and nothing else changed; shown
    on a small pattern with the same recipe."""
    import dataclasses
    from synth import WORKLOADS, Workload, bf16_bits_to_f32, make_qkv
    hot = WORKLOADS["hotframe"]
    assert dataclasses.replace(hot, name="720p", hot_frame=()) == WORKLOADS["720p"]
    assert hot.hot_frame == (6, 2.0)
    p = Pattern(8, 48, 1, 1, (0,))
    base = Workload("small", 1, 2, 64, p)
    q0, k0, v0 = make_qkv(base)
    q1, k1, v1 = make_qkv(dataclasses.replace(base, hot_frame=(6, 2.0)))
    T = p.tokens_per_frame
    rows = slice(6 * T, 7 * T)
    for a, b in ((q0, q1), (k0, k1)):
        assert np.array_equal(bf16_bits_to_f32(b[:, :, rows]), 2.0 * bf16_bits_to_f32(a[:, :, rows]))
        assert np.array_equal(np.delete(a, np.s_[6 * T:7 * T], axis=2), np.delete(b, np.s_[6 * T:7 * T], axis=2))
    assert np.array_equal(v0, v1)


def test_row_bound_takes_only_attended_keys():
    """The row bound's key maximum runs over the keys the row attends, not over
    all keys (vatt-ghern section 拿掉 softmax 的序列相依: the shift is the query
    norm times the largest key norm the row can meet).  One key of the last
    frame is scaled 50x; rows whose frames cannot see that frame must keep a
    bound strictly below the all-keys value, and every row's bound must equal
    an explicit loop over the frames it attends."""
    p = Pattern(4, 32, 1, 0)   # frame f sees frames f-1 and f only
    q, k, _ = random_qkv(1, 2, p.seq_len, 16, seed=5)
    kf = bf16_bits_to_f32(k).astype(np.float32)
    kf[:, :, 3 * 32 + 7] *= 50.0   # a key of frame 3, seen by frame 3 only
    from synth import f32_to_bf16_bits
    k = f32_to_bf16_bits(kf)
    scale = 0.25
    got = NM.row_bound(q, k, p, scale)
    qf, kw = A.widen(q), A.widen(k)
    knorm = [[math.sqrt(math.fsum(x * x for x in kw[0, h, j])) for j in range(p.seq_len)] for h in range(2)]
    for h in range(2):
        all_max = max(knorm[h])
        for i in range(p.seq_len):
            f = i // 32
            seen = [g for g in range(4) if f - 1 <= g <= f]
            kmax = max(knorm[h][j] for g in seen for j in range(32 * g, 32 * g + 32))
            qn = math.sqrt(math.fsum(x * x for x in qf[0, h, i]))
            want = scale * qn * kmax
            assert abs(got[0, h, i] - want) <= 1e-12 * want
            if f < 3:
                # the outlier lies outside this row's frames: strictly below
                assert got[0, h, i] < 0.5 * scale * qn * all_max
            else:
                assert got[0, h, i] == pytest.approx(scale * qn * all_max, rel=1e-12)


def checked_inputs():
    """Four 32-token frames, D 16, every key close to +e0 (|k| about 1).  Query
    rows by frame: 0 aligned with e0, |q| 40 (certificate about 80 nats, every
    row's largest term near the bound); 1 aligned with |q| 60 but one row
    anti-aligned with |q| 75 (its terms all near e^-150 of the bound); 2 aligned with
    |q| 10 (certificate about 20); 3 aligned with |q| 200 (certificate about
    400)."""
    from synth import f32_to_bf16_bits
    p = Pattern(4, 32, 1, 0)
    rng = np.random.default_rng(11)
    D, N = 16, p.seq_len
    e0 = np.zeros(D, np.float32); e0[0] = 1.0
    k = (e0 + np.float32(0.1) * rng.standard_normal((1, 1, N, D), dtype=np.float32)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = (e0 + np.float32(0.05) * rng.standard_normal((1, 1, N, D), dtype=np.float32)).astype(np.float32)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    q[0, 0, 0:32] *= 40.0
    q[0, 0, 32:64] *= 60.0
    q[0, 0, 32 + 5] = -75.0 * e0
    q[0, 0, 64:96] *= 10.0
    q[0, 0, 96:128] *= 200.0
    v = rng.standard_normal((1, 1, N, D), dtype=np.float32)
    return p, f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def test_checked_tile_paths_pins():
    """The checked per-tile test against explicit loops: per row the shift (the
    query norm times the largest attended key norm, less 40 nats), l by
    math.fsum of exp(s - m), and the tile's path from its certificate and the
    smallest ln l (kept iff l >= 2^-100 in every row).  The four frames give one tile of each
    kind: checked and kept, checked and rejected by one row, certified, and
    beyond the check limit."""
    p, q, k, v = checked_inputs()
    scale = 1.0
    tiles = [(0, 32), (32, 32), (64, 32), (96, 32)]
    paths, min_ln_l = NM.checked_tile_paths(q, k, v, p, scale, tiles)
    qf, kf = A.widen(q)[0, 0], A.widen(k)[0, 0]
    norm = lambda x: math.sqrt(math.fsum(float(t) * float(t) for t in x))
    want_paths = []
    for t, (qs, nr) in enumerate(tiles):
        keys = [j for j in range(p.seq_len) if -1 <= j // 32 - t <= 0]
        kmax = max(norm(kf[j]) for j in keys)
        cert = 2 * scale * max(norm(qf[i]) for i in range(qs, qs + nr)) * kmax
        if cert <= NM.ELIGIBLE_NATS:
            want_paths.append(1)
            assert math.isnan(min_ln_l[0, 0, t])
            continue
        if cert > NM.CHECK_NATS:
            want_paths.append(0)
            assert math.isnan(min_ln_l[0, 0, t])
            continue
        lows = []
        for i in range(qs, qs + nr):
            m = scale * norm(qf[i]) * kmax - 40.0
            s = [scale * math.fsum(float(a) * float(b) for a, b in zip(qf[i], kf[j])) for j in keys]
            lows.append(math.log(math.fsum(math.exp(x - m) for x in s)))
        assert abs(min(lows) - min_ln_l[0, 0, t]) <= 1e-9 * abs(min(lows)) + 1e-12
        want_paths.append(2 if min(lows) >= -100.0 * math.log(2.0) else 0)
    assert list(paths[0, 0]) == want_paths == [2, 0, 1, 0]
    assert min_ln_l[0, 0, 0] > 30.0 and min_ln_l[0, 0, 1] < -72.0


def test_checked_tile_paths_reduce_to_the_tile_test():
    """Where every tile's certificate is within the eligibility limit the
    checked test evaluates nothing and agrees with the per-tile test."""
    p = Pattern(5, 48, 1, 1, (0,))
    q, k, v = small(p)
    tiles = [(f * 48, 48) for f in range(5)]
    cert = NM.tile_slack_bound(q, k, p, 0.125, tiles)
    assert (cert <= NM.ELIGIBLE_NATS).all()
    paths, min_ln_l = NM.checked_tile_paths(q, k, v, p, 0.125, tiles)
    assert (paths == 1).all() and np.isnan(min_ln_l).all()


def test_spread_recipe():
    """The spread input is the stress construction with sigma 0.25 and no
    outliers on the 720p shape: every Q and K row of the N(0,1) draw scaled by
    exp(0.25 z), z drawn after Q, K, V; shown on a small shape against the
    recipe written out."""
    import dataclasses
    from synth import f32_to_bf16_bits
    sp = WORKLOADS["spread"]
    assert dataclasses.replace(sp, name="720p", stress=False, stress_params=(0.75, 0.01, 8.0)) == WORKLOADS["720p"]
    assert sp.stress and sp.stress_params == (0.25, 0.0, 8.0)
    q, k, v = random_qkv(1, 2, 64, 16, seed=3, stress=True, stress_params=(0.25, 0.0, 8.0))
    rng = np.random.default_rng(3)
    draw = lambda shape: rng.standard_normal(size=shape, dtype=np.float32)
    q0, k0, v0 = draw((1, 2, 64, 16)), draw((1, 2, 64, 16)), draw((1, 2, 64, 16))
    zq, zk = draw((1, 2, 64)), draw((1, 2, 64))
    assert np.array_equal(q, f32_to_bf16_bits(q0 * np.exp(np.float32(0.25) * zq)[..., None]))
    assert np.array_equal(k, f32_to_bf16_bits(k0 * np.exp(np.float32(0.25) * zk)[..., None]))
    assert np.array_equal(v, f32_to_bf16_bits(v0))
