"""GPU parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Bar: O max |err| <= 1e-2 and mean |err| <= 1e-3, LSE |err| / max(|LSE|, 1)
<= 1e-3, for both softmax variants; block lists bit-exact (CPU tests); norms
within 1e-6 relative; each mode bitwise deterministic run to run.
Full-size workloads use the launch configuration bench.py times (block_q 256,
scheduled launch order) and compare sampled rows (every tile's first and last
row plus a seeded random sample), which the oracle computes row by row.
"""
import hashlib
import math

import numpy as np
import pytest

from oracle import attention as OA
from oracle import norms as ON
from synth import WORKLOADS, Pattern, bf16_bits_to_f32, f32_to_bf16_bits, make_qkv, random_qkv

pytestmark = pytest.mark.gpu

import block_sparse_video_frame_amd as bs
from gpu_util import errors, record, run_gpu, sample_rows, within

_INPUTS = {}
_ORACLE = {}


def inputs(name):
    if name not in _INPUTS:
        _INPUTS[name] = make_qkv(WORKLOADS[name])
    return _INPUTS[name]


def oracle_rows(name, rows):
    key = (name, len(rows))
    if key not in _ORACLE:
        wl = WORKLOADS[name]
        q, k, v = inputs(name)
        _ORACLE[key] = OA.attention(q, k, v, wl.pattern, wl.scale, rows=rows)
    return _ORACLE[key]


def out_scale(name, O):
    """1, or for the spread and hotframe inputs max(1, |O_ref|) per element:
    their large-norm rows attend sharply and reach |O| of 2-4, where half an
    ulp of the bf16 output alone is 0.008 (0.016 above 4), so the absolute
    bound is scaled there, as for the other peaked inputs."""
    return np.maximum(1.0, np.abs(O)) if name in ("spread", "hotframe") else 1.0


def rows_for(name):
    wl = WORKLOADS[name]
    blk = bs.build_blocks_for(wl.pattern, 256)
    return sample_rows(blk.q_tiles, 256, wl.seq_len)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_norms(name):
    wl = WORKLOADS[name]
    q, k, v = inputs(name)
    res = run_gpu(q, k, v, wl.pattern, wl.scale, bs.SOFTMAX_BOUND)
    qn, kg, hm = res["norms"]
    qr, kr = ON.row_norms(q), ON.row_norms(k)
    assert np.abs(qn - qr).max() <= 1e-6 * qr.max()
    assert (np.abs(qn - qr) <= 1e-6 * qr + 1e-30).all()
    kgr = ON.granule_max(kr)
    assert (np.abs(kg - kgr) <= 1e-6 * kgr).all()
    hmr = ON.head_max(qr, kr)
    assert (np.abs(hm - hmr) <= 1e-6 * hmr).all()


SMALL = [
    # (pattern, B, H, D, block_q): several tiles, ragged query and key tails
    (Pattern(4, 48, 1, 1), 1, 2, 64, 256),             # tiny workload shape
    (Pattern(3, 304, 1, 1, (0,)), 1, 2, 128, 256),     # 304 = 256 + 48 rows; key runs of 608 / 912
    (Pattern(5, 80, 0, 0), 2, 3, 64, 32),              # frame-local, 80 = 2 x 32 + 16
    (Pattern(2, 16, 1, 1), 1, 1, 128, 16),             # smallest frame (one granule)
    (Pattern(1, 528, 0, 0), 1, 2, 128, 256),           # single frame, 16-row tail tile
    (Pattern(7, 112, 2, 0, (3, 6)), 1, 2, 64, 64),     # lopsided window, two globals
    (Pattern(6, 160, 1, 2, (0, 5)), 2, 2, 128, 128),   # 160 = 2.5 stages of 64 keys
    (Pattern(3, 96, 2, 2), 1, 2, 128, 64),             # window over every frame: dense attention
    (Pattern(3, 320, 1, 1), 1, 2, 64, 256),            # 64-row tail: two row groups, 10 and 15 stages
    (Pattern(4, 144, 0, 0), 1, 2, 128, 128),           # 16-row tail over 144 keys: last stage of 16
]


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4, 5])
def test_small_all_rows(case, mode):
    p, B, H, D, bq = SMALL[case]
    q, k, v = random_qkv(B, H, p.seq_len, D, seed=100 + case)
    scale = 1.0 / math.sqrt(D)
    res = run_gpu(q, k, v, p, scale, mode, block_q=bq)
    O, L = OA.attention(q, k, v, p, scale)
    e = errors(res["o"], res["lse"], O, L)
    record("small_all_rows", str(case), mode, e)
    assert within(e), e
    # every query row was written
    assert np.isfinite(res["o"]).all() and np.isfinite(res["lse"]).all()


@pytest.mark.parametrize("name", [n for n in WORKLOADS if n != "hotframe"])   # hotframe: its own test
@pytest.mark.parametrize("mode", [0, 1, 4])
def test_workload_sampled_rows(name, mode):
    wl = WORKLOADS[name]
    q, k, v = inputs(name)
    rows = rows_for(name)
    res = run_gpu(q, k, v, wl.pattern, wl.scale, mode)
    O, L = oracle_rows(name, rows)
    s = out_scale(name, O)
    e = errors(res["o"][:, :, rows] / s, res["lse"][:, :, rows], O / s, L)
    print(name, mode, e)
    record("workload_sampled_rows", name, mode, e)
    assert within(e), e
    assert np.isfinite(res["o"]).all() and np.isfinite(res["lse"]).all()


def near_limit_qkv(B, H, N, D, seed, target, heavy):
    """Seeded N(0,1) Q, K, V whose heads are scaled so that the head-wide slack
    bound 2 * scale * max|q| * max|k| is about `target` nats, just inside the
    eligibility limit: the bound path then runs with its largest logits.
    With `heavy`, 1% of the key rows are doubled first, so a few keys set
    max|k| and most rows keep a slack far above their row maximum."""
    q, k, v = random_qkv(B, H, N, D, seed=seed)
    qf = bf16_bits_to_f32(q).copy()
    kf = bf16_bits_to_f32(k).copy()
    if heavy:
        sel = np.random.default_rng(seed + 1000).random((B, H, N)) < 0.01
        kf[sel] *= np.float32(2.0)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    qn = np.sqrt((qf.astype(np.float64) ** 2).sum(-1)).max(-1)
    kn = np.sqrt((kf.astype(np.float64) ** 2).sum(-1)).max(-1)
    c = np.sqrt(target / (2.0 * scale * qn * kn)).astype(np.float32)[..., None, None]
    return f32_to_bf16_bits(qf * c), f32_to_bf16_bits(kf * c), v


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("heavy", [False, True])
@pytest.mark.parametrize("mode", [1, 3, 4, 0])
def test_near_limit_eligible_heads(D, heavy, mode):
    """Heads whose slack bound sits at 55-59 nats, just inside the 60-nat
    limit, take the bound path in modes 1 and 3 and still meet the plain
    absolute band on every row: the largest logits the bound path accepts,
    where the rounding of Q * scale * log2(e) to bf16 weighs most."""
    p = Pattern(6, 256, 1, 1, (0,))
    B, H = 1, 4
    q, k, v = near_limit_qkv(B, H, p.seq_len, D, seed=40 + D + heavy, target=57.0, heavy=heavy)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    sl = ON.slack_bound(ON.head_max(ON.row_norms(q), ON.row_norms(k)), scale)
    assert ((sl >= 55.0) & (sl <= 59.0)).all(), sl
    res = run_gpu(q, k, v, p, scale, mode)
    O, L = OA.attention(q, k, v, p, scale)
    e = errors(res["o"], res["lse"], O, L)
    print(D, heavy, mode, e)
    record("near_limit", f"D{D}{'_heavy' if heavy else ''}", mode, e)
    assert within(e), e
    assert np.isfinite(res["o"]).all() and np.isfinite(res["lse"]).all()
    if mode in (1, 4):
        assert (res["head_path"] == bs.PATH_BOUND).all()
    if mode in (1, 3, 4):
        # every row ran on the bound: its shift is the bound times (1 + 2^-8)
        bd = ON.row_bound(q, k, p, scale)
        assert np.allclose(res["shift"], bd * (1 + 2.0 ** -8), rtol=1e-5)


def test_stress_forced_bound_underflows():
    """The bound is far too loose on the stress heads: forcing it must fail
    the band (l underflows), which is why those heads fall back to online."""
    wl = WORKLOADS["stress"]
    q, k, v = inputs("stress")
    rows = rows_for("stress")
    res = run_gpu(q, k, v, wl.pattern, wl.scale, bs.SOFTMAX_BOUND_FORCED)
    O, L = oracle_rows("stress", rows)
    e = errors(res["o"][:, :, rows], res["lse"][:, :, rows], O, L)
    print("stress forced bound", e)
    assert not within(e)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_head_path_matches_oracle_eligibility(name):
    wl = WORKLOADS[name]
    q, k, v = inputs(name)
    hm = ON.head_max(ON.row_norms(q), ON.row_norms(k))
    sl = ON.slack_bound(hm, wl.scale)
    assert (np.abs(sl - ON.ELIGIBLE_NATS) > 1e-3 * ON.ELIGIBLE_NATS).all()
    want = ON.eligible(hm, wl.scale).astype(np.int32)
    for mode, expect in [(0, np.zeros_like(want)), (1, want), (2, np.ones_like(want)), (4, want)]:
        res = run_gpu(q, k, v, wl.pattern, wl.scale, mode)
        assert (res["head_path"] == expect).all(), (mode, res["head_path"], expect)


@pytest.mark.parametrize("name", ["tiny", "720p", "sr"])
@pytest.mark.parametrize("mode", [1, 4])
def test_bound_never_below_row_max(name, mode):
    wl = WORKLOADS[name]
    q, k, v = inputs(name)
    rows = rows_for(name)
    res = run_gpu(q, k, v, wl.pattern, wl.scale, mode)
    mx = OA.scores_max(q, k, wl.pattern, wl.scale, rows=rows)
    shift = res["shift"][:, :, rows]
    assert (shift >= mx).all()
    # and it is the oracle's per-row bound times the kernel's documented
    # safety factor (1 + 2^-8), up to fp32 rounding
    bd = ON.row_bound(q, k, wl.pattern, wl.scale, rows=rows)
    assert (np.abs(shift - bd * (1 + 2.0 ** -8)) <= 1e-5 * np.maximum(bd, 1.0)).all()


@pytest.mark.parametrize("mode", [0, 1, 4])
def test_bitwise_deterministic(mode):
    wl = WORKLOADS["720p"]
    q, k, v = inputs("720p")
    a = run_gpu(q, k, v, wl.pattern, wl.scale, mode)
    b = run_gpu(q, k, v, wl.pattern, wl.scale, mode, repeat=2)
    ha = hashlib.sha256(a["o_bytes"] + a["lse_bytes"]).hexdigest()
    hb = hashlib.sha256(b["o_bytes"] + b["lse_bytes"]).hexdigest()
    assert ha == hb


def test_online_and_bound_agree():
    wl = WORKLOADS["720p"]
    q, k, v = inputs("720p")
    a = run_gpu(q, k, v, wl.pattern, wl.scale, 0)
    b = run_gpu(q, k, v, wl.pattern, wl.scale, 1)
    e = errors(a["o"], a["lse"], b["o"], b["lse"])
    print("online vs bound", e)
    assert within(e), e


@pytest.mark.parametrize("name", ["1080p", "720p", "hotframe"])
def test_launch_order_does_not_change_results(name):
    """The persistent launch (items taken dynamically from per-die queues),
    the static launch in the same order and the natural order give the same
    bits."""
    wl = WORKLOADS[name]
    q, k, v = inputs(name)
    for mode in (0, 1, 3):
        a = run_gpu(q, k, v, wl.pattern, wl.scale, mode, schedule=True)
        b = run_gpu(q, k, v, wl.pattern, wl.scale, mode, schedule=True, persistent=False)
        c = run_gpu(q, k, v, wl.pattern, wl.scale, mode, schedule=False)
        assert a["o_bytes"] == b["o_bytes"] == c["o_bytes"]
        assert a["lse_bytes"] == b["lse_bytes"] == c["lse_bytes"]
        assert (a["head_path"] == b["head_path"]).all() and (a["head_path"] == c["head_path"]).all()


@pytest.mark.parametrize("mode", [0, 1])
def test_strided_bnhd_layout(mode):
    p = Pattern(5, 96, 1, 1, (0,))
    q, k, v = random_qkv(2, 3, p.seq_len, 128, seed=7)
    a = run_gpu(q, k, v, p, 1 / math.sqrt(128), mode, layout="bnhd")
    O, L = OA.attention(q, k, v, p, 1 / math.sqrt(128))
    e = errors(a["o"], a["lse"], O, L)
    assert within(e), e


def test_errors_with_device_tensors():
    import torch
    p = Pattern(2, 32, 1, 1)
    q, k, v = (torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    blk = bs.build_blocks_for(p, 32).to_device(torch.device("cuda"), 1, 1)
    # the binding refuses tensors that do not match the block list or each other
    with pytest.raises(ValueError, match="tokens"):
        bs.attention(q[:, :, :48], k[:, :, :48], v[:, :, :48], blk, 0.125, 0)
    with pytest.raises(ValueError, match="shape"):
        bs.attention(q, k[:, :, :48], v, blk, 0.125, 0)
    bad = torch.zeros(1, 1, 64, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bs.AttnError) as e:
        bs.attention(bad, bad, bad, blk, 0.125, 0)
    assert e.value.status == 5


# ---- frame-unaware layout: fixed blocks with a per-element frame mask ---------------------

GRANULAR = [c for c in range(len(SMALL)) if SMALL[c][0].tokens_per_frame >= 64]


@pytest.mark.parametrize("case", GRANULAR)
@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("granule,bq", [(128, 256), (64, 128)])
def test_granular_small_all_rows(case, mode, granule, bq):
    p, B, H, D, _ = SMALL[case]
    q, k, v = random_qkv(B, H, p.seq_len, D, seed=200 + case)
    scale = 1.0 / math.sqrt(D)
    res = run_gpu(q, k, v, p, scale, mode, block_q=bq, granule=granule)
    O, L = OA.attention(q, k, v, p, scale)
    e = errors(res["o"], res["lse"], O, L)
    assert within(e), e
    assert np.isfinite(res["o"]).all() and np.isfinite(res["lse"]).all()


@pytest.mark.parametrize("name", ["720p", "sr"])
@pytest.mark.parametrize("mode", [0, 1])
def test_granular_workload_sampled_rows(name, mode):
    wl = WORKLOADS[name]
    q, k, v = inputs(name)
    rows = rows_for(name)
    res = run_gpu(q, k, v, wl.pattern, wl.scale, mode, granule=128)
    O, L = oracle_rows(name, rows)
    e = errors(res["o"][:, :, rows], res["lse"][:, :, rows], O, L)
    print(name, mode, e)
    assert within(e), e
    assert np.isfinite(res["o"]).all() and np.isfinite(res["lse"]).all()


def test_granular_agrees_with_aligned():
    """Both layouts compute the same attention: outputs within the band of each
    other, and the same head paths."""
    p, B, H, D, _ = SMALL[6]
    q, k, v = random_qkv(B, H, p.seq_len, D, seed=77)
    scale = 1.0 / math.sqrt(D)
    a = run_gpu(q, k, v, p, scale, 1)
    g = run_gpu(q, k, v, p, scale, 1, granule=128)
    e = errors(g["o"], g["lse"], a["o"], a["lse"])
    assert within(e), e
    assert (a["head_path"] == g["head_path"]).all()


# ---- per-tile eligibility (mode 3) --------------------------------------------------------


def _frame_scaled_inputs(p, B, H, D, frame, factor, seed):
    """N(0,1) bf16 inputs whose Q and K rows in one frame are scaled by
    `factor` (rounded to bf16 once): heads that are ineligible as a whole,
    with benign tiles away from that frame."""
    from synth import f32_to_bf16_bits
    q, k, v = random_qkv(B, H, p.seq_len, D, seed=seed)
    T = p.tokens_per_frame
    out = []
    for x in (q, k):
        f = OA.widen(x).astype(np.float32)
        f[:, :, frame * T:(frame + 1) * T] *= np.float32(factor)
        out.append(f32_to_bf16_bits(f))
    return out[0], out[1], v


def test_tile_eligibility_keeps_the_bound_on_benign_tiles():
    p = Pattern(6, 160, 1, 1)
    B, H, D = 1, 2, 128
    q, k, v = _frame_scaled_inputs(p, B, H, D, frame=4, factor=3.0, seed=31)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    O, L = OA.attention(q, k, v, p, scale)
    head = ON.slack_bound(ON.head_max(ON.row_norms(q), ON.row_norms(k)), scale)
    assert (head > ON.ELIGIBLE_NATS).all()                      # mode 1: every head online
    r1 = run_gpu(q, k, v, p, scale, bs.SOFTMAX_BOUND)
    assert (r1["head_path"] == bs.PATH_ONLINE).all()
    r3 = run_gpu(q, k, v, p, scale, bs.SOFTMAX_BOUND_TILE)
    # Frame 4's rows attend sharply, so |O| reaches about 3 there; bf16's
    # half-ulp alone is then ~0.008.  The absolute bound of the workloads
    # (whose |O| stays below 1) is scaled by max(1, |O_ref|) per element.
    s = np.maximum(1.0, np.abs(O))
    for r in (r1, r3):
        e = errors(r["o"] / s, r["lse"], O / s, L)
        assert within(e), e
    blk = bs.build_blocks_for(p, 256)
    tiles = [tuple(map(int, t)) for t in blk.q_tiles]
    tb = ON.tile_slack_bound(q, k, p, scale, tiles)
    elig = tb <= ON.ELIGIBLE_NATS
    # keep a margin from the threshold so fp32 and fp64 agree on every decision
    assert (np.abs(tb - ON.ELIGIBLE_NATS) > 1e-3 * ON.ELIGIBLE_NATS).all()
    assert elig.any() and (~elig).any()
    mx = OA.scores_max(q, k, p, scale)
    bd = ON.row_bound(q, k, p, scale)
    for t, (qs, nr) in enumerate(tiles):
        sl = slice(qs, qs + nr)
        for b in range(B):
            for h in range(H):
                shift = r3["shift"][b, h, sl]
                if elig[b, h, t]:   # bound: the tile's fixed Cauchy-Schwarz shift
                    assert (shift >= mx[b, h, sl]).all()
                    assert (np.abs(shift - bd[b, h, sl] * (1 + 2.0 ** -8)) <= 1e-5 * np.maximum(bd[b, h, sl], 1)).all()
                else:               # online: the running max ends at the row max
                    assert (np.abs(shift - mx[b, h, sl]) <= 1e-3 * np.maximum(np.abs(mx[b, h, sl]), 1)).all()


@pytest.mark.parametrize("name", ["720p", "stress"])
def test_tile_eligibility_workloads(name):
    wl = WORKLOADS[name]
    q, k, v = inputs(name)
    rows = rows_for(name)
    res = run_gpu(q, k, v, wl.pattern, wl.scale, bs.SOFTMAX_BOUND_TILE)
    O, L = oracle_rows(name, rows)
    e = errors(res["o"][:, :, rows], res["lse"][:, :, rows], O, L)
    assert within(e), e


@pytest.mark.parametrize("mode", [0, 1, 3])
def test_hot_frame_workload(mode):
    """The 720p chunk with frame 6's Q and K rows doubled.  Every head fails
    the per-head test, so mode 1 runs online; the per-tile test keeps the
    bound on the tiles whose rows and keys avoid frame 6.  Sampled rows
    against the oracle; rows there attend sharply (|O| up to about 4), so the
    absolute bound is scaled by max(1, |O_ref|) per element, as for the
    frame-scaled inputs above."""
    name = "hotframe"
    wl = WORKLOADS[name]
    p = wl.pattern
    q, k, v = inputs(name)
    rows = rows_for(name)
    res = run_gpu(q, k, v, p, wl.scale, mode)
    O, L = oracle_rows(name, rows)
    s = np.maximum(1.0, np.abs(O))
    e = errors(res["o"][:, :, rows] / s, res["lse"][:, :, rows], O / s, L)
    print(name, mode, e)
    record("hot_frame_scaled", name, mode, e)
    record("hot_frame_plain", name, mode, errors(res["o"][:, :, rows], res["lse"][:, :, rows], O, L))
    assert within(e), e
    assert np.isfinite(res["o"]).all() and np.isfinite(res["lse"]).all()
    head = ON.slack_bound(ON.head_max(ON.row_norms(q), ON.row_norms(k)), wl.scale)
    assert (head > ON.ELIGIBLE_NATS).all()
    if mode == 1:
        assert (res["head_path"] == bs.PATH_ONLINE).all()
    if mode == 3:
        blk = bs.build_blocks_for(p, 256)
        tiles = [tuple(map(int, t)) for t in blk.q_tiles]
        tb = ON.tile_slack_bound(q, k, p, wl.scale, tiles)
        elig = tb <= ON.ELIGIBLE_NATS
        # the norms agree with fp64 to 1e-6 relative (test_norms), so the
        # kernel's fp32 test agrees with this one away from 1e-5 of the limit
        # (the closest tile here is 4e-4 relative away)
        assert (np.abs(tb - ON.ELIGIBLE_NATS) > 1e-5 * ON.ELIGIBLE_NATS).all()
        assert 0.6 < elig.mean() < 0.9, elig.mean()
        # A bound tile's rows carry the shift bound * (1 + 2^-8); an online
        # tile's rows end at their row max, which never exceeds the bound.
        bd = ON.row_bound(q, k, p, wl.scale, rows=rows)
        tile_of = np.searchsorted(blk.q_tiles[:, 0], rows, side="right") - 1
        shift = res["shift"][:, :, rows]
        on_bound = shift > bd * (1 + 2.0 ** -9)
        assert (on_bound == elig[:, :, tile_of]).all()
        b_ = elig[:, :, tile_of]
        assert (np.abs(shift - bd * (1 + 2.0 ** -8))[b_] <= 1e-5 * np.maximum(bd[b_], 1)).all()


def _mixed_head_inputs():
    """Four heads of N(0,1) bf16 inputs; heads 1 and 3 have every Q and K row
    doubled (exact in bf16), which fails the per-head test."""
    from synth import bf16_bits_to_f32, f32_to_bf16_bits
    p = Pattern(5, 304, 1, 1, (0,))
    B, H, D = 1, 4, 128
    q, k, v = random_qkv(B, H, p.seq_len, D, seed=41)
    q, k = q.copy(), k.copy()
    for x in (q, k):
        x[:, 1::2] = f32_to_bf16_bits(bf16_bits_to_f32(x[:, 1::2]) * np.float32(2.0))
    return p, D, q, k, v


def test_mixed_head_paths_in_one_call():
    """Mode 1 with heads on both paths in one call: each head takes the path
    the oracle's per-head test gives, the results match the oracle, and the
    persistent launch (both paths from one queue) gives the bits of the
    static launches (one per path)."""
    p, D, q, k, v = _mixed_head_inputs()
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    hm = ON.head_max(ON.row_norms(q), ON.row_norms(k))
    sl = ON.slack_bound(hm, scale)
    assert (np.abs(sl - ON.ELIGIBLE_NATS) > 1e-3 * ON.ELIGIBLE_NATS).all()
    want = ON.eligible(hm, scale).astype(np.int32)
    assert (want == np.array([[1, 0, 1, 0]])).all()
    O, L = OA.attention(q, k, v, p, scale)
    # the doubled heads attend sharply (|O| above 1): band scaled by max(1, |O_ref|)
    s = np.maximum(1.0, np.abs(O))
    a = run_gpu(q, k, v, p, scale, bs.SOFTMAX_BOUND)
    b = run_gpu(q, k, v, p, scale, bs.SOFTMAX_BOUND, persistent=False)
    for r in (a, b):
        assert (r["head_path"] == want).all(), r["head_path"]
        e = errors(r["o"] / s, r["lse"], O / s, L)
        assert within(e), e
    assert a["o_bytes"] == b["o_bytes"] and a["lse_bytes"] == b["lse_bytes"]


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_uniform_attention_closed_form(mode):
    """Q = 0 makes every attended score 0: O is the mean of V over the
    attended keys and LSE = ln(attended keys), the closed forms stored in
    tests/golden/uniform_lse.json for the tiny pattern."""
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "uniform_lse.json")))
    wl = WORKLOADS["tiny"]
    p = wl.pattern
    q, k, v = random_qkv(1, 2, p.seq_len, wl.head_dim, seed=7)
    q = np.zeros_like(q)
    res = run_gpu(q, k, v, p, wl.scale, mode)
    T = p.tokens_per_frame
    vf = np.asarray(v, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    vf = vf.view(np.float32).astype(np.float64)
    for f in range(p.num_frames):
        rows = slice(f * T, (f + 1) * T)
        lse_want = gold["lse_per_frame"][f]
        assert np.abs(res["lse"][:, :, rows] - lse_want).max() <= 1e-3 * lse_want
        keys = [g for g in range(p.num_frames) if -p.win_before <= g - f <= p.win_after]
        assert len(keys) * T == gold["attended_keys_per_frame"][f]
        mean = np.concatenate([vf[:, :, g * T:(g + 1) * T] for g in keys], axis=2).mean(axis=2)
        err = np.abs(res["o"][:, :, rows] - mean[:, :, None, :])
        assert err.max() <= 1e-2 and err.mean() <= 1e-3



# ---- seeded random patterns ---------------------------------------------------------------


def _random_case(i):
    """Pattern, shape and tile size of random case i (seeded): frame counts,
    frame sizes, windows, global frames and tile sizes the fixed cases do not
    pin down, including short tiles of 16-64 rows over long key runs."""
    rng = np.random.default_rng(5000 + i)
    F = int(rng.integers(1, 7))
    T = 16 * int(rng.integers(1, 26))
    before, after = (int(x) for x in rng.integers(0, 4, size=2))
    g = tuple(sorted(set(int(x) for x in rng.integers(0, F, size=int(rng.integers(0, 3))))))
    D = int(rng.choice([64, 128]))
    bq = 16 * int(rng.integers(1, 17))
    H = int(rng.integers(1, 4))
    return Pattern(F, T, before, after, g), 1, H, D, bq


@pytest.mark.parametrize("stages", list(range(2, 13)))
def test_d64_walk_every_stage_count(stages):
    """At D = 64 the walk runs its steps in groups of four, each with its
    buffer offsets fixed at compile time, then the rest two by two.  One
    frame of 64 * stages - 48 tokens attended frame-locally gives 256-row
    tiles (and the last, shorter tile) 2 to 12 stages of keys, the last one
    16 keys: every count of leftover steps after the groups of four.  All rows
    against the oracle in modes 0 and 1; the persistent and the static launch
    give the same bits."""
    T = 64 * stages - 48
    p = Pattern(1, T, 0, 0)
    q, k, v = random_qkv(1, 2, T, 64, seed=7000 + stages)
    scale = 0.125
    O, L = OA.attention(q, k, v, p, scale)
    for mode in (bs.SOFTMAX_ONLINE, bs.SOFTMAX_BOUND):
        a = run_gpu(q, k, v, p, scale, mode)
        b = run_gpu(q, k, v, p, scale, mode, persistent=False)
        e = errors(a["o"], a["lse"], O, L)
        record("d64_walk_every_stage_count", str(stages), mode, e)
        assert within(e), (stages, mode, e)
        assert a["o_bytes"] == b["o_bytes"] and a["lse_bytes"] == b["lse_bytes"], (stages, mode)


@pytest.mark.parametrize("case", range(24))
def test_random_patterns_all_rows(case):
    p, B, H, D, bq = _random_case(case)
    q, k, v = random_qkv(B, H, p.seq_len, D, seed=6000 + case)
    scale = 1.0 / math.sqrt(D)
    O, L = OA.attention(q, k, v, p, scale)
    persistent = case % 3 != 2   # every third case takes the static launch
    for mode in (0, 1, 3):
        res = run_gpu(q, k, v, p, scale, mode, block_q=bq, persistent=persistent)
        e = errors(res["o"], res["lse"], O, L)
        assert within(e), (p, D, bq, mode, e)
        if p.tokens_per_frame >= 64:
            res = run_gpu(q, k, v, p, scale, mode, block_q=bq, granule=64 * (1 + case % 2), persistent=persistent)
            e = errors(res["o"], res["lse"], O, L)
            assert within(e), (p, D, bq, mode, "granular", e)


@pytest.mark.parametrize("mode", [bs.SOFTMAX_BOUND, bs.SOFTMAX_ONLINE])
@pytest.mark.parametrize("num_xcd,group", [(1, 0), (3, 0), (16, 0), (8, 32)])
def test_persistent_launch_any_queue_layout(num_xcd, group, mode):
    """The persistent launch (both paths, or the online path alone) takes its
    die's queue modulo the queue count, so any num_xcd (and the group-dealt
    order) gives the natural order's bits; two calls in a row check that each
    call leaves the counters at zero."""
    import torch
    p, B, H, D = Pattern(5, 304, 1, 1, (0,)), 1, 3, 128
    q, k, v = random_qkv(B, H, p.seq_len, D, seed=11)
    scale = 1.0 / math.sqrt(D)
    ref = run_gpu(q, k, v, p, scale, mode, schedule=False)
    from gpu_util import to_device
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    blk = bs.build_blocks_for(p, 256).to_device(torch.device("cuda"), B, H, group=group, num_xcd=num_xcd)
    assert blk.work_ctr is not None and blk.work_ctr.numel() == num_xcd + 1
    nm = bs.norms(qd, kd)
    for _ in range(2):
        o, lse = bs.attention(qd, kd, vd, blk, scale, mode, norms=nm if mode != bs.SOFTMAX_ONLINE else None)
        torch.cuda.synchronize()
        assert o.contiguous().view(torch.int16).cpu().numpy().tobytes() == ref["o_bytes"]
        assert lse.cpu().numpy().tobytes() == ref["lse_bytes"]
        assert not blk.work_ctr.cpu().numpy().any()


@pytest.mark.parametrize("D", [128, 64])
def test_per_head_mode_runs_one_kernel(D):
    """Mode 1's persistent launch is two kernels, the combined one and the
    online-only one, of which exactly one takes items, chosen on the device
    from the head norms: with every head beyond the per-head limit (Q scaled
    up) the bits equal mode 0's and every head reports the online path; with
    every head within it they equal the static launch's.  Two calls each, and
    the slot counters are zero after every call."""
    import torch
    from gpu_util import to_device
    p, B, H = Pattern(5, 304, 1, 1, (0,)), 1, 3
    scale = 1.0 / math.sqrt(D)
    q0, k, v = random_qkv(B, H, p.seq_len, D, seed=13)
    for qmul, want_path in ((8.0, 0), (1.0, 1)):
        q = f32_to_bf16_bits(bf16_bits_to_f32(q0) * np.float32(qmul))
        hm = ON.head_max(ON.row_norms(q), ON.row_norms(k))
        sl = ON.slack_bound(hm, scale)
        assert (sl > ON.ELIGIBLE_NATS).all() if want_path == 0 else (sl < bs.PRESCALE_NATS).all(), sl
        ref = run_gpu(q, k, v, p, scale, bs.SOFTMAX_ONLINE if want_path == 0 else bs.SOFTMAX_BOUND,
                      persistent=want_path == 0)
        qd, kd, vd = to_device(q), to_device(k), to_device(v)
        blk = bs.build_blocks_for(p, 256).to_device(torch.device("cuda"), B, H)
        assert blk.work_ctr is not None
        nm = bs.norms(qd, kd)
        for _ in range(2):
            hp = torch.full((B, H), -1, dtype=torch.int32, device="cuda")
            o, lse = bs.attention(qd, kd, vd, blk, scale, bs.SOFTMAX_BOUND, norms=nm, head_path=hp)
            torch.cuda.synchronize()
            assert o.contiguous().view(torch.int16).cpu().numpy().tobytes() == ref["o_bytes"]
            assert lse.cpu().numpy().tobytes() == ref["lse_bytes"]
            assert (hp.cpu().numpy() == want_path).all()
            assert not blk.work_ctr.cpu().numpy().any()


def _checked_inputs(D):
    """N(0,1) draws with every Q row scaled by exp(0.35 z) and every key
    shifted by 3 along the first axis; frame 3's query rows point against that
    axis (|q| about 98 at D 128, 90 at D 64, plus noise of 0.3); frame 5's Q
    rows are quadrupled.  Certificates then span 30 to 400 nats: tiles within
    the limit, checked tiles that keep the shift (the spread rows), checked
    tiles that fail it (frame 3: every score lies about 120 nats below the
    bound) and tiles beyond the check limit (frame 5)."""
    p = Pattern(6, 272, 1, 1, (0,))   # 256 + 16 rows per frame: full and thin tiles
    q, k, v = random_qkv(1, 2, p.seq_len, D, seed=41)
    T = p.tokens_per_frame
    qf, kf = OA.widen(q).astype(np.float32), OA.widen(k).astype(np.float32)
    rng = np.random.default_rng(42)
    qf *= np.exp(np.float32(0.35) * rng.standard_normal((1, 2, p.seq_len, 1), dtype=np.float32))
    kf[..., 0] += np.float32(3.0)
    qf[:, :, 3 * T:4 * T] = np.float32(0.3) * rng.standard_normal((1, 2, T, D), dtype=np.float32)
    qf[:, :, 3 * T:4 * T, 0] = np.float32(-98.0 if D == 128 else -90.0)
    qf[:, :, 5 * T:6 * T] *= np.float32(4.0)
    return p, f32_to_bf16_bits(qf), f32_to_bf16_bits(kf), v


@pytest.mark.parametrize("D", [128, 64])
def test_checked_tiles(D):
    """Softmax mode 5 against the oracle's checked per-tile test: all rows
    within the band; per tile, the shift the kernel used is the bound (tiles
    the certificate keeps), the bound less 40 nats (tiles the check keeps) or
    the row max (tiles beyond the check limit, and checked tiles some row of
    which has l < 2^-100 under the lowered shift, which run again); bitwise
    the same run to run and in the static launch."""
    p, q, k, v = _checked_inputs(D)
    B, H = q.shape[:2]
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    res = run_gpu(q, k, v, p, scale, bs.SOFTMAX_BOUND_CHECKED, repeat=2)
    O, L = OA.attention(q, k, v, p, scale)
    # frames 3 and 5 attend sharply (|O| up to about 3): the absolute bound
    # is scaled by max(1, |O_ref|) per element, as for the per-tile test
    s = np.maximum(1.0, np.abs(O))
    e = errors(res["o"] / s, res["lse"], O / s, L)
    record("checked_tiles", f"D{D}", 5, e)
    assert within(e), e
    blk = bs.build_blocks_for(p, 256)
    tiles = [tuple(map(int, t)) for t in blk.q_tiles]
    paths, min_ln_l = ON.checked_tile_paths(q, k, v, p, scale, tiles)
    cert = ON.tile_slack_bound(q, k, p, scale, tiles)
    # every kind of tile occurs, and no decision sits near a threshold
    assert {0, 1, 2} <= set(paths.ravel().tolist())
    assert ((paths == 0) & ~np.isnan(min_ln_l)).any()              # checked, then run again
    assert ((paths == 0) & np.isnan(min_ln_l)).any()               # beyond the check limit
    limit = bs.CHECK_LOG2_L * math.log(2.0)
    near = np.abs(min_ln_l - limit) < 2.0
    assert not near.any()
    # (a certificate near ELIGIBLE_NATS decides only between certified and
    # checked, and both keep the bound on these tiles)
    assert (np.abs(cert - ON.CHECK_NATS) > 2.0).all()
    mx = OA.scores_max(q, k, p, scale)
    bd = ON.row_bound(q, k, p, scale)
    for t, (qs, nr) in enumerate(tiles):
        sl = slice(qs, qs + nr)
        for b in range(B):
            for h in range(H):
                shift = res["shift"][b, h, sl]
                if paths[b, h, t]:
                    low = ON.CHECK_SHIFT_NATS if paths[b, h, t] == 2 else 0.0
                    want = bd[b, h, sl] * (1 + 2.0 ** -8) - low
                    assert (shift >= mx[b, h, sl] - low).all()
                    assert (np.abs(shift - want) <= 1e-5 * np.maximum(bd[b, h, sl], 1)).all()
                else:
                    assert (np.abs(shift - mx[b, h, sl]) <= 1e-3 * np.maximum(np.abs(mx[b, h, sl]), 1)).all()
    want_hp = np.where(paths[:, :, 0] > 0, bs.PATH_BOUND, bs.PATH_ONLINE)
    assert np.array_equal(res["head_path"], want_hp)
    again = run_gpu(q, k, v, p, scale, bs.SOFTMAX_BOUND_CHECKED)
    static = run_gpu(q, k, v, p, scale, bs.SOFTMAX_BOUND_CHECKED, persistent=False)
    for r in (again, static):
        assert r["o_bytes"] == res["o_bytes"] and r["lse_bytes"] == res["lse_bytes"]


@pytest.mark.parametrize("name", ["spread", "stress", "720p", "hotframe"])
def test_checked_workloads(name):
    """Mode 5 at full size on sampled rows: within the band; per tile, the
    sampled rows all used the bound (times 1 + 2^-8; less 40 nats on a checked
    tile) or all the row max; tiles whose certificate passes keep the bound,
    tiles beyond the check limit take the row max, and a checked tile with a
    sampled row whose l under the lowered shift is below 2^-100 (by more than
    2 nats) was run again."""
    wl = WORKLOADS[name]
    q, k, v = inputs(name)
    rows = rows_for(name)
    res = run_gpu(q, k, v, wl.pattern, wl.scale, bs.SOFTMAX_BOUND_CHECKED)
    O, L = oracle_rows(name, rows)
    s = out_scale(name, O)
    e = errors(res["o"][:, :, rows] / s, res["lse"][:, :, rows], O / s, L)
    record("checked_workloads", name, 5, e)
    assert within(e), e
    blk = bs.build_blocks_for(wl.pattern, 256)
    tiles = [tuple(map(int, t)) for t in blk.q_tiles]
    cert = ON.tile_slack_bound(q, k, wl.pattern, wl.scale, tiles)
    bd = ON.row_bound(q, k, wl.pattern, wl.scale, rows=rows)
    mx = OA.scores_max(q, k, wl.pattern, wl.scale, rows=rows)
    ln_l = L - bd + ON.CHECK_SHIFT_NATS     # under the lowered shift of a checked tile
    limit = bs.CHECK_LOG2_L * math.log(2.0)
    kept = np.zeros(cert.shape, dtype=bool)
    tile_of = np.searchsorted(np.array([t[0] for t in tiles]), rows, side="right") - 1
    for t in range(len(tiles)):
        idx = np.nonzero(tile_of == t)[0]
        for b in range(wl.batch):
            for h in range(wl.heads):
                sh = res["shift"][b, h, rows[idx]]
                low = ON.CHECK_SHIFT_NATS if cert[b, h, t] > ON.ELIGIBLE_NATS else 0.0
                on_bound = (np.abs(sh - (bd[b, h, idx] * (1 + 2.0 ** -8) - low))
                            <= 1e-5 * np.maximum(bd[b, h, idx], 1))
                on_max = np.abs(sh - mx[b, h, idx]) <= 1e-3 * np.maximum(np.abs(mx[b, h, idx]), 1)
                assert on_bound.all() or on_max.all()
                kept[b, h, t] = on_bound.all()
                if cert[b, h, t] <= ON.ELIGIBLE_NATS - 0.5:
                    assert kept[b, h, t]
                if cert[b, h, t] > ON.CHECK_NATS + 2.0 or (ln_l[b, h, idx] < limit - 2.0).any():
                    assert not kept[b, h, t]
    print(name, "tiles on the bound:", kept.mean())
    if name == "spread":       # nearly every certificate fails, and the check keeps nearly every tile
        assert (cert > ON.ELIGIBLE_NATS).mean() > 0.99 and kept.mean() > 0.9
    if name == "stress":       # certificates far beyond the check limit
        assert not kept.any()
