"""GPU parity of the Q/K producer (attn_qk_prep, through the C ABI) against
the fp64 oracle, and of attention fed by it.

Bar: every output element within one bf16 step of the oracle's (the GPU
computes in fp32 and rounds once, the oracle in fp64: the two roundings can
differ next to a rounding tie); norms within 1e-6 relative of the fp64 norms
of the rows the GPU wrote, and within 2^-7 of the oracle's; head maxima
bit-equal to the maxima of the GPU's own norms; attention on the producer's
output within the attention bar against the oracle's attention on the
oracle's producer output.
"""
import numpy as np
import pytest

from oracle import attention as OA
from oracle import norms as ON
from oracle import producer as OP
from synth import FRAME_GRID, WORKLOADS, Pattern, make_qkv, norm_weights, random_qkv, rope_tables

pytestmark = pytest.mark.gpu

import block_sparse_video_frame_amd as bs
from gpu_util import bf16_to_f64, errors, sample_rows, to_device, within

EPS = 1e-6


def _bits(t):
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _order(bits):
    """bf16 bits -> integers in the order of the values (+0 and -0 both 0)."""
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _ulp_check(got_bits, want_bits):
    d = np.abs(_order(got_bits) - _order(want_bits))
    assert d.max() <= 1, f"{int((d > 1).sum())} elements more than one bf16 step away"
    return float((d == 0).mean())


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def _run(q, k, gq, gk, cos, sin, layout="bhnd", norms=True):
    import torch
    B, H, N, D = q.shape
    if layout == "bnhd_in":   # projection-style [B, N, H, D] input, attention layout out
        qd, kd = (to_device(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3) for x in (q, k))
    else:
        qd, kd = to_device(q), to_device(k)
    qo = ko = None
    if layout == "inplace":
        qo, ko = qd, kd
    elif layout == "bnhd_out":
        qo, ko = (torch.empty(B, N, H, D, dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3) for _ in range(2))
    qo, ko, nm = bs.qk_prep(qd, kd, _dev(gq), _dev(gk), _dev(cos), _dev(sin), EPS, q_out=qo, k_out=ko, norms=norms)
    torch.cuda.synchronize()
    return qo, ko, nm


def _small_case(D, B, H, F, rows, cols, seed=0):
    pat = Pattern(F, rows * cols, 1, 1)
    q, k, _ = random_qkv(B, H, pat.seq_len, D, seed=seed)
    gq, gk = norm_weights(D)
    cos, sin = rope_tables(pat, D, (rows, cols))
    return pat, q, k, gq, gk, cos, sin


def _check_norms(qo, ko, nm, want=None):
    import torch
    qn, kg, hm = (x.cpu().numpy().astype(np.float64) for x in nm)
    # against the fp64 norms of the rows the GPU wrote
    own_q = torch.linalg.vector_norm(qo.double(), dim=-1).cpu().numpy()
    own_k = torch.linalg.vector_norm(ko.double(), dim=-1).cpu().numpy()
    assert (np.abs(qn - own_q) <= 1e-6 * own_q).all()
    B, H, N = own_k.shape
    own_kg = own_k.reshape(B, H, N // 16, 16).max(axis=-1)
    assert (np.abs(kg - own_kg) <= 1e-6 * own_kg).all()
    # head maxima are maxima of the emitted norms, bit for bit
    qn32, kg32, hm32 = (x.cpu().numpy() for x in nm)
    assert np.array_equal(hm32[..., 0], qn32.max(axis=-1)) and np.array_equal(hm32[..., 1], kg32.max(axis=-1))
    if want is not None:
        wq, wkg = want
        assert (np.abs(qn - wq) <= 2.0 ** -7 * wq).all()
        assert (np.abs(kg - wkg) <= 2.0 ** -7 * wkg).all()


@pytest.mark.parametrize("D,B,H,F,rows,cols,layout", [
    (64, 1, 2, 4, 6, 8, "bhnd"),          # the tiny shape
    (128, 2, 3, 1, 16, 37, "bhnd"),       # 37 granules: a ragged last workgroup
    (128, 1, 2, 2, 8, 37, "bnhd_in"),     # strided input
    (64, 1, 3, 3, 6, 8, "bnhd_out"),      # strided output
    (128, 1, 2, 1, 12, 12, "inplace"),
    (64, 2, 1, 1, 4, 4, "bhnd"),          # a single granule per head
    (64, 1, 40, 1, 6, 8, "bhnd"),         # many heads per wave, 3 granules
])
def test_qk_prep_small(D, B, H, F, rows, cols, layout):
    pat, q, k, gq, gk, cos, sin = _small_case(D, B, H, F, rows, cols)
    wq, wk, wqn, wkg, whm = OP.qk_prep(q, k, gq, gk, EPS, cos, sin)
    qo, ko, nm = _run(q, k, gq, gk, cos, sin, layout)
    fq = _ulp_check(_bits(qo), wq)
    fk = _ulp_check(_bits(ko), wk)
    assert fq > 0.98 and fk > 0.98, (fq, fk)
    _check_norms(qo, ko, nm, (wqn, wkg))
    # without the norms: the same rows, bit for bit
    qo2, ko2, none = _run(q, k, gq, gk, cos, sin, "bhnd", norms=False)
    assert none is None
    assert np.array_equal(_bits(qo2), _bits(qo)) and np.array_equal(_bits(ko2), _bits(ko))


def test_qk_prep_norms_equal_attn_norms_bitwise():
    """The epilogue sums squares in the same order as attn_norms, so the two
    give identical norms for the same rows."""
    pat, q, k, gq, gk, cos, sin = _small_case(128, 1, 4, 2, 9, 16)
    qo, ko, nm = _run(q, k, gq, gk, cos, sin)
    ref = bs.norms(qo, ko)
    for a, b in zip(nm, ref):
        assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())


def test_qk_prep_identity_rotation_and_unit_weight():
    """cos = 1, sin = 0 and unit weights with eps = 0: plain RMS
    normalisation, every written row of norm sqrt(D) up to bf16 rounding."""
    import torch
    pat, q, k, _, _, cos, sin = _small_case(64, 1, 2, 2, 4, 8)
    one = np.ones(64, np.float32)
    c1, s0 = np.ones_like(cos), np.zeros_like(sin)
    qd, kd = to_device(q), to_device(k)
    qo, ko, nm = bs.qk_prep(qd, kd, _dev(one), _dev(one), _dev(c1), _dev(s0), 0.0)
    torch.cuda.synchronize()
    want = OP.round_bf16(OP.rms_normalize(q, one, 0.0))
    _ulp_check(_bits(qo), want)
    qn = nm[0].cpu().numpy().astype(np.float64)
    assert np.abs(qn - 8.0).max() <= 8.0 * 2.0 ** -8


@pytest.mark.parametrize("name", ["720p", "sr"])
def test_qk_prep_workloads(name):
    """Full size: sampled rows against the oracle, norms checked on every row."""
    wl = WORKLOADS[name]
    q, k, _ = make_qkv(wl)
    gq, gk = norm_weights(wl.head_dim)
    cos, sin = rope_tables(wl.pattern, wl.head_dim, FRAME_GRID[name])
    qo, ko, nm = _run(q, k, gq, gk, cos, sin)
    rows = np.unique(np.concatenate([np.random.default_rng(2).integers(0, wl.seq_len, 512),
                                     np.arange(0, wl.seq_len, wl.pattern.tokens_per_frame),
                                     [wl.seq_len - 1]]))
    wq = OP.round_bf16(OP.qk_norm_rope(q[:, :, rows], gq, EPS, cos[rows], sin[rows]))
    wk = OP.round_bf16(OP.qk_norm_rope(k[:, :, rows], gk, EPS, cos[rows], sin[rows]))
    assert _ulp_check(_bits(qo[:, :, rows]), wq) > 0.98
    assert _ulp_check(_bits(ko[:, :, rows]), wk) > 0.98
    _check_norms(qo, ko, nm)


def _attention_case(name, q, k, v, gq, gk, cos, sin, n_random):
    import torch
    wl = WORKLOADS[name]
    qo, ko, nm = _run(q, k, gq, gk, cos, sin)
    vd = to_device(v)
    host = bs.build_blocks_for(wl.pattern, 256)
    blk = host.to_device(torch.device("cuda"), wl.batch, wl.heads)
    hp = torch.full((wl.batch, wl.heads), -1, dtype=torch.int32, device="cuda")
    o, lse = bs.attention(qo, ko, vd, blk, wl.scale, bs.SOFTMAX_BOUND, norms=nm, head_path=hp)
    torch.cuda.synchronize()
    # the oracle's own producer output feeds the oracle's attention
    wq, wk, _, _, whm = OP.qk_prep(q, k, gq, gk, EPS, cos, sin)
    rows = sample_rows(host.q_tiles, n_random, wl.seq_len) if n_random else None
    o_ref, lse_ref = OA.attention(wq, wk, v, wl.pattern, wl.scale, rows=rows)
    og, lg = bf16_to_f64(o), lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    return errors(og, lg, o_ref, lse_ref), hp.cpu().numpy(), ON.slack_bound(whm, wl.scale)


@pytest.mark.parametrize("name,n_random", [("tiny", 0), ("720p", 256)])
def test_producer_feeds_attention(name, n_random):
    wl = WORKLOADS[name]
    q, k, v = make_qkv(wl)
    gq, gk = norm_weights(wl.head_dim)
    cos, sin = rope_tables(wl.pattern, wl.head_dim, FRAME_GRID[name])
    e, hp, slack = _attention_case(name, q, k, v, gq, gk, cos, sin, n_random)
    assert within(e), e
    assert (slack <= ON.ELIGIBLE_NATS * (1 - 1e-3)).all()
    assert (hp == bs.PATH_BOUND).all()


def test_qk_norm_makes_stress_heads_eligible():
    """The stress inputs fail the per-head test as they are; after the QK
    norm every row's norm is at most sqrt(D) max|g|, and every head takes the
    bound path, within the attention bar."""
    wl = WORKLOADS["stress"]
    q, k, v = make_qkv(wl)
    gq, gk = norm_weights(wl.head_dim)
    cos, sin = rope_tables(wl.pattern, wl.head_dim, FRAME_GRID["stress"])
    raw = ON.slack_bound(ON.head_max(ON.row_norms(q), ON.row_norms(k)), wl.scale)
    assert (raw > ON.ELIGIBLE_NATS).all()
    e, hp, slack = _attention_case("stress", q, k, v, gq, gk, cos, sin, 256)
    assert within(e), e
    assert (slack <= ON.ELIGIBLE_NATS * (1 - 1e-3)).all()
    assert (hp == bs.PATH_BOUND).all()


def test_qk_prep_zero_rows():
    """An all-zero row stays zero (eps > 0) and has norm 0; its granule max
    and the head maxima come from the other rows."""
    import torch
    pat, q, k, gq, gk, cos, sin = _small_case(128, 1, 2, 1, 4, 8)
    q = q.copy(); k = k.copy()
    q[:, :, 3] = 0
    k[:, :, 16:32] = 0          # one whole zero granule
    wq, wk, wqn, wkg, whm = OP.qk_prep(q, k, gq, gk, EPS, cos, sin)
    qo, ko, nm = _run(q, k, gq, gk, cos, sin)
    # zero up to sign (0*cos - 0*sin is -0 where cos < 0)
    assert not (_bits(qo)[:, :, 3] & 0x7FFF).any() and not (_bits(ko)[:, :, 16:32] & 0x7FFF).any()
    qn, kg, hm = (x.cpu().numpy() for x in nm)
    assert (qn[:, :, 3] == 0).all() and (kg[:, :, 1] == 0).all()
    _ulp_check(_bits(qo), wq)
    _ulp_check(_bits(ko), wk)
    _check_norms(qo, ko, nm, (wqn, wkg))

