"""C-ABI library on the CPU: exported symbols, the host integer builders
(bit-exact against the oracle's derivation from the dense mask), the launch
schedule, and argument validation (errors are returned before any launch).
"""
import ctypes
import random
import re

import numpy as np
import pytest

import block_sparse_video_frame_amd as bs
from oracle import blocks as BL
from synth import WORKLOADS, Pattern

HEADER = __import__("os").path.join(__import__("os").path.dirname(__file__), "..", "include", "bsvf.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"attn_build_blocks", "attn_build_schedule", "attn_norms", "attn_fwd",
            "attn_abi_version", "attn_status_str", "attn_last_error"} <= set(names)
    L = ctypes.CDLL(bs.library_path())
    for n in names:
        assert hasattr(L, n), n
    hdr = open(HEADER).read()
    assert bs.abi_version() == int(re.search(r"#define BSVF_ABI_VERSION (\d+)", hdr).group(1)) == bs.ABI_VERSION
    assert bs.lib().attn_status_str(3) == b"ATTN_E_PATTERN"


def as_lists(blk):
    return ([tuple(x) for x in blk.q_tiles.tolist()], blk.kv_ptr.tolist(),
            [tuple(x) for x in blk.kv_iv.tolist()])


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("bq", [16, 128, 256])
def test_builder_matches_oracle_on_workloads(name, bq):
    p = WORKLOADS[name].pattern
    got = bs.build_blocks_for(p, bq)
    want = BL.derive_blocks(p, bq)
    qt, kp, kv = as_lists(got)
    assert qt == want["q_tiles"] and kp == want["kv_ptr"] and kv == want["kv_iv"]
    assert got.useful_pairs == want["useful_pairs"]


def test_builder_matches_oracle_on_random_patterns():
    rnd = random.Random(11)
    for _ in range(150):
        F = rnd.randint(1, 20)
        T = 16 * rnd.randint(1, 32)
        gl = tuple(sorted(set(rnd.randint(0, F - 1) for _ in range(rnd.randint(0, 3)))))
        p = Pattern(F, T, rnd.randint(0, 3), rnd.randint(0, 3), gl)
        bq = 16 * rnd.randint(1, 32)
        got = bs.build_blocks_for(p, bq)
        want = BL.derive_blocks(p, bq, check_rows="all" if F * T <= 2048 else "ends")
        qt, kp, kv = as_lists(got)
        assert qt == want["q_tiles"] and kp == want["kv_ptr"] and kv == want["kv_iv"], p
        assert got.useful_pairs == want["useful_pairs"]


def test_builder_repeated_global_frames_are_merged():
    a = bs.build_blocks(6, 32, 0, 0, (2, 2, 4), 32)
    b = bs.build_blocks(6, 32, 0, 0, (4, 2), 32)
    assert as_lists(a) == as_lists(b)


@pytest.mark.parametrize("args,status", [
    ((4, 40, 1, 1, (), 32), 2),        # T not a multiple of 16
    ((4, 48, 1, 1, (), 24), 2),        # block_q not a multiple of 16
    ((4, 48, 1, 1, (), 0), 2),
    ((0, 48, 1, 1, (), 32), 3),        # no frames
    ((4, 48, -1, 1, (), 32), 3),       # negative window
    ((4, 48, 1, 1, (4,), 32), 3),      # global frame out of range
    ((1 << 20, 4096, 1, 1, (), 256), 4),  # F*T above INT32_MAX
])
def test_builder_errors(args, status):
    with pytest.raises(bs.AttnError) as e:
        bs.build_blocks(*args)
    assert e.value.status == status


def test_builder_capacity_protocol():
    L = bs.lib()
    p = bs._Pattern(5, 64, 1, 1, 0, None)
    n_qt, nnz = ctypes.c_int32(0), ctypes.c_int32(0)
    assert L.attn_build_blocks(ctypes.byref(p), 32, None, None, None, None, ctypes.byref(n_qt), ctypes.byref(nnz)) == 0
    assert (n_qt.value, nnz.value) == (10, 10)
    qt = np.zeros((9, 2), np.int32); kp = np.zeros(10, np.int32); kv = np.zeros((10, 2), np.int32)
    small = ctypes.c_int32(9)
    st = L.attn_build_blocks(ctypes.byref(p), 32, bs._i32(qt), bs._i32(kp), bs._i32(kv), None,
                             ctypes.byref(small), ctypes.byref(nnz))
    assert st == 4 and small.value == 10
    assert b"capacity" in L.attn_last_error()
    assert not qt.any() and not kp.any()
    # NULL pattern / counts
    assert L.attn_build_blocks(None, 32, None, None, None, None, ctypes.byref(n_qt), ctypes.byref(nnz)) == 1


def _tile_costs(blk):
    """Scheduling cost of each tile: keys * max(rows, R/2), or keys * R/3 for
    a short tile of at most R/4 rows (R the largest tile's rows)."""
    R = int(blk.q_tiles[:, 1].max())
    cost = {}
    for t in range(blk.n_qt):
        keys = int(blk.kv_iv[blk.kv_ptr[t]:blk.kv_ptr[t + 1], 1].sum())
        rows = int(blk.q_tiles[t, 1])
        cost[t] = keys * (R // 3 if 4 * rows <= R else max(rows, R // 2))
    return cost


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_schedule_is_a_padded_permutation(name):
    wl = WORKLOADS[name]
    blk = bs.build_blocks_for(wl.pattern, 256)
    items = blk.n_qt * wl.heads * wl.batch
    for group, xcd in [(32, 8), (15, 8), (1, 1), (7, 3)]:
        order = bs.build_schedule(blk, wl.batch, wl.heads, group, xcd)
        assert len(order) % (group * xcd) == 0 and len(order) >= items
        real = order[order >= 0]
        assert sorted(real.tolist()) == list(range(items))
        assert (order[order < 0] == -1).all()
        # every die's queue runs longest work first
        cost = _tile_costs(blk)
        for x in range(xcd):
            seq = [cost[w % blk.n_qt] for w in order[x::xcd] if w >= 0]
            assert all(a >= b for a, b in zip(seq, seq[1:]))
    o1 = bs.build_schedule(blk, wl.batch, wl.heads)
    o2 = bs.build_schedule(blk, wl.batch, wl.heads)
    assert (o1 == o2).all()


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("block_q", [256, 64])
def test_frame_set_schedule(name, block_q):
    """group 0: a permutation; each set of tiles with equal key intervals of one
    head (short tiles left out) sits contiguously on a single die; the sets go
    to the dies in (head, frame) order, each die taking a contiguous run; the
    short tiles follow every set of their die, in the same order, each on its
    set's die; die loads end within the largest set (with its short tiles) of
    each other."""
    wl = WORKLOADS[name]
    blk = bs.build_blocks_for(wl.pattern, block_q)
    items = blk.n_qt * wl.heads * wl.batch
    xcd = 8
    order = bs.build_schedule(blk, wl.batch, wl.heads, 0, xcd)
    assert len(order) % xcd == 0
    real = order[order >= 0]
    assert sorted(real.tolist()) == list(range(items))
    R = int(blk.q_tiles[:, 1].max())
    short = {t: 4 * int(blk.q_tiles[t, 1]) <= R for t in range(blk.n_qt)}
    key = {t: tuple(map(tuple, blk.kv_iv[blk.kv_ptr[t]:blk.kv_ptr[t + 1]].tolist())) for t in range(blk.n_qt)}
    cost = _tile_costs(blk)
    loads = []
    seen = set()
    firsts = []
    for x in range(xcd):
        q = [w for w in order[x::xcd] if w >= 0]
        assert all(w == -1 for w in order[x::xcd][len(q):])       # padding only at the end
        loads.append(sum(cost[w % blk.n_qt] for w in q))
        flags = [short[w % blk.n_qt] for w in q]
        n_long = flags.count(False)
        assert not any(flags[:n_long])                            # short tiles after the sets
        assert q[:n_long] == sorted(q[:n_long]) and q[n_long:] == sorted(q[n_long:])   # (head, frame) order
        runs = []
        for w in q[:n_long]:
            s = (w // blk.n_qt, key[w % blk.n_qt])
            if not runs or runs[-1] != s:
                runs.append(s)
        assert len(runs) == len(set(runs))                        # each set contiguous
        assert not (set(runs) & seen)                             # and on one die only
        seen |= set(runs)
        firsts.append(q[0] if q else None)
        for w in q[n_long:]:                                      # a short tile on its set's die
            t = w % blk.n_qt
            same = [u for u in range(blk.n_qt) if key[u] == key[t] and not short[u]]
            assert not same or (w // blk.n_qt, key[t]) in set(runs)
    # the dies' runs follow one another in (head, frame) order
    nonempty = [f for f in firsts if f is not None]
    assert nonempty == sorted(nonempty)
    units = {}
    for w in range(items):
        t = w % blk.n_qt
        u = (w // blk.n_qt, key[t])
        units[u] = units.get(u, 0) + cost[t]
    assert max(loads) - min(loads) <= max(units.values())


def test_schedule_errors():
    blk = bs.build_blocks(3, 32, 1, 1, (), 32)
    with pytest.raises(bs.AttnError):
        bs.build_schedule(blk, 1, 1, -1, 8)
    with pytest.raises(bs.AttnError):
        bs.build_schedule(blk, 1, 1, 4, 0)
    with pytest.raises(bs.AttnError):
        bs.build_schedule(blk, 0, 1, 4, 8)


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# The validation cases below pass addresses that are never dereferenced: each
# case carries an argument that the library rejects before any HIP call.  They
# run where no GPU is visible only.
no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="validation-only test for CPU hosts")

FAKE = 0x10000  # 16-byte aligned, never dereferenced


def fwd_call(entry="attn_fwd", **over):
    L = bs.lib()
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, shift=None, B=1, H=2, N=192, D=64,
                strides=[192 * 64 * 2, 192 * 64, 64] * 4, scale=0.125, blocks="ok",
                qn=None, kg=None, hm=None, mode=0, hp=None)
    args.update(over)
    st = (ctypes.c_int64 * 12)(*args["strides"]) if args["strides"] is not None else None
    cb = bs._Blocks(FAKE, FAKE, FAKE, 4, 4, 256, None, 0)
    if isinstance(args["blocks"], dict):
        for k, v in args["blocks"].items():
            setattr(cb, k, v)
    bp = ctypes.byref(cb) if args["blocks"] is not None else None
    return getattr(L, entry)(args["q"], args["k"], args["v"], args["o"], args["lse"], args["shift"],
                      args["B"], args["H"], args["N"], args["D"], st, ctypes.c_float(args["scale"]), bp,
                      args["qn"], args["kg"], args["hm"], args["mode"], args["hp"], None)


@no_gpu_only
@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1),
    (dict(blocks=None), 1),
    (dict(strides=None), 1),
    (dict(B=0), 1),
    (dict(mode=6), 1),                     # no such mode
    (dict(mode=-1), 1),                    # no such mode
    (dict(mode=5), 5),                     # checked bound without norms
    (dict(mode=4), 5),                     # exact bound without norms
    (dict(mode=3), 5),                     # per-tile bound without norms
    (dict(scale=0.0), 1),
    (dict(scale=float("nan")), 1),
    (dict(D=96), 5),
    (dict(N=200), 2),
    (dict(q=FAKE + 2), 2),
    (dict(strides=[192 * 64 * 2, 192 * 64, 60] + [192 * 64 * 2, 192 * 64, 64] * 3), 2),
    (dict(strides=[192 * 64 * 2, 192 * 64, 32] + [192 * 64 * 2, 192 * 64, 64] * 3), 2),
    (dict(blocks={"block_q": 24}), 2),
    (dict(blocks={"block_q": 512}), 5),
    (dict(blocks={"n_qt": 0}), 1),
    (dict(blocks={"q_tiles": None}), 1),
    (dict(mode=1), 5),                 # bound mode without norms
    (dict(blocks={"work_ctr": FAKE}), 1),                                   # counters without a work_order
    (dict(blocks={"work_ctr": FAKE, "work_order": FAKE, "n_work": 16, "num_xcd": 0}), 1),
    (dict(blocks={"work_ctr": FAKE, "work_order": FAKE, "n_work": 66, "num_xcd": 33}), 1),
    (dict(blocks={"work_ctr": FAKE, "work_order": FAKE, "n_work": 12, "num_xcd": 8}), 1),  # not whole queues
    (dict(N=1 << 26, strides=[(1 << 26) * 64 * 2, (1 << 26) * 64, 64] * 4), 4),  # head span > 2^31
])
def test_fwd_validation(over, status):
    assert fwd_call(**over) == status
    assert bs.lib().attn_last_error().startswith(bs.lib().attn_status_str(status))


@no_gpu_only
@pytest.mark.parametrize("over,status", [
    (dict(), 1),                                                               # no work_order
    (dict(blocks={"work_order": FAKE, "n_work": 16, "num_xcd": 8, "work_ctr": FAKE}), 1),  # its own counters given
    (dict(blocks={"work_order": FAKE, "n_work": 66, "num_xcd": 33}), 4),       # beyond the counter array
    (dict(blocks={"work_order": FAKE, "n_work": 16, "num_xcd": 0}), 1),
    (dict(blocks={"work_order": FAKE, "n_work": 12, "num_xcd": 8}), 1),        # not whole queues
    (dict(q=None, blocks={"work_order": FAKE, "n_work": 16, "num_xcd": 8}), 1),
])
def test_fwd_noalloc_validation(over, status):
    """attn_fwd_noalloc rejects what it cannot run before any HIP call: no launch
    order, a caller workspace, more queues than its counter array holds."""
    assert fwd_call("attn_fwd_noalloc", **over) == status
    assert bs.lib().attn_last_error().startswith(bs.lib().attn_status_str(status))


@no_gpu_only
@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1), (dict(D=32), 5), (dict(N=100), 2), (dict(k=FAKE + 8), 2), (dict(qn=None), 1),
])
def test_norms_validation(over, status):
    L = bs.lib()
    a = dict(q=FAKE, k=FAKE, B=1, H=2, N=192, D=64, qn=FAKE, kg=FAKE, hm=FAKE)
    a.update(over)
    s = (ctypes.c_int64 * 3)(a["N"] * a["D"] * 2, a["N"] * a["D"], a["D"])
    st = L.attn_norms(a["q"], a["k"], a["B"], a["H"], a["N"], a["D"], s, s, a["qn"], a["kg"], a["hm"], None)
    assert st == status


def prep_call(**over):
    L = bs.lib()
    a = dict(qi=FAKE, ki=FAKE + 0x100000, qo=FAKE + 0x200000, ko=FAKE + 0x300000, B=1, H=2, N=192, D=64,
             strides=[192 * 64 * 2, 192 * 64, 64] * 4, gq=FAKE, gk=FAKE, eps=1e-6, cos=FAKE, sin=FAKE,
             qn=FAKE, kg=FAKE, hm=FAKE)
    a.update(over)
    st = (ctypes.c_int64 * 12)(*a["strides"]) if a["strides"] is not None else None
    return L.attn_qk_prep(a["qi"], a["ki"], a["qo"], a["ko"], a["B"], a["H"], a["N"], a["D"], st, a["gq"],
                          a["gk"], ctypes.c_float(a["eps"]), a["cos"], a["sin"], a["qn"], a["kg"], a["hm"], None)


_S = [192 * 64 * 2, 192 * 64, 64]


@no_gpu_only
@pytest.mark.parametrize("over,status", [
    (dict(qi=None), 1), (dict(ko=None), 1), (dict(strides=None), 1), (dict(B=0), 1), (dict(H=-1), 1),
    (dict(D=96), 5), (dict(N=200), 2), (dict(qo=FAKE + 0x200008), 2),
    (dict(strides=_S * 2 + [192 * 64 * 2, 192 * 64, 60] + _S), 2),
    (dict(gq=None), 1), (dict(sin=None), 1), (dict(cos=FAKE + 4), 2), (dict(gk=FAKE + 8), 2),
    (dict(eps=-1.0), 1), (dict(eps=float("nan")), 1), (dict(eps=float("inf")), 1),
    (dict(kg=None), 1), (dict(qn=None, hm=None), 1),                     # some norm outputs only
    (dict(qo=FAKE + 0x300000), 1),                                       # q_out == k_out
    (dict(qo=FAKE + 0x100000), 1),                                       # q_out == k_in
    (dict(qo=FAKE, strides=_S * 2 + [192 * 64 * 2, 192 * 64, 128] + _S), 1),  # in place, other strides
    (dict(B=70000, strides=_S * 4), 4),
    (dict(H=70000, N=16, strides=[70000 * 16 * 64, 16 * 64, 64] * 4), 4),   # B * H above 65535
])
def test_qk_prep_validation(over, status):
    assert prep_call(**over) == status
    assert bs.lib().attn_last_error().startswith(bs.lib().attn_status_str(status))


def test_binding_checks_shapes_before_any_device_work():
    """The library sees pointers and strides only, so the binding refuses
    tensors whose shapes disagree (they would be read past their end); these
    checks come before the device checks, so they run on CPU tensors."""
    import torch
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)
    short = torch.zeros(1, 2, 48, 64, dtype=torch.bfloat16)
    dev = bs.build_blocks_for(Pattern(2, 32, 1, 1), 32).to_device(torch.device("cpu"), 1, 2)
    with pytest.raises(ValueError, match="shape"):
        bs.norms(q, short)
    with pytest.raises(ValueError, match="shape"):
        bs.attention(q, short, q, dev)
    with pytest.raises(ValueError, match="shape"):
        bs.attention(q, q, q, dev, out=short)
    with pytest.raises(ValueError, match="tokens"):
        bs.attention(short, short, short, dev)
    other = bs.build_blocks_for(Pattern(2, 32, 1, 1), 32).to_device(torch.device("cpu"), 1, 4)
    with pytest.raises(ValueError, match="launch order"):
        bs.attention(q, q, q, other)
    g = torch.ones(64)
    t = torch.ones(64, 32)
    with pytest.raises(ValueError, match="shape"):
        bs.qk_prep(q, q, g, g, t, t, q_out=short)
    with pytest.raises(ValueError, match="CUDA"):
        bs.attention(q, q, q, dev)


# ---- frame-unaware layout (alignment ablation) -------------------------------------------


def _granular_lists(blk):
    return ([tuple(x) for x in blk.q_tiles.tolist()], blk.kv_ptr.tolist(),
            [tuple(x) for x in blk.kv_iv.tolist()], blk.kv_flag.tolist())


@pytest.mark.parametrize("name", [n for n in WORKLOADS if n != "stress"])
@pytest.mark.parametrize("granule", [64, 128])
def test_granular_builder_matches_oracle_on_workloads(name, granule):
    p = WORKLOADS[name].pattern
    got = bs.build_blocks_granular(p, granule, 256)
    want = BL.derive_blocks_granular(p, granule, 256)
    qt, kp, kv, fl = _granular_lists(got)
    assert qt == want["q_tiles"] and kp == want["kv_ptr"] and kv == want["kv_iv"] and fl == want["kv_flag"]
    assert got.useful_pairs == BL.derive_blocks(p, 256)["useful_pairs"]


def test_granular_builder_matches_oracle_on_random_patterns():
    rnd = random.Random(23)
    for _ in range(60):
        F = rnd.randint(1, 9)
        T = 16 * rnd.randint(4, 24)
        gl = tuple(sorted(set(rnd.randint(0, F - 1) for _ in range(rnd.randint(0, 2)))))
        p = Pattern(F, T, rnd.randint(0, 2), rnd.randint(0, 2), gl)
        granule = rnd.choice([64, 128, 192])
        bq = 16 * rnd.randint(1, 16)
        got = bs.build_blocks_granular(p, granule, bq)
        want = BL.derive_blocks_granular(p, granule, bq, check_rows="all")
        qt, kp, kv, fl = _granular_lists(got)
        assert qt == want["q_tiles"] and kp == want["kv_ptr"] and kv == want["kv_iv"] and fl == want["kv_flag"], p


def test_granular_layout_covers_the_mask_exactly():
    """Runs flagged 0 are fully attended by every row of the tile, and the union
    of a tile's runs contains every attended key of every row."""
    from oracle.attention import frame_mask
    p = Pattern(6, 160, 1, 1, (0,))
    blk = bs.build_blocks_granular(p, 128, 128)
    N = p.num_frames * p.tokens_per_frame
    for t in range(blk.n_qt):
        qs, nr = blk.q_tiles[t]
        M = frame_mask(p, np.arange(qs, qs + nr), N)
        cover = np.zeros(N, bool)
        for e in range(blk.kv_ptr[t], blk.kv_ptr[t + 1]):
            ks, kl = blk.kv_iv[e]
            cover[ks:ks + kl] = True
            if blk.kv_flag[e] == 0:
                assert M[:, ks:ks + kl].all()
            else:
                assert not M[:, ks:ks + kl].all()
        assert not (M & ~cover[None, :]).any()


def test_granular_builder_errors():
    p = Pattern(3, 64, 1, 1)
    with pytest.raises(bs.AttnError):
        bs.build_blocks_granular(p, 96, 128)      # granule not a multiple of 64
    with pytest.raises(bs.AttnError):
        bs.build_blocks_granular(p, 128, 40)      # block_q not a multiple of 16


def test_device_blocks_workspace():
    """The device block list carries the persistent launch's counters: zeroed,
    num_xcd + 1 of them, passed through attn_blocks_t; none for a static launch."""
    import torch
    blk = bs.build_blocks_for(Pattern(2, 32, 1, 1), 32)
    cpu = torch.device("cpu")
    d = blk.to_device(cpu, 1, 2, num_xcd=8)
    assert d.work_ctr is not None and d.work_ctr.dtype == torch.int32
    assert d.work_ctr.numel() == 9 and not d.work_ctr.any()
    cs = d.c_struct()
    assert cs.num_xcd == 8 and cs.work_ctr == d.work_ctr.data_ptr()
    assert cs.work_order == d.work_order.data_ptr() and cs.n_work == d.work_order.numel()
    assert d.work_order.numel() % 8 == 0
    assert blk.to_device(cpu, 1, 2, persistent=False).work_ctr is None
    assert blk.to_device(cpu, 1, 2, persistent=False).c_struct().work_ctr is None
    assert blk.to_device(cpu, 1, 2, schedule=False).work_ctr is None
    assert blk.to_device(cpu, 1, 2, num_xcd=3).work_ctr.numel() == 4


def test_device_blocks_orders_calls_across_streams():
    """Launches that share the slot counters are ordered across streams: a call
    on a new stream first waits for the previous stream's work; a call on the
    same stream adds nothing; a static list (no counters) never waits."""
    blk = bs.build_blocks_for(Pattern(2, 32, 1, 1), 32)
    cpu = __import__("torch").device("cpu")

    class FakeStream:
        def __init__(self, name, log):
            self.name, self.log = name, log

        def wait_stream(self, other):
            self.log.append((self.name, other.name))

    log = []
    a, b = FakeStream("a", log), FakeStream("b", log)
    d = blk.to_device(cpu, 1, 2)
    for s in (a, a, b, b, a, b):
        d.order_on(s)
    assert log == [("b", "a"), ("a", "b"), ("b", "a")]
    log.clear()
    st = blk.to_device(cpu, 1, 2, persistent=False)
    for s in (a, b, a):
        st.order_on(s)
    assert log == []



@no_gpu_only
def test_masked_entry_rejects_the_checked_mode():
    """attn_fwd_masked takes softmax modes 0 to 4: mode 5 is refused before any
    device work (ATTN_E_UNSUPPORTED), mode 6 as no mode at all."""
    L = bs.lib()
    pat = bs._Pattern(4, 48, 1, 1, 0, None)
    st = (ctypes.c_int64 * 12)(*([192 * 64 * 2, 192 * 64, 64] * 4))
    cb = bs._Blocks(FAKE, FAKE, FAKE, 4, 4, 256, None, 0)
    for mode, want in ((5, 5), (6, 1)):
        got = L.attn_fwd_masked(FAKE, FAKE, FAKE, FAKE, None, None, 1, 2, 192, 64, st, ctypes.c_float(0.125),
                                ctypes.byref(cb), FAKE, ctypes.byref(pat), FAKE, FAKE, FAKE, mode, None, None)
        assert got == want, (mode, got, bs.lib().attn_last_error())
