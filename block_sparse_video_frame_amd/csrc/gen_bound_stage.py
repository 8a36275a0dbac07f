#!/usr/bin/env python3
"""Generates attn_bound_stage.h: the per-stage instruction blocks of the
bound-softmax attention kernel for gfx950 (head_dim 64 and 128).

Run from this directory:  python3 gen_bound_stage.py  (rewrites the header).

Why generated assembly.  One wave owns 64 query rows, so per 64-key stage it
issues 64 MFMAs (32x32x16 bf16), 64 exps and 48 LDS reads.  Its state needs
about 450 registers: Q (bf16, B operand) and the output accumulator in AGPRs,
score tiles, the shift, P and operand buffers in VGPRs.  The compiler, given
MFMA builtins, puts every accumulator in AGPRs once a wave may use more than
256 registers and then copies each score to a VGPR before its exp.  Here the
register file is laid out by hand instead: the kernel caps the compiler at
the low VGPRs (amdgpu_num_vgpr) and the blocks below own the rest.  Values
live in fixed registers across blocks; the C++ code around them only issues
the LDS copies, barriers and loop control, which use no AGPRs and no VGPR
above the cap.

Each block is straight-line code with its own s_waitcnt bookkeeping (LDS reads
complete in order; a block starts by draining lgkmcnt).  Hazards that the
hardware does not interlock are respected by construction and checked here:
  * MFMA result -> VALU read or MFMA A/B operand: >= 12 wait states (scores
    are written in one block and read in the next; the last write of a block
    is followed by at least 8 MFMAs or explicit s_nop);
  * VALU write -> MFMA A/B operand: >= 2 wait states (P is written in one
    phase and read in a later one; checked per instruction);
  * transcendental (v_exp) result -> other VALU read: >= 1 wait state (the
    pair conversion is issued after the next independent instruction);
  * back-to-back MFMAs accumulating into the same registers need none.

Per stage s the main block does, with S(kb) the 32x32 score tiles of key
block kb (keys 32kb..32kb+31) and P their bf16 probabilities:
  phase 1: S(s+1, kb=1) = K*Q'^T - m (16 MFMAs), O += V(s-1, kb=1)^T P(s-1, kb=1)
           (16 MFMAs), P(s, kb=0) = exp2(S(s, kb=0)) with row sums;
  phase 2: S(s+1, kb=0) (16 MFMAs), O += V(s, kb=0)^T P(s, kb=0) (16 MFMAs),
           P(s, kb=1) = exp2(S(s, kb=1)) with row sums.
Score tiles rotate through three register blocks: kb=0 always in block A (its
exps finish in phase 1 before phase 2 overwrites it), kb=1 alternates between
B and C, so blocks come in an even and an odd form.
"""
from __future__ import annotations

import os

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "attn_bound_stage.h")

NQB = 2          # 32-row query blocks per wave
N_KOP = 4        # K operand buffers (reads run up to 3 QK items ahead)
N_VOP = 3        # V operand buffers (2 PV items ahead)
N_ETMP = 4
ONES_BF16X2 = "0x3f803f80"


class Layout:
    def __init__(self, D):
        self.D = D
        self.KSTEPS = D // 16
        self.DBLK = D // 32
        self.RS = 2 * D                    # bytes per K/V row in LDS
        self.VREG = 64 * D * 2             # byte offset of the V region in a stage
        # AGPRs: Q' (B operand of Q*K^T), then the output accumulators.
        self.QA = 0
        self.OA = 4 * NQB * self.KSTEPS
        self.n_agpr = self.OA + 16 * NQB * self.DBLK
        # VGPRs owned by the blocks, allocated from `base` upward.
        v = []

        def take(n):
            start = len(v)
            v.extend(range(start, start + n))
            return start
        self.S = {blk: [take(16) for _ in range(NQB)] for blk in "ABC"}
        self.NEG = [take(16) for _ in range(NQB)]
        self.P = {(qb, kb, kst): take(4) for qb in range(NQB) for kb in range(2) for kst in range(2)}
        self.KOP = [take(4) for _ in range(N_KOP)]
        self.VOP = [take(4) for _ in range(N_VOP)]
        self.KADR = [take(1) for _ in range(2)]
        self.VADR = {(h, db): take(1) for h in range(2) for db in range(self.DBLK)}
        self.LSUM = {(qb, j): take(1) for qb in range(NQB) for j in range(2)}
        self.ETMP = [take(1) for _ in range(N_ETMP)]
        self.n_vgpr = len(v)
        self.base = 256 - self.n_vgpr      # first block-owned VGPR; the compiler gets v0..base-1

    # register names
    def v(self, off, n=1):
        r = self.base + off
        return f"v{r}" if n == 1 else f"v[{r}:{r + n - 1}]"

    def q(self, qb, st):
        r = self.QA + 4 * (qb * self.KSTEPS + st)
        return f"a[{r}:{r + 3}]"

    def o(self, qb, db):
        r = self.OA + 16 * (qb * self.DBLK + db)
        return f"a[{r}:{r + 15}]"


class Stream:
    """Straight-line instruction list with LDS-read bookkeeping and hazard checks."""

    def __init__(self, L):
        self.L = L
        self.out = []
        self.n_reads = 0          # LDS reads issued in this block
        self.done_upto = 0        # reads known complete (by a wait)
        self.last_valu_write = {}  # vgpr offset -> instruction index
        self.last_mfma_write = {}  # vgpr offset -> instruction index (VGPR results only)
        self.last_trans_write = {}  # vgpr offset -> instruction index of a v_exp writing it

    def emit(self, s):
        self.out.append(s)

    def idx(self):
        return len(self.out)

    def read(self, instr):
        self.emit(instr)
        self.n_reads += 1
        return self.n_reads - 1

    def wait_read(self, r):
        """Make LDS read r (0-based, this block) complete."""
        if r < self.done_upto:
            return
        outstanding_allowed = self.n_reads - r - 1
        assert 0 <= outstanding_allowed <= 15
        self.emit(f"s_waitcnt lgkmcnt({outstanding_allowed})")
        self.done_upto = r + 1

    def valu_write(self, offs):
        for o in offs:
            self.last_valu_write[o] = self.idx()

    def mfma_operand_check(self, offs):
        """VALU write -> MFMA operand needs 2 wait states."""
        need = 0
        for o in offs:
            w = self.last_valu_write.get(o)
            if w is not None:
                need = max(need, 2 - (self.idx() - w - 1))
        if need > 0:
            self.emit(f"s_nop {need - 1}")

    def trans_read_check(self, offs):
        """v_exp result -> non-transcendental VALU read needs 1 wait state."""
        for o in offs:
            w = self.last_trans_write.get(o)
            if w is not None and self.idx() - w - 1 < 1:
                self.emit("s_nop 0")
                return

    def valu_read_check(self, offs):
        need = 0
        for o in offs:
            w = self.last_mfma_write.get(o)
            if w is not None:
                need = max(need, 12 - (self.idx() - w - 1))
        if need > 0:
            self.emit(f"s_nop {min(need, 16) - 1}")
            if need > 16:
                self.emit(f"s_nop {need - 17}")


def build_block(L, kind, parity, first, nvalid=64):
    """kind: 'qk0' (scores of stage 0), 'main', 'last'.
    parity: 0 -> current kb=1 scores in B, next in C; 1 -> current in C, next in B.
    first: no P*V of a previous stage.  nvalid: keys of the (last) stage."""
    S = Stream(L)
    KS, DB = L.KSTEPS, L.DBLK
    cur1 = "B" if parity == 0 else "C"
    nxt1 = "C" if parity == 0 else "B"
    S.emit("s_waitcnt lgkmcnt(0)")

    # operands: %0 K base (next stage, or stage 0 for qk0), %1/%2 V bases of the
    # current stage (h = 0/1), %3/%4 V bases of the previous stage.
    KBASE, VCUR, VPREV = "%0", ("%1", "%2"), ("%3", "%4")

    # ---- work lists -------------------------------------------------------
    # QK items: (kb, st) -> destination block
    def qk_items(kb, dst_blk):
        return [("qk", kb, st, dst_blk) for st in range(KS)]

    def pv_items(kb, src, granules):
        # src: 'prev' or 'cur' V buffer; granules: valid (kb, kst) of the stage
        return [("pv", kb, kst, db, src) for kst in range(2) for db in range(DB) if (kb, kst) in granules]

    all_g = {(kb, kst) for kb in range(2) for kst in range(2)}
    valid_g = {(kb, kst) for kb in range(2) for kst in range(2) if 16 * (2 * kb + kst) < nvalid}

    def exp_ops(kb, blk, granules):
        """VALU ops computing P(qb, kb, kst) = bf16(exp2(S)) and row sums."""
        ops = []
        t = 0
        pending = None
        for qb in range(NQB):
            for kst in range(2):
                if (kb, kst) not in granules:
                    continue
                sreg = L.S[blk][qb]
                preg = L.P[(qb, kb, kst)]
                for j in range(4):
                    e0 = L.ETMP[t % N_ETMP]
                    e1 = L.ETMP[(t + 1) % N_ETMP]
                    t += 2
                    s0 = sreg + 8 * kst + 2 * j
                    ops.append(("exp", e0, s0))
                    ops.append(("exp", e1, s0 + 1))
                    # the row-sum update of the previous pair separates the
                    # second exp from the conversion that reads it
                    if pending is not None:
                        ops.append(pending)
                    ops.append(("cvt", preg + j, e0, e1))
                    pending = ("dot", L.LSUM[(qb, j & 1)], preg + j)
        if pending is not None:
            ops.append(pending)
        return ops

    phases = []
    if kind == "qk0":
        phases.append((qk_items(1, "B") + qk_items(0, "A"), []))
    elif kind == "main":
        m1 = qk_items(1, nxt1) + ([] if first else pv_items(1, "prev", all_g))
        m2 = qk_items(0, "A") + pv_items(0, "cur", all_g)
        phases.append((m1, exp_ops(0, "A", all_g)))
        phases.append((m2, exp_ops(1, cur1, all_g)))
    else:  # last
        m1 = [] if first else pv_items(1, "prev", all_g)
        phases.append((m1, exp_ops(0, "A", valid_g)))
        phases.append((pv_items(0, "cur", valid_g), exp_ops(1, cur1, valid_g)))
        phases.append((pv_items(1, "cur", valid_g), []))

    # interleave QK and PV items of a phase (QK first, then alternate)
    def interleave(items):
        qk = [x for x in items if x[0] == "qk"]
        pv = [x for x in items if x[0] == "pv"]
        outl = []
        while qk or pv:
            if qk:
                outl.append(qk.pop(0))
            if pv:
                outl.append(pv.pop(0))
        return outl

    # ---- reads ------------------------------------------------------------
    # Build the global read list over all phases, in consumption order.
    plan = []   # per phase: list of items with read ids
    reads = []  # dicts: item, phase, pos, kind
    for ph, (items, _) in enumerate(phases):
        seq = interleave(items)
        plan.append(seq)
        for pos, it in enumerate(seq):
            reads.append({"item": it, "phase": ph, "pos": pos})

    kop_i = 0
    vop_i = 0
    for r in reads:
        if r["item"][0] == "qk":
            r["buf"] = kop_i % N_KOP
            r["bufseq"] = kop_i
            kop_i += 1
        else:
            r["buf"] = vop_i % N_VOP
            r["bufseq"] = vop_i
            vop_i += 1

    issued = 0                  # index into reads
    read_ids = {}               # read list index -> (lo id, hi id) or (id,)
    consumed = set()            # read list indices whose MFMAs were emitted
    vadr_src = None             # which V base VADR currently holds

    def buffer_free(ri):
        r = reads[ri]
        # the previous user of this buffer (bufseq - N) must have been consumed
        n = N_KOP if r["item"][0] == "qk" else N_VOP
        prev_seq = r["bufseq"] - n
        if prev_seq < 0:
            return True
        for j, rr in enumerate(reads):
            if rr["item"][0] == r["item"][0] and rr["bufseq"] == prev_seq:
                return j in consumed
        return True

    def issue_read(ri):
        nonlocal vadr_src
        r = reads[ri]
        it = r["item"]
        if it[0] == "qk":
            _, kb, st, _ = it
            kop = L.KOP[r["buf"]]
            if st == 0:
                addr = KBASE
            else:
                a = L.KADR[r["bufseq"] % 2]
                S.emit(f"v_xor_b32_e32 {L.v(a)}, {32 * st}, {KBASE}")
                S.valu_write([a])
                addr = L.v(a)
            off = 32 * L.RS * kb
            read_ids[ri] = (S.read(f"ds_read_b128 {L.v(kop, 4)}, {addr} offset:{off}"),)
        else:
            _, kb, kst, db, src = it
            bases = VPREV if src == "prev" else VCUR
            if vadr_src != src:
                for h in range(2):
                    for d in range(DB):
                        a = L.VADR[(h, d)]
                        if d == 0:
                            S.emit(f"v_mov_b32 {L.v(a)}, {bases[h]}")
                        else:
                            S.emit(f"v_xor_b32_e32 {L.v(a)}, {64 * d}, {bases[h]}")
                        S.valu_write([a])
                vadr_src = src
            vop = L.VOP[r["buf"]]
            off = L.VREG + L.RS * (32 * kb + 16 * kst)
            lo = S.read(f"ds_read_b64_tr_b16 {L.v(vop, 2)}, {L.v(L.VADR[(0, db)])} offset:{off}")
            hi = S.read(f"ds_read_b64_tr_b16 {L.v(vop + 2, 2)}, {L.v(L.VADR[(1, db)])} offset:{off}")
            read_ids[ri] = (lo, hi)

    def emit_valu(op):
        if op[0] == "exp":
            _, dst, src = op
            S.valu_read_check([src])
            S.emit(f"v_exp_f32 {L.v(dst)}, {L.v(src)}")
            S.valu_write([dst])
            S.last_trans_write[dst] = S.idx() - 1
        elif op[0] == "cvt":
            _, dst, a, b = op
            S.trans_read_check([a, b])
            S.emit(f"v_cvt_pk_bf16_f32 {L.v(dst)}, {L.v(a)}, {L.v(b)}")
            S.valu_write([dst])
        elif op[0] == "dot":
            _, acc, p = op
            S.emit(f"v_dot2c_f32_bf16_e32 {L.v(acc)}, {ONES_BF16X2}, {L.v(p)}")
            S.valu_write([acc])
        elif op[0] == "zero":
            _, dst = op
            S.emit(f"v_mov_b32 {L.v(dst)}, 0")
            S.valu_write([dst])

    ahead_qk = N_KOP - 1
    ahead_pv = N_VOP - 1
    global_pos = 0
    ri_base = 0
    for ph, seq in enumerate(plan):
        valu = list(phases[ph][1])
        n_items = len(seq)
        n_mfma = sum(NQB for _ in seq)
        total_valu = len(valu)
        done_valu = 0
        slot = 0
        for pos, it in enumerate(seq):
            my_ri = ri_base + pos
            # issue reads inside the look-ahead window whose buffers are free
            while issued < len(reads):
                r = reads[issued]
                gpos = r["phase"], r["pos"]
                dist = (sum(len(p) for p in plan[:r["phase"]]) + r["pos"]) - (sum(len(p) for p in plan[:ph]) + pos)
                ahead = ahead_qk if r["item"][0] == "qk" else ahead_pv
                if dist > ahead or not buffer_free(issued):
                    break
                issue_read(issued)
                issued += 1
            assert my_ri in read_ids, "operand read not issued before its MFMA"
            S.wait_read(read_ids[my_ri][-1])
            for qb in range(NQB):
                if it[0] == "qk":
                    _, kb, st, dst_blk = it
                    dst = L.S[dst_blk][qb]
                    srcc = L.v(L.NEG[qb], 16) if st == 0 else L.v(dst, 16)
                    kop = L.KOP[reads[my_ri]["buf"]]
                    S.mfma_operand_check(range(kop, kop + 4))
                    S.emit(f"v_mfma_f32_32x32x16_bf16 {L.v(dst, 16)}, {L.v(kop, 4)}, {L.q(qb, st)}, {srcc}")
                    for o in range(dst, dst + 16):
                        S.last_mfma_write[o] = S.idx() - 1
                else:
                    _, kb, kst, db, src = it
                    vop = L.VOP[reads[my_ri]["buf"]]
                    p = L.P[(qb, kb, kst)]
                    S.mfma_operand_check(list(range(vop, vop + 4)) + list(range(p, p + 4)))
                    S.emit(f"v_mfma_f32_32x32x16_bf16 {L.o(qb, db)}, {L.v(vop, 4)}, {L.v(p, 4)}, {L.o(qb, db)}")
                slot += 1
                # spread this phase's VALU work evenly over its MFMAs
                target = (total_valu * slot + n_mfma - 1) // n_mfma if n_mfma else total_valu
                while done_valu < target:
                    emit_valu(valu[done_valu])
                    done_valu += 1
            consumed.add(my_ri)
        while done_valu < total_valu:
            emit_valu(valu[done_valu])
            done_valu += 1
        ri_base += n_items
    assert issued == len(reads)
    # leave no LDS read in flight, and (qk0) give the score results time to land
    S.emit("s_waitcnt lgkmcnt(0)")
    if kind == "qk0":
        S.emit("s_nop 7")
        S.emit("s_nop 7")
    return S.out


def clobbers(L):
    vs = [f'"v{L.base + i}"' for i in range(L.n_vgpr)]
    as_ = [f'"a{i}"' for i in range(L.n_agpr)]
    return ", ".join(['"memory"'] + vs + as_)


def c_string(lines):
    return "\n".join(f'      "{l}\\n"' for l in lines)


def gen(D):
    L = Layout(D)
    out = []
    name = f"D{D}"
    clob = clobbers(L)
    out.append(f"// ---- head_dim {D}: VGPR v{L.base}..v255 and AGPR a0..a{L.n_agpr - 1} belong to these blocks")
    out.append(f"template <> struct BoundStage<{D}> {{")
    out.append(f"  static constexpr int kFirstOwnedVgpr = {L.base};")
    out.append(f"  static constexpr int kAgprs = {L.n_agpr};")

    def block_fn(fname, lines, nargs):
        args = ", ".join(f"uint32_t x{i}" for i in range(nargs))
        ins = ", ".join(f'"v"(x{i})' for i in range(nargs))
        out.append(f"  static __device__ __forceinline__ void {fname}({args}) {{")
        out.append("    asm volatile(")
        out.append(c_string(lines))
        out.append(f"      :: {ins}")
        out.append(f"      : {clob});")
        out.append("  }")

    block_fn("qk0", build_block(L, "qk0", 0, True), 5)
    for parity in (0, 1):
        for first in ((True, False) if parity == 0 else (False,)):
            block_fn(f"main_p{parity}{'_first' if first else ''}", build_block(L, "main", parity, first), 5)
    for parity in (0, 1):
        for first in ((True, False) if parity == 0 else (False,)):
            for nv in (16, 32, 48, 64):
                block_fn(f"last_p{parity}{'_first' if first else ''}_n{nv}",
                         build_block(L, "last", parity, first, nv), 5)

    # set-up and read-out helpers
    # Q'(qb, st) <- 4 packed bf16 pairs
    out.append("  // Q' rows of query block qb, k-step st, into the AGPRs of the B operand")
    out.append("  static __device__ __forceinline__ void set_q(int qb, int st, uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {")
    out.append("    switch (qb * %d + st) {" % L.KSTEPS)
    for qb in range(NQB):
        for st in range(L.KSTEPS):
            r = L.QA + 4 * (qb * L.KSTEPS + st)
            body = "".join(f'"v_accvgpr_write_b32 a{r + j}, %{j}\\n" ' for j in range(4))
            out.append(f'      case {qb * L.KSTEPS + st}: asm volatile({body}:: "v"(w0), "v"(w1), "v"(w2), "v"(w3) : {clob}); break;')
    out.append("      default: break;")
    out.append("    }")
    out.append("  }")
    # shift, zero accumulators and row sums
    out.append("  // -m (log2 units) of the rows of query blocks 0 and 1; clears O and the row sums")
    lines = []
    for qb in range(NQB):
        for i in range(16):
            lines.append(f"v_mov_b32 {L.v(L.NEG[qb] + i)}, %{qb}")
    for qb in range(NQB):
        for j in range(2):
            lines.append(f"v_mov_b32 {L.v(L.LSUM[(qb, j)])}, 0")
    for r in range(L.OA, L.n_agpr):
        lines.append(f"v_accvgpr_write_b32 a{r}, 0")
    lines += ["s_nop 7", "s_nop 7"]
    out.append("  static __device__ __forceinline__ void init(float neg0, float neg1) {")
    out.append("    asm volatile(")
    out.append(c_string(lines))
    out.append('      :: "v"(neg0), "v"(neg1)')
    out.append(f"      : {clob});")
    out.append("  }")
    # row sums out
    out.append("  // this lane's partial row sums of query blocks 0 and 1")
    out.append("  static __device__ __forceinline__ void row_sums(float& l0, float& l1) {")
    out.append("    asm volatile(")
    out.append(c_string([f"v_add_f32 %0, {L.v(L.LSUM[(0, 0)])}, {L.v(L.LSUM[(0, 1)])}",
                         f"v_add_f32 %1, {L.v(L.LSUM[(1, 0)])}, {L.v(L.LSUM[(1, 1)])}"]))
    out.append('      : "=v"(l0), "=v"(l1)')
    out.append(f"      :: {clob});")
    out.append("  }")
    # O out: 16 values of (qb, db)
    out.append("  // the 16 accumulator values of output block db of query block qb")
    out.append("  static __device__ __forceinline__ void read_o(int qb, int db, float (&r)[16]) {")
    outs = ", ".join(f'"=v"(r[{i}])' for i in range(16))
    out.append("    switch (qb * %d + db) {" % L.DBLK)
    for qb in range(NQB):
        for db in range(L.DBLK):
            a0 = L.OA + 16 * (qb * L.DBLK + db)
            body = '"s_nop 7\\n" "s_nop 7\\n" "s_nop 7\\n" ' + "".join(
                f'"v_accvgpr_read_b32 %{i}, a{a0 + i}\\n" ' for i in range(16))
            out.append(f"      case {qb * L.DBLK + db}: asm volatile({body}: {outs} :: {clob}); break;")
    out.append("      default: break;")
    out.append("    }")
    out.append("  }")
    out.append("};")
    return out


def main():
    lines = [
        "// Generated by gen_bound_stage.py -- do not edit by hand.",
        "// Instruction blocks of the bound-softmax attention kernel for gfx950; see",
        "// the generator for the register layout, the schedule and the hazard rules.",
        "#pragma once",
        "#include <hip/hip_runtime.h>",
        "#include <stdint.h>",
        "",
        "namespace bsvf {",
        "template <int D> struct BoundStage;",
        "",
    ]
    for D in (64, 128):
        lines += gen(D)
        lines.append("")
    lines.append("}  // namespace bsvf")
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")
    for D in (64, 128):
        L = Layout(D)
        print(f"D={D}: block VGPRs v{L.base}..v255 ({L.n_vgpr}), AGPRs {L.n_agpr}")


if __name__ == "__main__":
    main()
