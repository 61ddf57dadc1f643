"""Generate attn_fwd_asm.inc: the hand-scheduled program of one forward wave.

python gen_attn_fwd_asm.py            # writes attn_fwd_asm.inc beside this file
python gen_attn_fwd_asm.py --check    # exits 1 when the file is out of date

The forward kernel (attn_fwd_bf16.hip) runs this program as one inline-asm
block per wave: 32 queries of one (batch, head) against 64-key tiles that
stream through a three-stage LDS ring. Scheduling it by hand is what lets the
matrix cores, the vector ALU and the LDS work at once: the scores S^T = K Q^T
of tile j+1 are issued one MFMA at a time between the exponentials and the
row-sum adds of tile j, and the P V MFMAs of tile j between the conversions of
its second half. The lazy rescale is tested on each lane's sum of P over the
tile (against 2^8) and handled out of line. Compiled from C++, the same work
ran 2.4 times slower per tile (each MFMA waited on an LDS read issued just
before it, and the phases did not overlap).

The generator tracks the wait states the hardware leaves to software:
  * an MFMA result read (or overwritten) by a non-MFMA instruction: at least
    MFMA_RESULT_WAIT instructions after the MFMA;
  * a VALU result read by an MFMA: at least VALU_TO_MFMA_WAIT instructions;
  * LDS reads (s_waitcnt lgkmcnt) and tile loads (s_waitcnt vmcnt), counted
    in issue order.
Where the distance is short it inserts s_nop.

Register map (VGPR): v0-15 Q^T operands (4 k-steps); v16-47 / v48-79 the two
score buffers (S^T of a tile as two 32x32 C blocks); v80-87 K operand ring
(2); v88-95 V^T operand ring (2); v96-111 P^T operands (4); v112-143 O^T
accumulators (2 d blocks); v144 reference m (base 2, scaled); v145/v146 row
sum halves; v147 tile max (first tile and rescale blocks); v148/v149 the
lane's partial sums of P of the current tile, else temporaries; v150 -inf; v151 c (scale *
log2 e); v152-155 K read offsets (per k-step); v156-159 V^T read offsets
(d block, half); v160/161 tile-load offsets; v162 mask limit; v163 lane ^ 32
byte address for exchanges across the lane halves.
"""

from __future__ import annotations

import os
import sys

# Distances in instruction slots (an s_nop N fills N + 1): the compiler
# itself leaves 12 wait states between a 32x32x16 MFMA and a VALU read of its
# result, 2 between a VALU write and an MFMA read, and 1 between a
# transcendental and the VALU instruction that uses its result; the MFMA
# distance here keeps one slot of margin.
MFMA_RESULT_WAIT = 14
VALU_TO_MFMA_WAIT = 3
TRANS_WAIT = 2
TRANS_OPS = ("v_exp_f32", "v_log_f32", "v_rcp_f32")

Q, SA, SB, KR, VR, P, ACC = 0, 16, 48, 80, 88, 96, 112
M, L0, L1, MX, T0, T1, NINF, CREG = 144, 145, 146, 147, 148, 149, 150, 151
KOFF, VOFF, LDOFF, LIM, BPERM = 152, 156, 160, 162, 163
STAGE_BYTES = 8192
N_VGPR = 164

# fixed SGPRs: descriptor s[44:47], tile index j s48, temporaries s49/s50,
# next tile base s[52:53], bytes left from it s[54:55], records s56,
# saved exec s[58:59], second compare mask s[60:61]
SD, SJ, ST0, ST1, STB, SLEFT, SREC, SEXEC, SCMP = 44, 48, 49, 50, 52, 54, 56, 58, 60


def vt(base, n):
    return f"v[{base}:{base + n - 1}]"


class Prog:
    """Instruction stream with wait-state and wait-count bookkeeping."""

    def __init__(self):
        self.lines = []
        self.idx = 0          # slot position (s_nop N fills N + 1 slots)
        self.mfma_w = {}      # vgpr -> slot of the MFMA that last wrote it
        self.valu_w = {}      # vgpr -> slot of the VALU/memory op that last wrote it
        self.trans_w = {}     # vgpr -> slot of the transcendental that last wrote it
        self.lds = []         # outstanding LDS operations (tags), oldest first
        self.vmem_dst = set() # VGPRs a global load in flight will still write

    def _nop(self, n):
        while n > 0:
            k = min(n, 16)
            self.lines.append(f"s_nop {k - 1}")
            self.idx += k
            n -= k

    def emit(self, text, kind="salu", rd=(), wr=()):
        if text.startswith("s_waitcnt vmcnt(0)"):
            self.vmem_dst = set()
        touched = (set(rd) | set(wr)) & self.vmem_dst
        if touched:
            raise AssertionError(f"{text}: touches v{sorted(touched)} before their load lands")
        need = 0
        if kind != "mfma":
            for r in list(rd) + list(wr):
                if r in self.mfma_w:
                    need = max(need, self.mfma_w[r] + MFMA_RESULT_WAIT - self.idx)
        else:
            for r in list(rd) + list(wr):
                if r in self.valu_w:
                    need = max(need, self.valu_w[r] + VALU_TO_MFMA_WAIT - self.idx)
        if kind == "valu" and not text.startswith(TRANS_OPS):
            for r in rd:
                if r in self.trans_w:
                    need = max(need, self.trans_w[r] + TRANS_WAIT - self.idx)
        self._nop(need)
        self.lines.append(text)
        pos = self.idx
        self.idx += 1
        if kind == "vmem" and wr:
            self.vmem_dst |= set(wr)
        for r in wr:
            self.trans_w.pop(r, None)
            if kind == "mfma":
                self.mfma_w[r] = pos
                self.valu_w.pop(r, None)
            else:
                self.mfma_w.pop(r, None)
                self.valu_w[r] = pos
                if text.startswith(TRANS_OPS):
                    self.trans_w[r] = pos

    def label(self, name, align=False):
        if align:
            self.lines.append(".p2align 5")
        self.lines.append(f"{name}_%=:")

    def snapshot(self):
        return (dict(self.mfma_w), dict(self.valu_w), dict(self.trans_w), list(self.lds), self.idx)

    def restore(self, snap):
        self.mfma_w, self.valu_w, self.trans_w = dict(snap[0]), dict(snap[1]), dict(snap[2])
        self.lds = list(snap[3])
        # keep idx increasing: shift the restored slots to the current position
        shift = self.idx - snap[4]
        for d in (self.mfma_w, self.valu_w, self.trans_w):
            for r in d:
                d[r] += shift

    def join(self, snap):
        """Label reached both by falling through and by a branch taken at
        `snap`: every pending write is as recent as on either path."""
        shift = self.idx - snap[4]
        for mine, theirs in zip((self.mfma_w, self.valu_w, self.trans_w), snap[:3]):
            for r, pos in theirs.items():
                mine[r] = max(mine.get(r, pos + shift), pos + shift)
        assert self.lds == snap[3], "LDS queues differ at a join"

    def reset(self, recent=(), recent_valu=None):
        """Block start with predecessors the tracker did not follow: the
        registers in `recent` may have been written by MFMA or VALU just now
        (by VALU only for `recent_valu`, when given)."""
        self.mfma_w = {r: self.idx for r in recent}
        self.valu_w = {r: self.idx for r in (recent if recent_valu is None else
                                              list(recent) + list(recent_valu))}
        self.trans_w = {}
        assert not self.lds, "LDS operations outstanding at a block start"

    # -- helpers ---------------------------------------------------------
    def valu(self, text, rd=(), wr=()):
        self.emit(text, "valu", rd, wr)

    def lds_op(self, text, tag, rd=(), wr=()):
        self.emit(text, "lds", rd, wr)
        self.lds.append(tag)

    def wait_lds(self, tag):
        idx = [i for i, t in enumerate(self.lds) if t == tag]
        if not idx:
            return
        n = len(self.lds) - 1 - max(idx)
        self.emit(f"s_waitcnt lgkmcnt({min(n, 15)})")
        keep = min(n, 15)
        self.lds = self.lds[len(self.lds) - keep:] if keep else []

    def wait_lds_all(self):
        if self.lds:
            self.emit("s_waitcnt lgkmcnt(0)")
            self.lds = []

    def mfma(self, dst, a, b, c):
        rd = list(range(a, a + 4)) + list(range(b, b + 4))
        csrc = "0"
        if c is not None:
            rd += list(range(c, c + 16))
            csrc = vt(c, 16)
        self.emit(f"v_mfma_f32_32x32x16_bf16 {vt(dst, 16)}, {vt(a, 4)}, {vt(b, 4)}, {csrc}", "mfma",
                  rd, list(range(dst, dst + 16)))


# ---------------------------------------------------------------------------
# Lane address arithmetic, written once as a tiny program that both emits the
# VALU instructions and can be evaluated per lane in Python (for the check
# against the C++ formulas in the tests).
# ---------------------------------------------------------------------------
def lane_setup_ops():
    """(op, dst, srcs...) over symbolic registers; 'lane' is the lane id."""
    ops = [
        ("and", "l32", "lane", 31),
        ("shr", "hf", "lane", 5),
        ("bfe", "t_a", "l32", 1, 1),
        ("shl", "t_a", "t_a", 2),
        ("bfe", "t_b", "l32", 2, 2),
        ("or", "sw", "t_a", "t_b"),                 # swz(l32)
    ]
    for kk in range(4):                              # K row reads: koff[kk] (bytes)
        ops += [("add", f"x{kk}", "hf", 2 * kk),
                ("xor", f"x{kk}", f"x{kk}", "sw"),
                ("shl", f"x{kk}", f"x{kk}", 4),
                ("shladd", f"koff{kk}", "l32", 7, f"x{kk}")]   # l32*128 + x
    # transposed V reads: i = lane & 15, grp = lane >> 4, h = grp >> 1
    ops += [("and", "i", "lane", 15),
            ("shr", "grp", "lane", 4),
            ("shr", "h", "grp", 1),
            ("and", "g1", "grp", 1),
            ("and", "i3", "i", 3),
            ("shr", "i2", "i", 2),
            ("shladd", "r0", "h", 2, "i2"),             # 4h + (i >> 2)
            ("add", "r1", "r0", 8)]
    for half, r in ((0, "r0"), (1, "r1")):
        ops += [("bfe", f"sa{half}", r, 1, 1), ("shl", f"sa{half}", f"sa{half}", 2),
                ("bfe", f"sb{half}", r, 2, 2), ("or", f"sw{half}", f"sa{half}", f"sb{half}")]
    for db in range(2):
        # d = 32 db + 16 g1 + 4 i3; chunk = d >> 3 = 4 db + 2 g1 + (i3 >> 1); d & 7 = 4 (i3 & 1)
        ops += [("shr", f"c{db}", "i3", 1),
                ("shladd", f"c{db}", "g1", 1, f"c{db}"),
                ("add", f"c{db}", f"c{db}", 4 * db),
                ("and", f"e{db}", "i3", 1),
                ("shl", f"e{db}", f"e{db}", 3)]        # (d & 7) * 2 bytes
        for half, r in ((0, "r0"), (1, "r1")):
            nm = f"voff{db}{half}"
            ops += [("xor", nm, f"c{db}", f"sw{half}"),
                    ("shl", nm, nm, 4),
                    ("add", nm, nm, f"e{db}"),
                    ("shladd", nm, r, 7, nm)]            # r*128 + ...
    return ops


def eval_lane_setup(lane):
    """Evaluate lane_setup_ops for one lane (Python integers)."""
    env = {"lane": lane}
    val = lambda x: env[x] if isinstance(x, str) else x  # noqa: E731
    for op in lane_setup_ops():
        k, dst = op[0], op[1]
        a = [val(x) for x in op[2:]]
        if k == "and":
            env[dst] = a[0] & a[1]
        elif k == "shr":
            env[dst] = a[0] >> a[1]
        elif k == "shl":
            env[dst] = (a[0] << a[1]) & 0xFFFFFFFF
        elif k == "bfe":
            env[dst] = (a[0] >> a[1]) & ((1 << a[2]) - 1)
        elif k == "or":
            env[dst] = a[0] | a[1]
        elif k == "xor":
            env[dst] = a[0] ^ a[1]
        elif k == "add":
            env[dst] = (a[0] + a[1]) & 0xFFFFFFFF
        elif k == "shladd":
            env[dst] = ((a[0] << a[1]) + a[2]) & 0xFFFFFFFF
        else:
            raise ValueError(k)
    return env


def lane_halves(p, lane_reg):
    """l32 = lane & 31 and hf = lane >> 5 into the registers emit_lane_setup
    gives them (the first two of its scratch)."""
    l32, hf = SB, SB + 1
    p.valu(f"v_and_b32 v{l32}, 31, v{lane_reg}", [lane_reg], [l32])
    p.valu(f"v_lshrrev_b32 v{hf}, 5, v{lane_reg}", [lane_reg], [hf])
    return l32, hf


def emit_lane_setup(p, regmap, lane_reg):
    """Emit lane_setup_ops; symbolic names map to VGPRs through regmap (the
    final offsets) or to scratch VGPRs allocated from the score buffers."""
    scratch = list(range(SB, SB + 32))
    loc = dict(regmap)
    loc["lane"] = lane_reg

    def reg(x):
        if isinstance(x, int):
            return None
        if x not in loc:
            loc[x] = scratch.pop(0)
        return loc[x]

    def src(x):
        return str(x) if isinstance(x, int) else f"v{reg(x)}"

    for op in lane_setup_ops():
        k, dst = op[0], op[1]
        args = op[2:]
        d = reg(dst)
        rd = [reg(a) for a in args if isinstance(a, str)]
        if k == "and":
            p.valu(f"v_and_b32 v{d}, {src(args[1])}, {src(args[0])}", rd, [d])
        elif k == "shr":
            p.valu(f"v_lshrrev_b32 v{d}, {args[1]}, {src(args[0])}", rd, [d])
        elif k == "shl":
            p.valu(f"v_lshlrev_b32 v{d}, {args[1]}, {src(args[0])}", rd, [d])
        elif k == "bfe":
            p.valu(f"v_bfe_u32 v{d}, {src(args[0])}, {args[1]}, {args[2]}", rd, [d])
        elif k == "or":
            p.valu(f"v_or_b32 v{d}, {src(args[0])}, {src(args[1])}", rd, [d])
        elif k == "xor":
            p.valu(f"v_xor_b32 v{d}, {src(args[0])}, {src(args[1])}", rd, [d])
        elif k == "add":
            p.valu(f"v_add_u32 v{d}, {src(args[1])}, {src(args[0])}", rd, [d])
        elif k == "shladd":
            p.valu(f"v_lshl_add_u32 v{d}, {src(args[0])}, {args[1]}, {src(args[2])}", rd, [d])
    return loc


# ---------------------------------------------------------------------------
# Program pieces
# ---------------------------------------------------------------------------
def issue_tile(p, stage):
    """Direct buffer->LDS loads of the next K and V tile into `stage`."""
    p.emit(f"s_cmp_lg_u32 s{SLEFT + 1}, 0")
    p.emit(f"s_cselect_b32 s{SREC}, -1, s{SLEFT}")
    p.emit(f"s_mov_b32 s{SD}, s{STB}")
    p.emit(f"s_and_b32 s{SD + 1}, s{STB + 1}, 0xffff")
    p.emit(f"s_mov_b32 s{SD + 2}, s{SREC}")
    p.emit(f"s_mov_b32 s{SD + 3}, 0x20000")
    for i in range(2):
        p.emit(f"s_add_u32 m0, %[kldw], {stage * STAGE_BYTES + i * 1024}")
        p.emit(f"buffer_load_dwordx4 v{LDOFF + i}, s[{SD}:{SD + 3}], 0 offen lds", "vmem_lds",
               [LDOFF + i])
    for i in range(2):
        p.emit(f"s_add_u32 m0, %[vldw], {stage * STAGE_BYTES + i * 1024}")
        p.emit(f"buffer_load_dwordx4 v{LDOFF + i}, s[{SD}:{SD + 3}], %[voffs] offen lds", "vmem_lds",
               [LDOFF + i])
    p.emit(f"s_add_u32 s{STB}, s{STB}, %[tbytes]")
    p.emit(f"s_addc_u32 s{STB + 1}, s{STB + 1}, 0")
    p.emit(f"s_sub_u32 s{SLEFT}, s{SLEFT}, %[tbytes]")
    p.emit(f"s_subb_u32 s{SLEFT + 1}, s{SLEFT + 1}, 0")


def read_k(p, stage, f, slot_base=None):
    """K operand f (k-step kk = f // 2, key block kb = f % 2) of the tile in
    `stage` into the K ring slot f % 2 (or slot_base)."""
    kk, kb = f // 2, f % 2
    dst = KR + 4 * (f % 2) if slot_base is None else slot_base
    p.lds_op(f"ds_read_b128 {vt(dst, 4)}, v{KOFF + kk} offset:{stage * STAGE_BYTES + kb * 4096}",
             ("k", f), [KOFF + kk], list(range(dst, dst + 4)))
    return dst


def read_v(p, stage, g):
    """V^T operand g (key chunk kc = g // 2, d block db = g % 2) of the tile in
    `stage` into the V ring slot g % 2: two transposing 8-byte reads."""
    kc, db = g // 2, g % 2
    dst = VR + 4 * (g % 2)
    off = stage * STAGE_BYTES + kc * 2048
    p.lds_op(f"ds_read_b64_tr_b16 {vt(dst, 2)}, v{VOFF + 2 * db} offset:{off}", ("v", g),
             [VOFF + 2 * db], [dst, dst + 1])
    p.lds_op(f"ds_read_b64_tr_b16 {vt(dst + 2, 2)}, v{VOFF + 2 * db + 1} offset:{off}", ("v", g),
             [VOFF + 2 * db + 1], [dst + 2, dst + 3])
    return dst


def exps(p, s, elems):
    """P = exp2(c s - m) in place, two elements at a time (two FMAs, then
    the two exponentials)."""
    elems = list(elems)
    for k in range(0, len(elems), 2):
        pair = [s + e for e in elems[k:k + 2]]
        for r in pair:
            p.valu(f"v_fma_f32 v{r}, v{r}, v{CREG}, -v{M}", [r, CREG, M], [r])
        for r in pair:
            p.valu(f"v_exp_f32 v{r}, v{r}", [r], [r])


def cvt(p, s, kc, j):
    """P^T operand kc, register j: elements 16*(kc//2) + 8*(kc%2) + 2j, +1."""
    e0 = 16 * (kc // 2) + 8 * (kc % 2) + 2 * j
    p.valu(f"v_cvt_pk_bf16_f32 v{P + 4 * kc + j}, v{s + e0}, v{s + e0 + 1}", [s + e0, s + e0 + 1],
           [P + 4 * kc + j])


def mask_scores(p, s):
    """Key 32 kb + 8 (i // 4) + (i % 4) of the tile hides when it exceeds
    the lane's limit (query - first key of the tile - 4 hf)."""
    masks = ["vcc", f"s[{SCMP}:{SCMP + 1}]"]
    pend = []
    for e in range(32):
        kb, i = e // 16, e % 16
        idx = kb * 32 + 8 * (i // 4) + (i % 4)
        mreg = masks[e % 2]
        p.valu(f"v_cmp_gt_i32_e64 {mreg}, {idx}, v{LIM}", [LIM], [])
        pend.append((e, mreg))
        if len(pend) == 2:
            e0, m0 = pend.pop(0)
            p.valu(f"v_cndmask_b32_e64 v{s + e0}, v{s + e0}, v{NINF}, {m0}", [s + e0, NINF], [s + e0])
    e0, m0 = pend.pop(0)
    p.valu(f"v_cndmask_b32_e64 v{s + e0}, v{s + e0}, v{NINF}, {m0}", [s + e0, NINF], [s + e0])


def max_ops(s):
    """The 16 instructions of a tile's row max over this lane's 32 scores."""
    ops = [f"v_max3_f32 v{MX}, v{s}, v{s + 1}, v{s + 2}"]
    e = 3
    while e + 1 < 32:
        ops.append((e, e + 1))
        e += 2
    ops.append((31,))
    return ops


def emit_max_op(p, s, op):
    if isinstance(op, str):
        p.valu(op, [s, s + 1, s + 2], [MX])
    elif len(op) == 2:
        a, b = op
        p.valu(f"v_max3_f32 v{MX}, v{MX}, v{s + a}, v{s + b}", [MX, s + a, s + b], [MX])
    else:
        p.valu(f"v_max_f32 v{MX}, v{MX}, v{s + op[0]}", [MX, s + op[0]], [MX])


def max_tail(p, name):
    """Row max across the lane halves, then the lazy rescale: a row moves its
    reference m only when its tile max exceeds m by more than 8 (base 2);
    then l and O scale by 2^(m - m_new)."""
    p.lds_op(f"ds_bpermute_b32 v{T0}, v{BPERM}, v{MX}", ("bperm",), [BPERM, MX], [T0])
    p.wait_lds(("bperm",))
    p.valu(f"v_max_f32 v{MX}, v{MX}, v{T0}", [MX, T0], [MX])
    p.valu(f"v_mul_f32 v{MX}, v{MX}, v{CREG}", [MX, CREG], [MX])
    p.valu(f"v_add_f32 v{T0}, 0x41000000, v{M}", [M], [T0])
    p.valu(f"v_cmp_gt_f32 vcc, v{MX}, v{T0}", [MX, T0], [])
    snap = p.snapshot()
    p.emit(f"s_cbranch_vccz {name}_%=")
    # rows that keep their m scale by exactly 1 (also while m is still -inf)
    p.valu(f"v_cndmask_b32 v{T1}, v{M}, v{MX}, vcc", [M, MX], [T1])
    p.valu(f"v_sub_f32 v{T0}, v{M}, v{T1}", [M, T1], [T0])
    p.valu(f"v_exp_f32 v{T0}, v{T0}", [T0], [T0])
    p.valu(f"v_cndmask_b32 v{T0}, 1.0, v{T0}, vcc", [T0], [T0])
    p.valu(f"v_mul_f32 v{L0}, v{L0}, v{T0}", [L0, T0], [L0])
    p.valu(f"v_mul_f32 v{L1}, v{L1}, v{T0}", [L1, T0], [L1])
    for r in range(ACC, ACC + 32):
        p.valu(f"v_mul_f32 v{r}, v{r}, v{T0}", [r, T0], [r])
    p.valu(f"v_mov_b32 v{M}, v{T1}", [T1], [M])
    p.label(name)
    p.join(snap)


# The rescale test. After the exponentials of a tile with the row's current
# reference m, each lane sums its 32 P values: if no sum exceeds 2^8, no P
# does, and the tile needs nothing more. Otherwise (rarely: a row's scores
# grew past its reference) the program leaves the straight path for a block
# that recomputes the tile's scores, takes the row max, moves m and rescales
# l and O for the rows whose sums exceeded 2^8 (in either lane half), and
# redoes the exponentials. Rows that did not trigger recompute bit-identical
# values with their unchanged m and scale by exactly 1, so a row's arithmetic
# never depends on the other rows of the wave.
SUM_LIMIT = "0x43800000"   # 256.0
REDO = []                   # out-of-line blocks, emitted after the epilogue


def sums_into(p, cur, elems):
    for e in elems:
        t = T0 if e % 2 == 0 else T1
        p.valu(f"v_add_f32 v{t}, v{t}, v{cur + e}", [t, cur + e], [t])


def rescale_check(p, r, cur, kind):
    """The test and its out-of-line block; returns with L updated."""
    p.valu(f"v_add_f32 v{T0}, v{T0}, v{T1}", [T0, T1], [T0])
    p.valu(f"v_cmp_lt_f32 vcc, {SUM_LIMIT}, v{T0}", [T0], [])
    name = f"fwd_redo{kind}{r}"
    snap = p.snapshot()
    p.emit(f"s_cbranch_vccnz {name}_%=")
    REDO.append((name, r, cur, kind, snap))
    p.label(f"{name}_ret")
    # the block's last writes before it branches back are VALU (its score
    # MFMAs lie far behind); the LDS queue of the straight path is kept,
    # which only over-counts after the block has drained it
    for reg in (list(range(cur, cur + 32)) + list(range(ACC, ACC + 32)) +
                list(range(P, P + 16)) + [M, L0, L1, T0, T1]):
        p.valu_w[reg] = p.idx
        p.trans_w.pop(reg, None)
    p.valu(f"v_add_f32 v{L0}, v{L0}, v{T0}", [L0, T0], [L0])


def redo_block(p, name, r, cur, kind, snap):
    """Recompute the tile's scores (K of tile j is still in its stage), mask
    them on the diagonal tile, move m for the rows that triggered, rescale,
    and redo the exponentials, the sums and the P operands made before the
    test. T0 holds the lane's sum on entry."""
    st = r % 3
    p.restore(snap)
    p.label(name)
    for f in range(8):
        kk, kb = f // 2, f % 2
        read_k(p, st, f)
        p.wait_lds(("k", f))
        p.mfma(cur + 16 * kb, KR + 4 * (f % 2), Q + 4 * kk, None if kk == 0 else cur + 16 * kb)
    p.lds_op(f"ds_bpermute_b32 v{T1}, v{BPERM}, v{T0}", ("rb",), [BPERM, T0], [T1])
    if kind == "final":
        mask_scores(p, cur)
    # rows to move: this lane's sum or its partner's exceeded the limit
    flag = f"s[{SCMP}:{SCMP + 1}]"
    p.valu(f"v_cmp_lt_f32 vcc, {SUM_LIMIT}, v{T0}", [T0], [])
    p.emit(f"s_mov_b64 {flag}, vcc")
    p.wait_lds(("rb",))
    p.valu(f"v_cmp_lt_f32 vcc, {SUM_LIMIT}, v{T1}", [T1], [])
    p.emit(f"s_or_b64 {flag}, {flag}, vcc")
    for op in max_ops(cur):
        emit_max_op(p, cur, op)
    p.lds_op(f"ds_bpermute_b32 v{T0}, v{BPERM}, v{MX}", ("bperm",), [BPERM, MX], [T0])
    p.wait_lds(("bperm",))
    p.valu(f"v_max_f32 v{MX}, v{MX}, v{T0}", [MX, T0], [MX])
    p.valu(f"v_mul_f32 v{MX}, v{MX}, v{CREG}", [MX, CREG], [MX])
    # m_new = max(m, tile max) on the rows that triggered, m elsewhere
    p.valu(f"v_max_f32 v{T0}, v{M}, v{MX}", [M, MX], [T0])
    p.valu(f"v_cndmask_b32_e64 v{T1}, v{M}, v{T0}, {flag}", [M, T0], [T1])
    p.valu(f"v_sub_f32 v{T0}, v{M}, v{T1}", [M, T1], [T0])
    p.valu(f"v_exp_f32 v{T0}, v{T0}", [T0], [T0])
    p.valu(f"v_cndmask_b32_e64 v{T0}, 1.0, v{T0}, {flag}", [T0], [T0])
    p.valu(f"v_mul_f32 v{L0}, v{L0}, v{T0}", [L0, T0], [L0])
    p.valu(f"v_mul_f32 v{L1}, v{L1}, v{T0}", [L1, T0], [L1])
    for reg in range(ACC, ACC + 32):
        p.valu(f"v_mul_f32 v{reg}, v{reg}, v{T0}", [reg, T0], [reg])
    p.valu(f"v_mov_b32 v{M}, v{T1}", [T1], [M])
    exps(p, cur, range(32))
    p.valu(f"v_mov_b32 v{T0}, 0", [], [T0])
    p.valu(f"v_mov_b32 v{T1}, 0", [], [T1])
    sums_into(p, cur, range(32))
    p.valu(f"v_add_f32 v{T0}, v{T0}, v{T1}", [T0, T1], [T0])
    n_cvt = 4 if kind == "final" else 2
    for kc in range(n_cvt):
        for j in range(4):
            cvt(p, cur, kc, j)
    p.wait_lds_all()
    p.emit(f"s_branch {name}_ret_%=")


def pipelined_step(p, r, masked_next):
    """Tile j (scores in cur) with the scores of tile j+1 (into nxt)."""
    cur, nxt = (SA, SB) if r % 2 == 0 else (SB, SA)
    st_v, st_k = r % 3, (r + 1) % 3
    p.valu(f"v_mov_b32 v{T0}, 0", [], [T0])
    p.valu(f"v_mov_b32 v{T1}, 0", [], [T1])
    # K operands 0, 1 of tile j+1, then four exponentials while they land
    read_k(p, st_k, 0)
    read_k(p, st_k, 1)
    exps(p, cur, range(0, 4))
    for f in range(8):
        kk, kb = f // 2, f % 2
        p.wait_lds(("k", f))
        p.mfma(nxt + 16 * kb, KR + 4 * (f % 2), Q + 4 * kk, None if kk == 0 else nxt + 16 * kb)
        if f < 6:
            read_k(p, st_k, f + 2)
        else:
            read_v(p, st_v, f - 6)
        if f < 7:
            exps(p, cur, range(4 + 4 * f, 8 + 4 * f))
        sums_into(p, cur, range(4 * f, 4 * f + 4))
    for kc in range(2):
        for j in range(4):
            cvt(p, cur, kc, j)
    rescale_check(p, r, cur, "m" if masked_next else "p")
    if masked_next:
        mask_scores(p, nxt)
    cv = [(kc, j) for kc in (2, 3) for j in range(4)]
    for g in range(8):
        kc, db = g // 2, g % 2
        p.wait_lds(("v", g))
        p.mfma(ACC + 16 * db, VR + 4 * (g % 2), P + 4 * kc, ACC + 16 * db)
        if g < 6:
            read_v(p, st_v, g + 2)
        for _ in range(2):
            if cv:
                cvt(p, cur, *cv.pop(0))
    p.wait_lds_all()


def final_step(p, r):
    """The wave's last tile: exponentials, the row sum and P V; no next tile."""
    cur = SA if r % 2 == 0 else SB
    st_v = r % 3
    p.valu(f"v_mov_b32 v{T0}, 0", [], [T0])
    p.valu(f"v_mov_b32 v{T1}, 0", [], [T1])
    read_v(p, st_v, 0)
    read_v(p, st_v, 1)
    exps(p, cur, range(32))
    sums_into(p, cur, range(32))
    for kc in range(4):
        for j in range(4):
            cvt(p, cur, kc, j)
    rescale_check(p, r, cur, "final")
    for g in range(8):
        kc, db = g // 2, g % 2
        p.wait_lds(("v", g))
        p.mfma(ACC + 16 * db, VR + 4 * (g % 2), P + 4 * kc, ACC + 16 * db)
        if g < 6:
            read_v(p, st_v, g + 2)
    p.wait_lds_all()


def program():
    p = Prog()
    REDO.clear()
    acc_regs = list(range(ACC, ACC + 32))
    # ---- lane setup (temporaries live in the second score buffer) ----------
    lane = 163
    p.valu(f"v_mbcnt_lo_u32_b32 v{lane}, -1, 0", [], [lane])
    p.valu(f"v_mbcnt_hi_u32_b32 v{lane}, -1, v{lane}", [lane], [lane])
    # l32 and hf first (the lane arithmetic below recomputes them in place),
    # so that the loads go out before the rest of the lane arithmetic
    l32, hf = lane_halves(p, lane)
    # tile loads: row tr = 16 wave + 8 i + (lane >> 3), chunk (lane & 7) ^ swz(tr)
    t_lane3, t_tr, t_sw, t_x, t_qo = SB + 27, SB + 28, SB + 29, SB + 30, SB + 31
    p.valu(f"v_lshrrev_b32 v{t_lane3}, 3, v{lane}", [lane], [t_lane3])
    for i in range(2):
        p.valu(f"v_add_u32 v{t_tr}, %[wave16], v{t_lane3}", [t_lane3], [t_tr])
        if i:
            p.valu(f"v_add_u32 v{t_tr}, 8, v{t_tr}", [t_tr], [t_tr])
        p.valu(f"v_bfe_u32 v{t_sw}, v{t_tr}, 1, 1", [t_tr], [t_sw])
        p.valu(f"v_lshlrev_b32 v{t_sw}, 2, v{t_sw}", [t_sw], [t_sw])
        p.valu(f"v_bfe_u32 v{t_x}, v{t_tr}, 2, 2", [t_tr], [t_x])
        p.valu(f"v_or_b32 v{t_sw}, v{t_sw}, v{t_x}", [t_sw, t_x], [t_sw])
        p.valu(f"v_and_b32 v{t_x}, 7, v{lane}", [lane], [t_x])
        p.valu(f"v_xor_b32 v{t_x}, v{t_x}, v{t_sw}", [t_x, t_sw], [t_x])
        p.valu(f"v_lshlrev_b32 v{t_x}, 4, v{t_x}", [t_x], [t_x])
        p.valu(f"v_mul_lo_u32 v{LDOFF + i}, v{t_tr}, %[rs2]", [t_tr], [LDOFF + i])
        p.valu(f"v_add_u32 v{LDOFF + i}, v{LDOFF + i}, v{t_x}", [LDOFF + i, t_x], [LDOFF + i])
    # mask limit: (first query of the wave - first key of its last tile) + l32 - 4 hf
    p.valu(f"v_lshlrev_b32 v{LIM}, 2, v{hf}", [hf], [LIM])
    p.valu(f"v_sub_u32 v{LIM}, v{l32}, v{LIM}", [l32, LIM], [LIM])
    p.valu(f"v_add_u32 v{LIM}, %[limb], v{LIM}", [LIM], [LIM])
    # Q: byte offset l32 * row stride + 16 hf from the wave's first query row
    p.valu(f"v_mul_lo_u32 v{t_qo}, v{l32}, %[rs2]", [l32], [t_qo])
    p.valu(f"v_lshl_add_u32 v{t_qo}, v{hf}, 4, v{t_qo}", [hf, t_qo], [t_qo])
    # ---- first two tiles ----------------------------------------------------
    p.emit(f"s_mov_b32 s{STB}, %[kat_lo]")
    p.emit(f"s_mov_b32 s{STB + 1}, %[kat_hi]")
    p.emit(f"s_mov_b32 s{SLEFT}, %[kleft_lo]")
    p.emit(f"s_mov_b32 s{SLEFT + 1}, %[kleft_hi]")
    issue_tile(p, 0)
    p.emit("s_cmp_lt_u32 1, %[nkt]")
    p.emit("s_cbranch_scc0 fwd_one_tile_%=")
    issue_tile(p, 1)
    p.label("fwd_one_tile")
    # ---- Q (zeros for queries past the sequence), constants, accumulators ---
    for r in range(Q, Q + 16):
        p.valu(f"v_mov_b32 v{r}, 0", [], [r])
    p.valu(f"v_cmp_gt_i32 vcc, %[nq], v{l32}", [l32], [])
    p.emit(f"s_and_saveexec_b64 s[{SEXEC}:{SEXEC + 1}], vcc")
    for kk in range(4):
        p.emit(f"global_load_dwordx4 {vt(Q + 4 * kk, 4)}, v{t_qo}, %[qbase] offset:{32 * kk}", "vmem",
               [t_qo], list(range(Q + 4 * kk, Q + 4 * kk + 4)))
    p.emit(f"s_mov_b64 exec, s[{SEXEC}:{SEXEC + 1}]")
    # the rest of the lane arithmetic while the loads are in flight
    regs = {f"koff{kk}": KOFF + kk for kk in range(4)}
    regs.update({f"voff{db}{h}": VOFF + 2 * db + h for db in range(2) for h in range(2)})
    loc = emit_lane_setup(p, regs, lane)
    assert (loc["l32"], loc["hf"]) == (l32, hf)
    for kk in range(4):
        p.valu(f"v_add_u32 v{KOFF + kk}, %[klds], v{KOFF + kk}", [KOFF + kk], [KOFF + kk])
    for k in range(4):
        p.valu(f"v_add_u32 v{VOFF + k}, %[vlds], v{VOFF + k}", [VOFF + k], [VOFF + k])
    p.valu(f"v_xor_b32 v{BPERM}, 32, v{lane}", [lane], [BPERM])
    p.valu(f"v_lshlrev_b32 v{BPERM}, 2, v{BPERM}", [BPERM], [BPERM])
    p.valu(f"v_mov_b32 v{NINF}, 0xff800000", [], [NINF])
    p.valu(f"v_mov_b32 v{M}, 0xff800000", [], [M])
    p.valu(f"v_mov_b32 v{L0}, 0", [], [L0])
    p.valu(f"v_mov_b32 v{L1}, 0", [], [L1])
    p.valu(f"v_mov_b32 v{CREG}, %[cbits]", [], [CREG])
    for r in acc_regs:
        p.valu(f"v_mov_b32 v{r}, 0", [], [r])
    p.emit("s_waitcnt vmcnt(0)")
    p.emit("s_barrier")
    # ---- scores of tile 0 (stage 0), operands staged in the other buffer ----
    for f in range(8):
        read_k(p, 0, f, slot_base=SB + 4 * f)
    for f in range(8):
        kk, kb = f // 2, f % 2
        p.wait_lds(("k", f))
        p.mfma(SA + 16 * kb, SB + 4 * f, Q + 4 * kk, None if kk == 0 else SA + 16 * kb)
    p.emit("s_cmp_eq_u32 %[jlast], 0")
    snap = p.snapshot()
    p.emit("s_cbranch_scc0 fwd_first_nomask_%=")
    mask_scores(p, SA)
    p.label("fwd_first_nomask")
    p.join(snap)
    for op in max_ops(SA):
        emit_max_op(p, SA, op)
    max_tail(p, "fwd_first_rescaled")
    p.emit(f"s_mov_b32 s{SJ}, 0")
    # ---- tile loop, unrolled by 6 (stage = j % 3, score buffer = j % 2) ----
    # Every path into a step label leaves no LDS operation outstanding; the
    # accumulators may have just been written (by MFMA or by a rescale).
    for r in range(6):
        p.label(f"fwd_step{r}", align=True)
        p.reset(acc_regs)
        p.emit("s_waitcnt vmcnt(0)")
        p.emit("s_barrier")
        p.emit(f"s_add_u32 s{ST0}, s{SJ}, 2")
        p.emit(f"s_cmp_lt_u32 s{ST0}, %[nkt]")
        p.emit(f"s_cbranch_scc0 fwd_noissue{r}_%=")
        issue_tile(p, (r + 2) % 3)
        p.label(f"fwd_noissue{r}")
        p.emit(f"s_cmp_lt_u32 s{SJ}, %[jlast]")
        p.emit(f"s_cbranch_scc1 fwd_pipe{r}_%=")
        p.emit(f"s_cmp_eq_u32 s{SJ}, %[jlast]")
        p.emit(f"s_cbranch_scc1 fwd_final{r}_%=")
        p.emit(f"s_branch fwd_next{r}_%=")
        dispatch = p.snapshot()
        # pipelined step; the next tile is the diagonal one when j + 1 = j_last
        p.label(f"fwd_pipe{r}", align=True)
        p.emit(f"s_add_u32 s{ST0}, s{SJ}, 1")
        p.emit(f"s_cmp_eq_u32 s{ST0}, %[jlast]")
        p.emit(f"s_cbranch_scc1 fwd_pipem{r}_%=")
        pipelined_step(p, r, False)
        p.emit(f"s_branch fwd_next{r}_%=")
        p.restore(dispatch)
        p.label(f"fwd_pipem{r}", align=True)
        pipelined_step(p, r, True)
        p.emit(f"s_branch fwd_next{r}_%=")
        p.restore(dispatch)
        p.label(f"fwd_final{r}", align=True)
        final_step(p, r)
        p.label(f"fwd_next{r}")
        p.reset(acc_regs)
        p.emit(f"s_add_u32 s{SJ}, s{SJ}, 1")
        p.emit(f"s_cmp_lt_u32 s{SJ}, %[nkt]")
        p.emit(f"s_cbranch_scc1 fwd_step{(r + 1) % 6}_%=")
        p.emit("s_branch fwd_done_%=")
    # ---- epilogue: O = acc / l, LSE = ln 2 (m + log2 l) ----------------------
    p.label("fwd_done")
    p.reset(acc_regs)
    t_out = SB                   # packed bf16 outputs: SB .. SB + 15
    e_lane, e_l32, e_hf, t_oo = SB + 16, SB + 17, SB + 18, SB + 19
    p.valu(f"v_add_f32 v{L0}, v{L0}, v{L1}", [L0, L1], [L0])
    p.lds_op(f"ds_bpermute_b32 v{T0}, v{BPERM}, v{L0}", ("bperm",), [BPERM, L0], [T0])
    p.valu(f"v_mbcnt_lo_u32_b32 v{e_lane}, -1, 0", [], [e_lane])
    p.valu(f"v_mbcnt_hi_u32_b32 v{e_lane}, -1, v{e_lane}", [e_lane], [e_lane])
    p.valu(f"v_and_b32 v{e_l32}, 31, v{e_lane}", [e_lane], [e_l32])
    p.valu(f"v_lshrrev_b32 v{e_hf}, 5, v{e_lane}", [e_lane], [e_hf])
    p.valu(f"v_mul_lo_u32 v{t_oo}, v{e_l32}, %[c2]", [e_l32], [t_oo])
    p.valu(f"v_lshl_add_u32 v{t_oo}, v{e_hf}, 3, v{t_oo}", [e_hf, t_oo], [t_oo])
    p.wait_lds(("bperm",))
    p.valu(f"v_add_f32 v{L0}, v{L0}, v{T0}", [L0, T0], [L0])
    p.valu(f"v_rcp_f32 v{T1}, v{L0}", [L0], [T1])
    p.valu(f"v_log_f32 v{T0}, v{L0}", [L0], [T0])
    p.valu(f"v_add_f32 v{T0}, v{M}, v{T0}", [M, T0], [T0])
    p.valu(f"v_mul_f32 v{T0}, 0x3f317218, v{T0}", [T0], [T0])       # ln 2
    for db in range(2):
        for g in range(4):
            base = ACC + 16 * db + 4 * g
            for k in range(4):
                p.valu(f"v_mul_f32 v{base + k}, v{base + k}, v{T1}", [base + k, T1], [base + k])
            o = t_out + 2 * (4 * db + g)
            p.valu(f"v_cvt_pk_bf16_f32 v{o}, v{base}, v{base + 1}", [base, base + 1], [o])
            p.valu(f"v_cvt_pk_bf16_f32 v{o + 1}, v{base + 2}, v{base + 3}", [base + 2, base + 3],
                   [o + 1])
    p.valu(f"v_cmp_gt_i32 vcc, %[nq], v{e_l32}", [e_l32], [])
    p.emit(f"s_and_saveexec_b64 s[{SEXEC}:{SEXEC + 1}], vcc")
    for db in range(2):
        for g in range(4):
            o = t_out + 2 * (4 * db + g)
            p.emit(f"global_store_dwordx2 v{t_oo}, {vt(o, 2)}, %[obase] offset:{(32 * db + 8 * g) * 2}",
                   "vmem", [t_oo, o, o + 1], [])
    p.emit(f"s_mov_b64 exec, s[{SEXEC}:{SEXEC + 1}]")
    p.valu(f"v_cmp_gt_i32 vcc, %[nlse], v{e_lane}", [e_lane], [])
    p.emit(f"s_and_saveexec_b64 s[{SEXEC}:{SEXEC + 1}], vcc")
    p.valu(f"v_lshlrev_b32 v{T1}, 2, v{e_l32}", [e_l32], [T1])
    p.emit(f"global_store_dword v{T1}, v{T0}, %[lbase]", "vmem", [T1, T0], [])
    p.emit(f"s_mov_b64 exec, s[{SEXEC}:{SEXEC + 1}]")
    # ---- the rescale blocks, out of line ----------------------------------------
    p.emit("s_branch fwd_exit_%=")
    for blk in list(REDO):
        redo_block(p, *blk)
    p.label("fwd_exit")
    return p.lines


def render(lines):
    body = "\n".join(f'    "{ln}\\n"' for ln in lines)
    clob_v = ", ".join(f'"v{i}"' for i in range(N_VGPR))
    clob_s = ", ".join(f'"s{i}"' for i in range(44, 62))
    return (
        "// Generated by gen_attn_fwd_asm.py; do not edit by hand.\n"
        "// The program of one forward wave (see the generator for the register map).\n"
        f"#define CATTN_FWD_ASM_BODY \\\n{body.replace(chr(10), ' ' + chr(92) + chr(10))}\n"
        f"#define CATTN_FWD_ASM_CLOBBERS {clob_v}, {clob_s}\n"
    )


def main(argv):
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "attn_fwd_asm.inc")
    text = render(program())
    if "--check" in argv:
        ok = os.path.exists(path) and open(path).read() == text
        print("up to date" if ok else "attn_fwd_asm.inc is out of date: run gen_attn_fwd_asm.py")
        return 0 if ok else 1
    with open(path, "w") as fh:
        fh.write(text)
    print(f"wrote {path} ({len(program())} instructions)")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
