"""Generate attn_dkdv_asm.inc: the hand-scheduled program of one dK/dV wave.

python gen_attn_dkdv_asm.py            # writes attn_dkdv_asm.inc beside this file
python gen_attn_dkdv_asm.py --check    # exits 1 when the file is out of date

A wave owns 32 keys of one (batch, head), with K and V of its keys in
registers, and walks the query tiles (64 rows: Q, dO and the MFMA terms of
8 LSE and D) that stream through a three-stage LDS ring. Each tile is two
halves of 32 queries, and each half goes through three phases:
  1. S - 8 LSE and dP - D on MFMA (10 MFMAs: four k-steps over d for each,
     then one over the row's terms);
  2. P = exp2(c (S - 8 LSE)) and dS = P (dP - D) on the VALU, rounded to
     bf16 operands (with the causal mask on the wave's first tile);
  3. dV^T += dO^T P and dK^T += Q^T dS on MFMA (8 MFMAs, the transposed
     operands read from the row-major tiles).
The program runs them as a pipeline over halves: slot k issues phase 3 of
half k-1 and phase 1 of half k+1 on MFMA (18 MFMAs) while phase 2 of half k
runs on the VALU between them, with every LDS operand read a few MFMAs
ahead through register rings. One barrier per tile, between the two slots
of the tile, publishes the next tile and frees the stage refilled next.

Waves 0 and 1 of a workgroup start at its first tile; waves 2 and 3, whose
keys follow every query of that tile, start at the second. A wave's first
tile holds its diagonal: its two halves are masked (the half before the
diagonal entirely, for waves 1 and 3).

Register map (VGPR): v0-15 K operands, v16-31 V operands, v32-63 / v64-95
S and dP of even / odd halves, v96-111 P and dS operands, v112-127 row
operand ring (4), v128-131 terms operand, v132-147 transposed operand ring
(4), v148-151 row read offsets, v152-155 transposed read offsets, v156 terms
read offset, v157-158 Q tile-load offsets, v159-160 dO tile-load offsets,
v161 terms load offset, v162-165 / v166-169 the terms k-step's B operands
for S / dP, v170 c, v171 mask limit, v172-173 temporaries, v174-237 the
accumulators dV^T (d blocks 0, 1), dK^T (d blocks 0, 1).
"""

from __future__ import annotations

import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

from gen_attn_fwd_asm import Prog, emit_lane_setup, lane_halves, vt  # noqa: E402

KREG, VREG, SD0, SD1, PDS = 0, 16, 32, 64, 96
ROW, TERMS, TR = 112, 128, 132
ROFF, TROFF, TOFF, LDQ, LDG, LDT = 148, 152, 156, 157, 159, 161
BS, BD, CREG, LIM, T0, T1 = 162, 166, 170, 171, 172, 173
DV, DK = 174, 206          # dV^T: 174-205 (d block 0, 1); dK^T: 206-237
N_VGPR = 238

Q_OFF, G_OFF, T_OFF = 0, 24576, 49152   # LDS regions (bytes from the Q base)
STAGE, TSTAGE = 8192, 2048

# SGPRs: Q descriptor s[44:47], dO descriptor s[48:51], next Q tile base
# s[52:53] and bytes left s[54:55], the same for dO s[56:57] / s[58:59], terms
# base s[60:61], tile index s62, temporary s63, saved exec s[64:65], second
# compare mask s[66:67]
SQD, SGD, SQB, SQL, SGB, SGL, STB, SJ, ST, SEXEC, SCMP = 44, 48, 52, 54, 56, 58, 60, 62, 63, 64, 66


def sd_regs(buf):
    base = SD0 if buf == 0 else SD1
    return base, base + 16          # S, dP


# ---------------------------------------------------------------------------
# Tile loads
# ---------------------------------------------------------------------------
def build_desc(p, d, base, left):
    p.emit(f"s_cmp_lg_u32 s{left + 1}, 0")
    p.emit(f"s_cselect_b32 s{d + 2}, -1, s{left}")
    p.emit(f"s_mov_b32 s{d}, s{base}")
    p.emit(f"s_and_b32 s{d + 1}, s{base + 1}, 0xffff")
    p.emit(f"s_mov_b32 s{d + 3}, 0x20000")


def advance(p, base, left, step):
    p.emit(f"s_add_u32 s{base}, s{base}, {step}")
    p.emit(f"s_addc_u32 s{base + 1}, s{base + 1}, 0")
    p.emit(f"s_sub_u32 s{left}, s{left}, {step}")
    p.emit(f"s_subb_u32 s{left + 1}, s{left + 1}, 0")


def issue_tile(p, stage, name):
    """Q and dO rows of the next tile into `stage`; waves 0 and 1 also load
    the tile's 2 KB of terms (1 KB each)."""
    build_desc(p, SQD, SQB, SQL)
    build_desc(p, SGD, SGB, SGL)
    for i in range(2):
        p.emit(f"s_add_u32 m0, %[qldw], {Q_OFF + stage * STAGE + i * 1024}")
        p.emit(f"buffer_load_dwordx4 v{LDQ + i}, s[{SQD}:{SQD + 3}], 0 offen lds", "vmem_lds",
               [LDQ + i])
    for i in range(2):
        p.emit(f"s_add_u32 m0, %[qldw], {G_OFF + stage * STAGE + i * 1024}")
        p.emit(f"buffer_load_dwordx4 v{LDG + i}, s[{SGD}:{SGD + 3}], 0 offen lds", "vmem_lds",
               [LDG + i])
    advance(p, SQB, SQL, "%[qtb]")
    advance(p, SGB, SGL, "%[gtb]")
    p.emit("s_cmp_lt_u32 %[wave], 2")
    snap = p.snapshot()
    p.emit(f"s_cbranch_scc0 {name}_%=")
    p.emit(f"s_add_u32 m0, %[tldw], {T_OFF + stage * TSTAGE}")
    p.emit(f"global_load_lds_dwordx4 v{LDT}, s[{STB}:{STB + 1}]", "vmem_lds", [LDT])
    p.label(name)
    p.join(snap)
    p.emit(f"s_add_u32 s{STB}, s{STB}, {TSTAGE}")
    p.emit(f"s_addc_u32 s{STB + 1}, s{STB + 1}, 0")


def barrier_point(p, t_issue_stage, name):
    """Tile t+1 has landed everywhere and every wave has left tile t-1:
    wait, meet, then load tile t+2 into the stage tile t-1 held."""
    p.emit("s_waitcnt vmcnt(0)")
    p.emit("s_barrier")
    p.emit(f"s_add_u32 s{ST}, s{SJ}, 2")
    p.emit(f"s_cmp_lt_u32 s{ST}, %[nit]")
    snap = p.snapshot()
    p.emit(f"s_cbranch_scc0 {name}_%=")
    issue_tile(p, t_issue_stage, name + "t")
    p.label(name)
    p.join(snap)


# ---------------------------------------------------------------------------
# One slot: phase 3 of one half, phase 1 of another on MFMA, phase 2 of a
# third on the VALU between them.
# ---------------------------------------------------------------------------
class Read:
    def __init__(self, tag, ops, dst):
        self.tag, self.ops, self.dst = tag, ops, dst


def phase1_plan(stage, qb, buf):
    """MFMAs and operand reads of S - 8 LSE and dP - D of a half."""
    s, dp = sd_regs(buf)
    mf, reads = [], []
    slot = 0
    for kk in range(4):
        for which, (off, breg, acc) in enumerate(((Q_OFF, KREG, s), (G_OFF, VREG, dp))):
            dst = ROW + 4 * (slot % 4)
            tag = ("row", stage, qb, kk, which)
            reads.append(Read(tag, [(f"ds_read_b128 {vt(dst, 4)}, v{ROFF + kk} offset:"
                                     f"{off + stage * STAGE + qb * 4096}", [ROFF + kk],
                                     list(range(dst, dst + 4)))], dst))
            mf.append((acc, dst, breg + 4 * kk, None if kk == 0 else acc, tag))
            slot += 1
    tag = ("terms", stage, qb)
    reads.append(Read(tag, [(f"ds_read_b128 {vt(TERMS, 4)}, v{TOFF} offset:"
                             f"{T_OFF + stage * TSTAGE + qb * 1024}", [TOFF],
                             list(range(TERMS, TERMS + 4)))], TERMS))
    mf.append((s, TERMS, BS, s, tag))
    mf.append((dp, TERMS, BD, dp, tag))
    return mf, reads


def phase3_plan(stage, qb):
    """MFMAs and transposed operand reads of dV^T += dO^T P, dK^T += Q^T dS."""
    mf, reads = [], []
    slot = 0
    for db in range(2):
        for j in range(2):
            kc = 2 * qb + j
            for which, (off, pd, acc) in enumerate(((G_OFF, PDS + 4 * j, DV + 16 * db),
                                                    (Q_OFF, PDS + 8 + 4 * j, DK + 16 * db))):
                dst = TR + 4 * (slot % 4)
                tag = ("tr", stage, qb, db, j, which)
                o = off + stage * STAGE + kc * 2048
                reads.append(Read(tag, [
                    (f"ds_read_b64_tr_b16 {vt(dst, 2)}, v{TROFF + 2 * db} offset:{o}",
                     [TROFF + 2 * db], [dst, dst + 1]),
                    (f"ds_read_b64_tr_b16 {vt(dst + 2, 2)}, v{TROFF + 2 * db + 1} offset:{o}",
                     [TROFF + 2 * db + 1], [dst + 2, dst + 3])], dst))
                mf.append((acc, dst, pd, acc, tag))
                slot += 1
    return mf, reads


def phase2_ops(buf, mask):
    """VALU work of a half: optional mask, then P, dS; the 16 conversions
    come separately (they overwrite the operands phase 3 reads)."""
    s, dp = sd_regs(buf)
    ops = []
    if mask is not None:
        masks = ["vcc", f"s[{SCMP}:{SCMP + 1}]"]
        pend = []
        for i in range(16):
            idx = 8 * (i // 4) + (i % 4) + mask
            m = masks[i % 2]
            ops.append((f"v_cmp_lt_i32_e64 {m}, {idx}, v{LIM}", [LIM], []))
            pend.append((i, m))
            if len(pend) == 2:
                j, mj = pend.pop(0)
                ops.append((f"v_cndmask_b32_e64 v{s + j}, v{s + j}, v{T0}, {mj}", [s + j, T0],
                            [s + j]))
        j, mj = pend.pop(0)
        ops.append((f"v_cndmask_b32_e64 v{s + j}, v{s + j}, v{T0}, {mj}", [s + j, T0], [s + j]))
    for i in range(0, 16, 2):
        pair = (i, i + 1)
        for e in pair:
            ops.append((f"v_mul_f32 v{s + e}, v{s + e}, v{CREG}", [s + e, CREG], [s + e]))
        for e in pair:
            ops.append((f"v_exp_f32 v{s + e}, v{s + e}", [s + e], [s + e]))
        for e in pair:
            ops.append((f"v_mul_f32 v{dp + e}, v{dp + e}, v{s + e}", [dp + e, s + e], [dp + e]))
    cvts = []
    for opnd, src in enumerate((s, s + 8, dp, dp + 8)):
        for r in range(4):
            d = PDS + 4 * opnd + r
            cvts.append((f"v_cvt_pk_bf16_f32 v{d}, v{src + 2 * r}, v{src + 2 * r + 1}",
                         [src + 2 * r, src + 2 * r + 1], [d]))
    return ops, cvts


RING = 4


def schedule(p, mfmas, reads, valu, cvts, n3, ring=RING):
    """Emit MFMAs in order with their operand reads a few MFMAs ahead (two
    register rings of RING operands, row and transposed) and the VALU queue
    spread between them; `cvts` (which overwrite operands of the first n3
    MFMAs) only after the n3-th MFMA has issued."""
    pending = list(reads)
    issued_tags = set()
    ring_use = {"row": [], "tr": []}

    def ring_of(rd):
        return {"tr": "tr", "row": "row"}.get(rd.tag[0])

    def can_issue(rd):
        r = ring_of(rd)
        return r is None or len(ring_use[r]) < ring

    def issue_reads(limit):
        n = 0
        while pending and n < limit and can_issue(pending[0]):
            rd = pending.pop(0)
            for text, rr, ww in rd.ops:
                p.lds_op(text, rd.tag, rr, ww)
            which = ring_of(rd)
            if which is not None:
                ring_use[which].append(rd.tag)
            issued_tags.add(rd.tag)
            n += 1

    issue_reads(ring + 1)
    n_mf = len(mfmas)
    queue = [(op, False) for op in valu] + [(op, True) for op in cvts]
    per = [0] * max(n_mf, 1)
    for i in range(len(queue)):
        per[min(i * n_mf // len(queue), n_mf - 1)] += 1
    qi = 0
    carry = 0
    for k, (dst, a, b, c, tag) in enumerate(mfmas):
        if tag not in issued_tags:
            issue_reads(len(pending))
        assert tag in issued_tags, tag
        p.wait_lds(tag)
        p.mfma(dst, a, b, c)
        for use in ring_use.values():
            if tag in use:
                use.remove(tag)
        issue_reads(2)
        carry += per[k]
        while carry > 0 and qi < len(queue):
            op, is_cvt = queue[qi]
            if is_cvt and k < n3 - 1:
                break
            p.valu(*op)
            qi += 1
            carry -= 1
    while qi < len(queue):
        p.valu(*queue[qi][0])
        qi += 1
    p.wait_lds_all()


def slot(p, ph3, ph1, ph2):
    """ph3 = (stage, qb) or None; ph1 = (stage, qb, buf) or None;
    ph2 = (buf, mask) or None."""
    mfmas, reads = [], []
    if ph3 is not None:
        m, r = phase3_plan(*ph3)
        mfmas += m
        reads += r
    n3 = len(mfmas)
    if ph1 is not None:
        m, r = phase1_plan(*ph1)
        mfmas += m
        reads += r
    valu, cvts = phase2_ops(*ph2) if ph2 is not None else ([], [])
    if ph2 is not None and ph2[1] is not None:
        p.valu(f"v_mov_b32 v{T0}, 0xff800000", [], [T0])
    schedule(p, mfmas, reads, valu, cvts, n3)


# ---------------------------------------------------------------------------
# The program
# ---------------------------------------------------------------------------
def program():
    p = Prog()
    acc = list(range(DV, DV + 64))
    lane = T1
    p.valu(f"v_mbcnt_lo_u32_b32 v{lane}, -1, 0", [], [lane])
    p.valu(f"v_mbcnt_hi_u32_b32 v{lane}, -1, v{lane}", [lane], [lane])
    # l32 and hf first, so that the loads go out before the rest of the lane
    # arithmetic (which recomputes them in place)
    l32, hf = lane_halves(p, lane)
    # tile-load offsets: row tr = 16 wave + 8 i + lane/8, chunk (lane & 7) ^ swz(tr)
    t_l3, t_tr, t_sw, t_x, t_ko = 88, 89, 90, 91, 92
    p.valu(f"v_lshrrev_b32 v{t_l3}, 3, v{lane}", [lane], [t_l3])
    for i in range(2):
        p.valu(f"v_add_u32 v{t_tr}, %[wave16], v{t_l3}", [t_l3], [t_tr])
        if i:
            p.valu(f"v_add_u32 v{t_tr}, 8, v{t_tr}", [t_tr], [t_tr])
        p.valu(f"v_bfe_u32 v{t_sw}, v{t_tr}, 1, 1", [t_tr], [t_sw])
        p.valu(f"v_lshlrev_b32 v{t_sw}, 2, v{t_sw}", [t_sw], [t_sw])
        p.valu(f"v_bfe_u32 v{t_x}, v{t_tr}, 2, 2", [t_tr], [t_x])
        p.valu(f"v_or_b32 v{t_sw}, v{t_sw}, v{t_x}", [t_sw, t_x], [t_sw])
        p.valu(f"v_and_b32 v{t_x}, 7, v{lane}", [lane], [t_x])
        p.valu(f"v_xor_b32 v{t_x}, v{t_x}, v{t_sw}", [t_x, t_sw], [t_x])
        p.valu(f"v_lshlrev_b32 v{t_x}, 4, v{t_x}", [t_x], [t_x])
        p.valu(f"v_mul_lo_u32 v{LDQ + i}, v{t_tr}, %[rs2]", [t_tr], [LDQ + i])
        p.valu(f"v_add_u32 v{LDQ + i}, v{LDQ + i}, v{t_x}", [LDQ + i, t_x], [LDQ + i])
        p.valu(f"v_mul_lo_u32 v{LDG + i}, v{t_tr}, %[c2]", [t_tr], [LDG + i])
        p.valu(f"v_add_u32 v{LDG + i}, v{LDG + i}, v{t_x}", [LDG + i, t_x], [LDG + i])
    p.valu(f"v_lshlrev_b32 v{LDT}, 4, v{lane}", [lane], [LDT])
    # K and V row offset: l32 * row stride + 16 hf
    p.valu(f"v_mul_lo_u32 v{t_ko}, v{l32}, %[rs2]", [l32], [t_ko])
    p.valu(f"v_lshl_add_u32 v{t_ko}, v{hf}, 4, v{t_ko}", [hf, t_ko], [t_ko])
    # ---- first two tiles -----------------------------------------------------
    for sreg, op in ((SQB, "qat"), (SQL, "qleft"), (SGB, "gat"), (SGL, "gleft"), (STB, "tat")):
        p.emit(f"s_mov_b32 s{sreg}, %[{op}_lo]")
        p.emit(f"s_mov_b32 s{sreg + 1}, %[{op}_hi]")
    issue_tile(p, 0, "dkv_i0")
    p.emit("s_cmp_lt_u32 1, %[nit]")
    p.emit("s_cbranch_scc0 dkv_one_tile_%=")
    issue_tile(p, 1, "dkv_i1")
    p.label("dkv_one_tile")
    # ---- K and V of this lane's key (zeros past the sequence) ----------------
    for r in range(KREG, VREG + 16):
        p.valu(f"v_mov_b32 v{r}, 0", [], [r])
    p.valu(f"v_cmp_gt_i32 vcc, %[nk], v{l32}", [l32], [])
    p.emit(f"s_and_saveexec_b64 s[{SEXEC}:{SEXEC + 1}], vcc")
    for kk in range(4):
        p.emit(f"global_load_dwordx4 {vt(KREG + 4 * kk, 4)}, v{t_ko}, %[kbase] offset:{32 * kk}",
               "vmem", [t_ko], list(range(KREG + 4 * kk, KREG + 4 * kk + 4)))
        p.emit(f"global_load_dwordx4 {vt(VREG + 4 * kk, 4)}, v{t_ko}, %[vbase] offset:{32 * kk}",
               "vmem", [t_ko], list(range(VREG + 4 * kk, VREG + 4 * kk + 4)))
    p.emit(f"s_mov_b64 exec, s[{SEXEC}:{SEXEC + 1}]")
    # the rest of the lane arithmetic while the loads are in flight (scratch:
    # the S/dP buffers, free until phase 1)
    regs = {f"koff{kk}": ROFF + kk for kk in range(4)}
    regs.update({f"voff{db}{h}": TROFF + 2 * db + h for db in range(2) for h in range(2)})
    loc = emit_lane_setup(p, regs, lane)
    assert (loc["l32"], loc["hf"]) == (l32, hf)
    for r in list(range(ROFF, ROFF + 4)) + list(range(TROFF, TROFF + 4)):
        p.valu(f"v_add_u32 v{r}, %[qlds], v{r}", [r], [r])
    # terms read offset: hf 512 + l32 16 (+ the LDS base)
    p.valu(f"v_lshlrev_b32 v{TOFF}, 4, v{l32}", [l32], [TOFF])
    p.valu(f"v_lshl_add_u32 v{TOFF}, v{hf}, 9, v{TOFF}", [hf, TOFF], [TOFF])
    p.valu(f"v_add_u32 v{TOFF}, %[qlds], v{TOFF}", [TOFF], [TOFF])
    # the terms k-step's B operands: -1 on the first three k of lane half 0
    # (S) or 1 (dP)
    p.valu(f"v_cmp_eq_u32 vcc, 0, v{hf}", [hf], [])
    for base, hf0 in ((BS, True), (BD, False)):
        for r, word in enumerate((0xBF80BF80, 0x0000BF80, 0, 0)):
            if word == 0:
                p.valu(f"v_mov_b32 v{base + r}, 0", [], [base + r])
            elif hf0:
                p.valu(f"v_mov_b32 v{T0}, {word:#x}", [], [T0])
                p.valu(f"v_cndmask_b32_e64 v{base + r}, 0, v{T0}, vcc", [T0], [base + r])
            else:
                p.valu(f"v_mov_b32 v{T0}, {word:#x}", [], [T0])
                p.valu(f"v_cndmask_b32_e64 v{base + r}, v{T0}, 0, vcc", [T0], [base + r])
    # mask limit of the wave's first tile: l32 - 4 hf + 32 (wave & 1)
    p.valu(f"v_lshlrev_b32 v{LIM}, 2, v{hf}", [hf], [LIM])
    p.valu(f"v_sub_u32 v{LIM}, v{l32}, v{LIM}", [l32, LIM], [LIM])
    p.valu(f"v_add_u32 v{LIM}, %[lim0], v{LIM}", [LIM], [LIM])
    p.valu(f"v_mov_b32 v{CREG}, %[cbits]", [], [CREG])
    for r in acc + list(range(PDS, PDS + 16)):
        p.valu(f"v_mov_b32 v{r}, 0", [], [r])
    p.emit("s_waitcnt vmcnt(0)")
    p.emit("s_barrier")
    p.emit(f"s_mov_b32 s{SJ}, 0")
    # ---- waves 2 and 3 start one tile later ----------------------------------
    p.emit("s_cmp_lt_u32 %[wave], 2")
    p.emit("s_cbranch_scc1 dkv_first0_%=")
    # waves 2, 3: the barrier point of tile 0, then their first tile
    barrier_point(p, 2, "dkv_bp_w23")
    p.emit(f"s_mov_b32 s{SJ}, 1")
    p.emit("s_cmp_lt_u32 1, %[nit]")
    p.emit("s_cbranch_scc0 dkv_end_%=")
    first_tile(p, 1)
    p.emit(f"s_mov_b32 s{SJ}, 2")
    p.emit("s_branch dkv_loop_entry2_%=")
    # waves 0, 1
    p.label("dkv_first0")
    first_tile(p, 0)
    p.emit(f"s_mov_b32 s{SJ}, 1")
    p.emit("s_branch dkv_loop_entry1_%=")
    # ---- steady tiles, unrolled by 3 (stage = t % 3) -------------------------
    for r in range(3):
        p.label(f"dkv_loop_entry{r}", align=True)
        p.reset(acc + list(range(SD0, SD1 + 32)), list(range(PDS, PDS + 16)))
        p.emit(f"s_cmp_lt_u32 s{SJ}, %[nit]")
        p.emit(f"s_cbranch_scc0 dkv_final{(r + 2) % 3}_%=")
        # slot A: phase 3 of half 2t-1 (tile t-1, stage r-1), phase 1 of half
        # 2t+1 (tile t, stage r), phase 2 of half 2t
        slot(p, ((r + 2) % 3, 1), (r, 1, 1), (0, None))
        barrier_point(p, (r + 2) % 3, f"dkv_bp{r}")
        # slot B: phase 3 of half 2t (tile t), phase 1 of half 2t+2 (tile t+1),
        # phase 2 of half 2t+1
        slot(p, (r, 0), ((r + 1) % 3, 0, 0), (1, None))
        p.emit(f"s_add_u32 s{SJ}, s{SJ}, 1")
        if r < 2:
            pass  # falls through to the next entry
        else:
            p.emit("s_branch dkv_loop_entry0_%=")
    # ---- the last half's phase 3 (stage of the last tile) --------------------
    for r in range(3):
        p.label(f"dkv_final{r}", align=True)
        p.reset(acc + list(range(SD0, SD1 + 32)), list(range(PDS, PDS + 16)))
        slot(p, (r, 1), None, None)
        p.emit("s_branch dkv_end_%=")
    # ---- epilogue: dK = scale dK^T, dV = dV^T, rounded to bf16 ----------------
    p.label("dkv_end")
    p.reset(acc)
    e_lane, e_l32, e_hf, t_off = 32, 33, 34, 35
    p.valu(f"v_mbcnt_lo_u32_b32 v{e_lane}, -1, 0", [], [e_lane])
    p.valu(f"v_mbcnt_hi_u32_b32 v{e_lane}, -1, v{e_lane}", [e_lane], [e_lane])
    p.valu(f"v_and_b32 v{e_l32}, 31, v{e_lane}", [e_lane], [e_l32])
    p.valu(f"v_lshrrev_b32 v{e_hf}, 5, v{e_lane}", [e_lane], [e_hf])
    p.valu(f"v_mul_lo_u32 v{t_off}, v{e_l32}, %[rs2]", [e_l32], [t_off])
    p.valu(f"v_lshl_add_u32 v{t_off}, v{e_hf}, 3, v{t_off}", [e_hf, t_off], [t_off])
    p.valu(f"v_mov_b32 v{T0}, %[sbits]", [], [T0])
    out = 40   # packed bf16: dK v40-55, dV v56-71
    for db in range(2):
        for g in range(4):
            k = DK + 16 * db + 4 * g
            v = DV + 16 * db + 4 * g
            for e in range(4):
                p.valu(f"v_mul_f32 v{k + e}, v{k + e}, v{T0}", [k + e, T0], [k + e])
            o = out + 2 * (4 * db + g)
            p.valu(f"v_cvt_pk_bf16_f32 v{o}, v{k}, v{k + 1}", [k, k + 1], [o])
            p.valu(f"v_cvt_pk_bf16_f32 v{o + 1}, v{k + 2}, v{k + 3}", [k + 2, k + 3], [o + 1])
            o2 = out + 16 + 2 * (4 * db + g)
            p.valu(f"v_cvt_pk_bf16_f32 v{o2}, v{v}, v{v + 1}", [v, v + 1], [o2])
            p.valu(f"v_cvt_pk_bf16_f32 v{o2 + 1}, v{v + 2}, v{v + 3}", [v + 2, v + 3], [o2 + 1])
    p.valu(f"v_cmp_gt_i32 vcc, %[nk], v{e_l32}", [e_l32], [])
    p.emit(f"s_and_saveexec_b64 s[{SEXEC}:{SEXEC + 1}], vcc")
    for db in range(2):
        for g in range(4):
            o = out + 2 * (4 * db + g)
            off = (32 * db + 8 * g) * 2
            p.emit(f"global_store_dwordx2 v{t_off}, {vt(o, 2)}, %[dkbase] offset:{off}", "vmem",
                   [t_off, o, o + 1], [])
            p.emit(f"global_store_dwordx2 v{t_off}, {vt(o + 16, 2)}, %[dvbase] offset:{off}",
                   "vmem", [t_off, o + 16, o + 17], [])
    p.emit(f"s_mov_b64 exec, s[{SEXEC}:{SEXEC + 1}]")
    return p.lines


def first_tile(p, t):
    """The wave's first tile t (stage t): phase 1 of its first half, then the
    two slots of the tile with both halves masked; ends before tile t+1."""
    st = t % 3
    slot(p, None, (st, 0, 0), None)
    slot(p, None, (st, 1, 1), (0, 0))
    barrier_point(p, (t + 2) % 3, f"dkv_bpf{t}")
    slot(p, (st, 0), ((st + 1) % 3, 0, 0), (1, 32))


def render(lines):
    body = "\n".join(f'    "{ln}\\n"' for ln in lines)
    clob_v = ", ".join(f'"v{i}"' for i in range(N_VGPR))
    clob_s = ", ".join(f'"s{i}"' for i in range(44, 68))
    return (
        "// Generated by gen_attn_dkdv_asm.py; do not edit by hand.\n"
        "// The program of one dK/dV wave (see the generator for the register map).\n"
        f"#define CATTN_DKDV_ASM_BODY \\\n{body.replace(chr(10), ' ' + chr(92) + chr(10))}\n"
        f"#define CATTN_DKDV_ASM_CLOBBERS {clob_v}, {clob_s}\n"
    )


def main(argv):
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "attn_dkdv_asm.inc")
    lines = program()
    text = render(lines)
    if "--check" in argv:
        ok = os.path.exists(path) and open(path).read() == text
        print("up to date" if ok else "attn_dkdv_asm.inc is out of date: run gen_attn_dkdv_asm.py")
        return 0 if ok else 1
    with open(path, "w") as fh:
        fh.write(text)
    print(f"wrote {path} ({len(lines)} instructions)")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
