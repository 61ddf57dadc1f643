"""Generate attn_dq_asm.inc: the hand-scheduled program of one dQ wave.

python gen_attn_dq_asm.py            # writes attn_dq_asm.inc beside this file
python gen_attn_dq_asm.py --check    # exits 1 when the file is out of date

A wave owns 32 queries of one (batch, head), with Q and dO of its queries in
registers and LSE * log2 e and D of its query in one register each, and
walks the key tiles (64 rows of K and V) that stream through a three-stage
LDS ring. Each tile is two halves of 32 keys, and each half goes through
three phases:
  1. S^T = K Q^T and dP^T = V dO^T on MFMA (8 MFMAs);
  2. P^T = exp2(c S^T - LSE log2 e) and dS^T = P^T (dP^T - D) on the VALU,
     rounded to bf16 operands (with the causal mask on the wave's diagonal
     half, its last);
  3. dQ^T += K^T dS^T on MFMA (4 MFMAs, K^T read from the row-major K tile
     by transposing reads).
As in the dK/dV program, slot k issues phase 3 of half k-1 and phase 1 of
half k+1 on MFMA while phase 2 of half k runs on the VALU between them, and
one barrier per tile sits between the tile's two slots. A wave's halves end
at its diagonal (half k1); from there it only meets the workgroup's
remaining barriers and issues its share of the remaining tile loads.

The program also forms the lane's D = rowsum(dO * O) (the same fmaf chain
as the preprocess, so the same bits) and LSE log2 e itself, so that the
kernel fits three waves per SIMD.

Register map (VGPR): v0-15 Q operands, v16-31 dO operands, v32-63 / v64-95
S^T and dP^T of even / odd halves, v96-103 dS^T operands, v104-111 row
operand ring (2), v112-119 transposed operand ring (2), v120-123 row read
offsets, v124-127 transposed read offsets, v128-129 tile-load offsets, v130
LSE log2 e, v131 D, v132 mask limit, v133 temporary, v134-165 the
accumulators dQ^T (d blocks 0, 1).
"""

from __future__ import annotations

import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

from gen_attn_dkdv_asm import Read, schedule  # noqa: E402
from gen_attn_fwd_asm import Prog, emit_lane_setup, lane_halves, vt  # noqa: E402

QREG, GREG, SD0, SD1, DS = 0, 16, 32, 64, 96
ROW, TR = 104, 112
ROFF, TROFF, LDOFF = 120, 124, 128
LSE2, DD, LIM, T0 = 130, 131, 132, 133
DQ = 134
N_VGPR = 166
LANE = 94          # the lane id, during the prologue only (a dP^T register)
DQ_RING = 2

K_OFF, V_OFF, STAGE = 0, 24576, 8192

# SGPRs: descriptor s[44:47], next tile base s[48:49], bytes left s[50:51],
# tile index s52, half index s53, temporary s54, saved exec s[56:57], second
# compare mask s[58:59], LSE row base s[60:61]
SD, SB, SL, SJ, SK, ST, SEXEC, SCMP, SLB = 44, 48, 50, 52, 53, 54, 56, 58, 60


def sd_regs(buf):
    base = SD0 if buf == 0 else SD1
    return base, base + 16


def issue_tile(p, stage):
    """K and V rows of the next tile into `stage`: one descriptor, V reached
    through the scalar offset (C elements further along the packed row)."""
    p.emit(f"s_cmp_lg_u32 s{SL + 1}, 0")
    p.emit(f"s_cselect_b32 s{SD + 2}, -1, s{SL}")
    p.emit(f"s_mov_b32 s{SD}, s{SB}")
    p.emit(f"s_and_b32 s{SD + 1}, s{SB + 1}, 0xffff")
    p.emit(f"s_mov_b32 s{SD + 3}, 0x20000")
    for i in range(2):
        p.emit(f"s_add_u32 m0, %[kldw], {K_OFF + stage * STAGE + i * 1024}")
        p.emit(f"buffer_load_dwordx4 v{LDOFF + i}, s[{SD}:{SD + 3}], 0 offen lds", "vmem_lds",
               [LDOFF + i])
    for i in range(2):
        p.emit(f"s_add_u32 m0, %[kldw], {V_OFF + stage * STAGE + i * 1024}")
        p.emit(f"buffer_load_dwordx4 v{LDOFF + i}, s[{SD}:{SD + 3}], %[voffs] offen lds",
               "vmem_lds", [LDOFF + i])
    p.emit(f"s_add_u32 s{SB}, s{SB}, %[tbytes]")
    p.emit(f"s_addc_u32 s{SB + 1}, s{SB + 1}, 0")
    p.emit(f"s_sub_u32 s{SL}, s{SL}, %[tbytes]")
    p.emit(f"s_subb_u32 s{SL + 1}, s{SL + 1}, 0")


def barrier_point(p, stage, name):
    """Tile j+1 has landed everywhere and every wave has left tile j-1:
    wait, meet, then load tile j+2 into the stage tile j-1 held."""
    p.emit("s_waitcnt vmcnt(0)")
    p.emit("s_barrier")
    p.emit(f"s_add_u32 s{ST}, s{SJ}, 2")
    p.emit(f"s_cmp_lt_u32 s{ST}, %[nkt]")
    snap = p.snapshot()
    p.emit(f"s_cbranch_scc0 {name}_%=")
    issue_tile(p, stage)
    p.label(name)
    p.join(snap)


def phase1_plan(stage, kb, buf):
    s, dp = sd_regs(buf)
    mf, reads = [], []
    slot = 0
    for kk in range(4):
        for which, (off, breg, acc) in enumerate(((K_OFF, QREG, s), (V_OFF, GREG, dp))):
            dst = ROW + 4 * (slot % DQ_RING)
            tag = ("row", stage, kb, kk, which)
            reads.append(Read(tag, [(f"ds_read_b128 {vt(dst, 4)}, v{ROFF + kk} offset:"
                                     f"{off + stage * STAGE + kb * 4096}", [ROFF + kk],
                                     list(range(dst, dst + 4)))], dst))
            mf.append((acc, dst, breg + 4 * kk, None if kk == 0 else acc, tag))
            slot += 1
    return mf, reads


def phase3_plan(stage, kb):
    mf, reads = [], []
    slot = 0
    for db in range(2):
        for j in range(2):
            kc = 2 * kb + j
            dst = TR + 4 * (slot % DQ_RING)
            tag = ("tr", stage, kb, db, j)
            o = K_OFF + stage * STAGE + kc * 2048
            reads.append(Read(tag, [
                (f"ds_read_b64_tr_b16 {vt(dst, 2)}, v{TROFF + 2 * db} offset:{o}",
                 [TROFF + 2 * db], [dst, dst + 1]),
                (f"ds_read_b64_tr_b16 {vt(dst + 2, 2)}, v{TROFF + 2 * db + 1} offset:{o}",
                 [TROFF + 2 * db + 1], [dst + 2, dst + 3])], dst))
            mf.append((DQ + 16 * db, dst, DS + 4 * j, DQ + 16 * db, tag))
            slot += 1
    return mf, reads


def phase2_ops(buf, masked):
    """P^T and dS^T of a half; the mask (diagonal half) hides keys above the
    lane's query: key row 8 (i / 4) + (i % 4) (+ 4 hf) > the lane's limit."""
    s, dp = sd_regs(buf)
    ops = []
    if masked:
        masks = ["vcc", f"s[{SCMP}:{SCMP + 1}]"]
        pend = []
        for i in range(16):
            idx = 8 * (i // 4) + (i % 4)
            m = masks[i % 2]
            ops.append((f"v_cmp_gt_i32_e64 {m}, {idx}, v{LIM}", [LIM], []))
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
            ops.append((f"v_fma_f32 v{s + e}, v{s + e}, %[cbits], -v{LSE2}", [s + e, LSE2],
                        [s + e]))
        for e in pair:
            ops.append((f"v_exp_f32 v{s + e}, v{s + e}", [s + e], [s + e]))
        for e in pair:
            ops.append((f"v_sub_f32 v{dp + e}, v{dp + e}, v{DD}", [dp + e, DD], [dp + e]))
        for e in pair:
            ops.append((f"v_mul_f32 v{dp + e}, v{dp + e}, v{s + e}", [dp + e, s + e], [dp + e]))
    cvts = []
    for opnd, src in enumerate((dp, dp + 8)):
        for r in range(4):
            d = DS + 4 * opnd + r
            cvts.append((f"v_cvt_pk_bf16_f32 v{d}, v{src + 2 * r}, v{src + 2 * r + 1}",
                         [src + 2 * r, src + 2 * r + 1], [d]))
    return ops, cvts


def slot(p, ph3, ph1, ph2):
    """ph3 = (stage, kb) or None; ph1 = (stage, kb, buf) or None;
    ph2 = (buf, masked) or None."""
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
    if ph2 is not None and ph2[1]:
        p.valu(f"v_mov_b32 v{T0}, 0xff800000", [], [T0])
    schedule(p, mfmas, reads, valu, cvts, n3, ring=DQ_RING)


def dispatch(p, name, variants):
    """Branch on the slot's half index s53 against k1: variants maps
    'full' / 'end' / 'ph3' to emitter callables (None: nothing to do);
    all paths meet at the end label."""
    p.emit(f"s_cmp_lt_u32 s{SK}, %[k1]")
    p.emit(f"s_cbranch_scc1 {name}_full_%=")
    p.emit(f"s_cmp_eq_u32 s{SK}, %[k1]")
    p.emit(f"s_cbranch_scc1 {name}_end_%=")
    p.emit(f"s_add_u32 s{ST}, %[k1], 1")
    p.emit(f"s_cmp_eq_u32 s{SK}, s{ST}")
    p.emit(f"s_cbranch_scc1 {name}_ph3_%=")
    p.emit(f"s_branch {name}_done_%=")
    start = p.snapshot()
    for key in ("full", "end", "ph3"):
        p.restore(start)
        p.label(f"{name}_{key}")
        if variants.get(key) is not None:
            variants[key]()
        p.emit(f"s_branch {name}_done_%=")
    p.label(f"{name}_done")
    p.reset(list(range(DQ, DQ + 32)) + list(range(SD0, SD1 + 32)), list(range(DS, DS + 8)))
    p.emit(f"s_add_u32 s{SK}, s{SK}, 1")


def mfma_terms(p, x, out0, out1, tmp):
    """The three bf16 terms a + b + c = x (each rounded to nearest even)
    packed as [a | b << 16, c]: out0, out1; tmp is a scratch register."""
    p.valu(f"v_cvt_pk_bf16_f32 v{out0}, v{x}, 0", [x], [out0])            # a
    p.valu(f"v_lshlrev_b32 v{tmp}, 16, v{out0}", [out0], [tmp])
    p.valu(f"v_sub_f32 v{tmp}, v{x}, v{tmp}", [x, tmp], [tmp])            # r = x - a
    p.valu(f"v_cvt_pk_bf16_f32 v{out1}, v{tmp}, 0", [tmp], [out1])        # b
    p.valu(f"v_lshl_or_b32 v{out0}, v{out1}, 16, v{out0}", [out1, out0], [out0])
    p.valu(f"v_lshlrev_b32 v{out1}, 16, v{out1}", [out1], [out1])
    p.valu(f"v_sub_f32 v{tmp}, v{tmp}, v{out1}", [tmp, out1], [tmp])      # r - b
    p.valu(f"v_cvt_pk_bf16_f32 v{out1}, v{tmp}, 0", [tmp], [out1])        # c


def workspace_rows(p, l32, hf, lse_raw):
    """The workspace rows of this wave's queries that lie below the padded
    length (lane half 0): D, LSE log2 e, and the MFMA terms of 8 LSE and of
    D (past T: the terms that make P = 0). The stores overlap the tile loop."""
    # scratch (the dS^T operands and the row ring, free here): the m terms
    # v102-105 and the D terms v106-109 as [w0, w1, 0, 0]
    x8, m0, d0, tmp, off, pad = 101, 102, 106, 110, 111, 99
    p.valu(f"v_mul_f32 v{x8}, 0x41000000, v{lse_raw}", [lse_raw], [x8])
    mfma_terms(p, x8, m0, m0 + 1, tmp)
    # past T the m terms are [0x7F7F, 0] (P = 0 there); D = 0 there already
    p.valu(f"v_mov_b32 v{pad}, 0x7f7f", [], [pad])
    p.valu(f"v_cndmask_b32_e64 v{m0}, v{pad}, v{m0}, vcc", [pad, m0], [m0])
    p.valu(f"v_cndmask_b32_e64 v{m0 + 1}, 0, v{m0 + 1}, vcc", [m0 + 1], [m0 + 1])
    mfma_terms(p, DD, d0, d0 + 1, tmp)
    for r in (m0 + 2, m0 + 3, d0 + 2, d0 + 3):
        p.valu(f"v_mov_b32 v{r}, 0", [], [r])
    p.valu(f"v_lshlrev_b32 v{off}, 2, v{l32}", [l32], [off])
    p.valu(f"v_cmp_gt_i32 vcc, %[nw], v{LANE}", [LANE], [])
    p.emit(f"s_mov_b32 s{SLB}, %[wsd_lo]")
    p.emit(f"s_mov_b32 s{SLB + 1}, %[wsd_hi]")
    p.emit(f"s_and_saveexec_b64 s[{SEXEC}:{SEXEC + 1}], vcc")
    p.emit(f"global_store_dword v{off}, v{DD}, s[{SLB}:{SLB + 1}]", "vmem", [off, DD], [])
    p.emit(f"s_mov_b32 s{SLB}, %[wsl_lo]")
    p.emit(f"s_mov_b32 s{SLB + 1}, %[wsl_hi]")
    p.emit(f"global_store_dword v{off}, v{LSE2}, s[{SLB}:{SLB + 1}]", "vmem", [off, LSE2], [])
    p.valu(f"v_lshlrev_b32 v{off}, 4, v{l32}", [l32], [off])
    p.emit(f"s_mov_b32 s{SLB}, %[wst_lo]")
    p.emit(f"s_mov_b32 s{SLB + 1}, %[wst_hi]")
    p.emit(f"global_store_dwordx4 v{off}, v[{m0}:{m0 + 3}], s[{SLB}:{SLB + 1}]", "vmem",
           [off] + list(range(m0, m0 + 4)), [])
    p.emit(f"global_store_dwordx4 v{off}, v[{d0}:{d0 + 3}], s[{SLB}:{SLB + 1}] offset:512", "vmem",
           [off] + list(range(d0, d0 + 4)), [])
    p.emit(f"s_mov_b64 exec, s[{SEXEC}:{SEXEC + 1}]")


def program():
    p = Prog()
    acc = list(range(DQ, DQ + 32))
    lane = LANE
    p.valu(f"v_mbcnt_lo_u32_b32 v{lane}, -1, 0", [], [lane])
    p.valu(f"v_mbcnt_hi_u32_b32 v{lane}, -1, v{lane}", [lane], [lane])
    # l32 and hf first, so that the loads go out before the rest of the lane
    # arithmetic (which recomputes them in place)
    l32, hf = lane_halves(p, lane)
    t_l3, t_tr, t_sw, t_x, t_qo, t_go = 88, 89, 90, 91, 92, 93
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
        p.valu(f"v_mul_lo_u32 v{LDOFF + i}, v{t_tr}, %[rs2]", [t_tr], [LDOFF + i])
        p.valu(f"v_add_u32 v{LDOFF + i}, v{LDOFF + i}, v{t_x}", [LDOFF + i, t_x], [LDOFF + i])
    p.valu(f"v_mul_lo_u32 v{t_qo}, v{l32}, %[rs2]", [l32], [t_qo])
    p.valu(f"v_lshl_add_u32 v{t_qo}, v{hf}, 4, v{t_qo}", [hf, t_qo], [t_qo])
    p.valu(f"v_mul_lo_u32 v{t_go}, v{l32}, %[c2]", [l32], [t_go])
    p.valu(f"v_lshl_add_u32 v{t_go}, v{hf}, 4, v{t_go}", [hf, t_go], [t_go])
    # ---- first two tiles ------------------------------------------------------
    p.emit(f"s_mov_b32 s{SB}, %[kat_lo]")
    p.emit(f"s_mov_b32 s{SB + 1}, %[kat_hi]")
    p.emit(f"s_mov_b32 s{SL}, %[kleft_lo]")
    p.emit(f"s_mov_b32 s{SL + 1}, %[kleft_hi]")
    issue_tile(p, 0)
    p.emit("s_cmp_lt_u32 1, %[nkt]")
    snap = p.snapshot()
    p.emit("s_cbranch_scc0 dq_one_tile_%=")
    issue_tile(p, 1)
    p.label("dq_one_tile")
    p.join(snap)
    # ---- Q and dO of this lane's query (zeros past the sequence) --------------
    for r in range(QREG, GREG + 16):
        p.valu(f"v_mov_b32 v{r}, 0", [], [r])
    p.valu(f"v_cmp_gt_i32 vcc, %[nq], v{l32}", [l32], [])
    p.emit(f"s_and_saveexec_b64 s[{SEXEC}:{SEXEC + 1}], vcc")
    for kk in range(4):
        p.emit(f"global_load_dwordx4 {vt(QREG + 4 * kk, 4)}, v{t_qo}, %[qbase] offset:{32 * kk}",
               "vmem", [t_qo], list(range(QREG + 4 * kk, QREG + 4 * kk + 4)))
        p.emit(f"global_load_dwordx4 {vt(GREG + 4 * kk, 4)}, v{t_go}, %[gbase] offset:{32 * kk}",
               "vmem", [t_go], list(range(GREG + 4 * kk, GREG + 4 * kk + 4)))
    p.emit(f"s_mov_b64 exec, s[{SEXEC}:{SEXEC + 1}]")
    # O of this lane's query (zeros past the sequence) and its LSE
    ob, t_lo = 76, 95      # clear of the lane arithmetic scratch (v48-74) while in flight
    for r in range(ob, ob + 16):
        p.valu(f"v_mov_b32 v{r}, 0", [], [r])
    p.valu(f"v_mov_b32 v{LSE2}, 0x7f800000", [], [LSE2])
    p.valu(f"v_lshlrev_b32 v{t_lo}, 2, v{l32}", [l32], [t_lo])
    p.emit(f"s_mov_b32 s{SLB}, %[lbase_lo]")
    p.emit(f"s_mov_b32 s{SLB + 1}, %[lbase_hi]")
    p.emit(f"s_and_saveexec_b64 s[{SEXEC}:{SEXEC + 1}], vcc")
    for kk in range(4):
        p.emit(f"global_load_dwordx4 {vt(ob + 4 * kk, 4)}, v{t_go}, %[obase] offset:{32 * kk}",
               "vmem", [t_go], list(range(ob + 4 * kk, ob + 4 * kk + 4)))
    p.emit(f"global_load_dword v{LSE2}, v{t_lo}, s[{SLB}:{SLB + 1}]", "vmem", [t_lo], [LSE2])
    p.emit(f"s_mov_b64 exec, s[{SEXEC}:{SEXEC + 1}]")
    # the rest of the lane arithmetic while the loads are in flight
    regs = {f"koff{kk}": ROFF + kk for kk in range(4)}
    regs.update({f"voff{db}{h}": TROFF + 2 * db + h for db in range(2) for h in range(2)})
    loc = emit_lane_setup(p, regs, lane)
    assert (loc["l32"], loc["hf"]) == (l32, hf)
    for r in list(range(ROFF, ROFF + 4)) + list(range(TROFF, TROFF + 4)):
        p.valu(f"v_add_u32 v{r}, %[klds], v{r}", [r], [r])
    # mask limit of the diagonal half: l32 - 4 hf + (qw - 32 k1)
    p.valu(f"v_lshlrev_b32 v{LIM}, 2, v{hf}", [hf], [LIM])
    p.valu(f"v_sub_u32 v{LIM}, v{l32}, v{LIM}", [l32, LIM], [LIM])
    p.valu(f"v_add_u32 v{LIM}, %[limb], v{LIM}", [LIM], [LIM])

    for r in acc + list(range(DS, DS + 8)):
        p.valu(f"v_mov_b32 v{r}, 0", [], [r])
    p.emit("s_waitcnt vmcnt(0)")
    # LSE log2 e (+inf past the sequence: P = 0 there); the raw LSE stays in
    # lse_raw for the workspace terms
    lse_raw = 100
    p.valu(f"v_mov_b32 v{lse_raw}, v{LSE2}", [LSE2], [lse_raw])
    p.valu(f"v_mul_f32 v{T0}, 0x3fb8aa3b, v{LSE2}", [LSE2], [T0])
    p.valu(f"v_cndmask_b32_e64 v{LSE2}, v{LSE2}, v{T0}, vcc", [LSE2, T0], [LSE2])
    # D: the lane's 32 products of dO and O in one fmaf chain (k = 16 kk +
    # 8 hf + e, kk and e ascending), then the other lane half's sum added
    gl, gh, olo, ohi = 96, 97, 98, 99
    p.valu(f"v_mov_b32 v{DD}, 0", [], [DD])
    for kk in range(4):
        for w in range(4):
            g, o = GREG + 4 * kk + w, ob + 4 * kk + w
            p.valu(f"v_lshlrev_b32 v{gl}, 16, v{g}", [g], [gl])
            p.valu(f"v_lshlrev_b32 v{olo}, 16, v{o}", [o], [olo])
            p.valu(f"v_and_b32 v{gh}, 0xffff0000, v{g}", [g], [gh])
            p.valu(f"v_and_b32 v{ohi}, 0xffff0000, v{o}", [o], [ohi])
            p.valu(f"v_fma_f32 v{DD}, v{gl}, v{olo}, v{DD}", [gl, olo, DD], [DD])
            p.valu(f"v_fma_f32 v{DD}, v{gh}, v{ohi}, v{DD}", [gh, ohi, DD], [DD])
    p.valu(f"v_xor_b32 v{T0}, 32, v{lane}", [lane], [T0])
    p.valu(f"v_lshlrev_b32 v{T0}, 2, v{T0}", [T0], [T0])
    p.lds_op(f"ds_bpermute_b32 v{T0}, v{T0}, v{DD}", ("bperm",), [T0, DD], [T0])
    p.wait_lds(("bperm",))
    p.valu(f"v_add_f32 v{DD}, v{DD}, v{T0}", [DD, T0], [DD])
    workspace_rows(p, l32, hf, lse_raw)
    for r in range(DS, DS + 8):
        p.valu(f"v_mov_b32 v{r}, 0", [], [r])
    p.emit("s_barrier")
    p.emit(f"s_mov_b32 s{SJ}, 0")
    p.emit(f"s_mov_b32 s{SK}, 0")
    # ---- tile 0: phase 1 of half 0, then its two slots -------------------------
    slot(p, None, (0, 0, 0), None)
    dispatch(p, "dq_a0", {"full": lambda: slot(p, None, (0, 1, 1), (0, False)),
                          "end": lambda: slot(p, None, None, (0, True))})
    barrier_point(p, 2, "dq_bp0")
    dispatch(p, "dq_b0", {"full": lambda: slot(p, (0, 0), (1, 0, 0), (1, False)),
                          "end": lambda: slot(p, (0, 0), None, (1, True)),
                          "ph3": lambda: slot(p, (0, 0), None, None)})
    p.emit(f"s_mov_b32 s{SJ}, 1")
    # ---- tiles 1 .. n_kt - 1, unrolled by 3 (stage = j % 3) --------------------
    for r in (1, 2, 0):
        p.label(f"dq_tile{r}", align=True)
        p.reset(acc + list(range(SD0, SD1 + 32)), list(range(DS, DS + 8)))
        p.emit(f"s_cmp_lt_u32 s{SJ}, %[nkt]")
        p.emit(f"s_cbranch_scc0 dq_after{(r + 2) % 3}_%=")
        rp, rn = (r + 2) % 3, (r + 1) % 3
        dispatch(p, f"dq_a{r}x", {"full": lambda r=r, rp=rp: slot(p, (rp, 1), (r, 1, 1), (0, False)),
                                  "end": lambda rp=rp: slot(p, (rp, 1), None, (0, True)),
                                  "ph3": lambda rp=rp: slot(p, (rp, 1), None, None)})
        barrier_point(p, rp, f"dq_bp{r}x")
        dispatch(p, f"dq_b{r}x", {"full": lambda r=r, rn=rn: slot(p, (r, 0), (rn, 0, 0), (1, False)),
                                  "end": lambda r=r: slot(p, (r, 0), None, (1, True)),
                                  "ph3": lambda r=r: slot(p, (r, 0), None, None)})
        p.emit(f"s_add_u32 s{SJ}, s{SJ}, 1")
        if r == 0:
            p.emit("s_branch dq_tile1_%=")
    # ---- past the last tile: phase 3 of half 2 n_kt - 1 when it is k1 ---------
    for r in range(3):
        p.label(f"dq_after{r}", align=True)
        p.reset(acc + list(range(SD0, SD1 + 32)), list(range(DS, DS + 8)))
        p.emit(f"s_add_u32 s{ST}, %[k1], 1")
        p.emit(f"s_cmp_eq_u32 s{SK}, s{ST}")
        p.emit("s_cbranch_scc0 dq_end_%=")
        slot(p, (r, 1), None, None)
        p.emit("s_branch dq_end_%=")
    # ---- epilogue: dQ = scale dQ^T, rounded to bf16 -----------------------------
    p.label("dq_end")
    p.reset(acc)
    e_lane, e_l32, e_hf, t_off = 32, 33, 34, 35
    p.valu(f"v_mbcnt_lo_u32_b32 v{e_lane}, -1, 0", [], [e_lane])
    p.valu(f"v_mbcnt_hi_u32_b32 v{e_lane}, -1, v{e_lane}", [e_lane], [e_lane])
    p.valu(f"v_and_b32 v{e_l32}, 31, v{e_lane}", [e_lane], [e_l32])
    p.valu(f"v_lshrrev_b32 v{e_hf}, 5, v{e_lane}", [e_lane], [e_hf])
    p.valu(f"v_mul_lo_u32 v{t_off}, v{e_l32}, %[rs2]", [e_l32], [t_off])
    p.valu(f"v_lshl_add_u32 v{t_off}, v{e_hf}, 3, v{t_off}", [e_hf, t_off], [t_off])
    p.valu(f"v_mov_b32 v{T0}, %[sbits]", [], [T0])
    out = 40
    for db in range(2):
        for g in range(4):
            q = DQ + 16 * db + 4 * g
            for e in range(4):
                p.valu(f"v_mul_f32 v{q + e}, v{q + e}, v{T0}", [q + e, T0], [q + e])
            o = out + 2 * (4 * db + g)
            p.valu(f"v_cvt_pk_bf16_f32 v{o}, v{q}, v{q + 1}", [q, q + 1], [o])
            p.valu(f"v_cvt_pk_bf16_f32 v{o + 1}, v{q + 2}, v{q + 3}", [q + 2, q + 3], [o + 1])
    p.valu(f"v_cmp_gt_i32 vcc, %[nq], v{e_l32}", [e_l32], [])
    p.emit(f"s_and_saveexec_b64 s[{SEXEC}:{SEXEC + 1}], vcc")
    for db in range(2):
        for g in range(4):
            o = out + 2 * (4 * db + g)
            p.emit(f"global_store_dwordx2 v{t_off}, {vt(o, 2)}, %[dqbase] offset:{(32 * db + 8 * g) * 2}",
                   "vmem", [t_off, o, o + 1], [])
    p.emit(f"s_mov_b64 exec, s[{SEXEC}:{SEXEC + 1}]")
    return p.lines


def render(lines):
    body = "\n".join(f'    "{ln}\\n"' for ln in lines)
    clob_v = ", ".join(f'"v{i}"' for i in range(N_VGPR))
    clob_s = ", ".join(f'"s{i}"' for i in range(44, 62))
    return (
        "// Generated by gen_attn_dq_asm.py; do not edit by hand.\n"
        "// The program of one dQ wave (see the generator for the register map).\n"
        f"#define CATTN_DQ_ASM_BODY \\\n{body.replace(chr(10), ' ' + chr(92) + chr(10))}\n"
        f"#define CATTN_DQ_ASM_CLOBBERS {clob_v}, {clob_s}\n"
    )


def main(argv):
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "attn_dq_asm.inc")
    lines = program()
    text = render(lines)
    if "--check" in argv:
        ok = os.path.exists(path) and open(path).read() == text
        print("up to date" if ok else "attn_dq_asm.inc is out of date: run gen_attn_dq_asm.py")
        return 0 if ok else 1
    with open(path, "w") as fh:
        fh.write(text)
    print(f"wrote {path} ({len(lines)} instructions)")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
