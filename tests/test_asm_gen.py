"""The generators of the hand-scheduled kernel programs (CPU only): the
committed includes match the generators, the lane address arithmetic equals
the tile layout's formulas, every wave of a workgroup meets the same number
of barriers and issues its tile loads, and in the dK/dV program every LDS
read falls between the barrier that publishes its tile and the one that
frees its stage."""

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_flash_attention_amd", "csrc")
sys.path.insert(0, CSRC)

import gen_attn_dkdv_asm as gen_dkdv  # noqa: E402
import gen_attn_dq_asm as gen_dq  # noqa: E402
import gen_attn_fwd_asm as gen  # noqa: E402
from asm_flow import Flow  # noqa: E402


def swz(r):
    # the tile swizzle: chunk c of row r sits at chunk c ^ swz(r)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)


@pytest.mark.parametrize("script", ["gen_attn_fwd_asm.py", "gen_attn_dkdv_asm.py",
                                    "gen_attn_dq_asm.py"])
def test_include_is_current(script):
    res = subprocess.run([sys.executable, os.path.join(CSRC, script), "--check"],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr


@pytest.mark.parametrize("lane", range(64))
def test_lane_offsets_match_tile_layout(lane):
    env = gen.eval_lane_setup(lane)
    l32, hf = lane & 31, lane >> 5
    for kk in range(4):
        # K operand: row l32, logical 16-byte chunk 2 kk + hf (bytes)
        assert env[f"koff{kk}"] == l32 * 128 + ((2 * kk + hf) ^ swz(l32)) * 16
    i, grp = lane & 15, lane >> 4
    h = grp >> 1
    for db in range(2):
        # transposed V reads: lane i of a 16-lane group addresses row
        # 4h + i/4 (and 8 rows on), column 32 db + 16 (grp & 1) + 4 (i & 3)
        d = db * 32 + 16 * (grp & 1) + 4 * (i & 3)
        for half in range(2):
            r = 4 * h + (i >> 2) + 8 * half
            want = r * 128 + ((d >> 3) ^ swz(r)) * 16 + (d & 7) * 2
            assert env[f"voff{db}{half}"] == want


def test_program_well_formed():
    lines = gen.program()
    labels = [ln[:-1] for ln in lines if ln.endswith(":")]
    assert len(labels) == len(set(labels)), "duplicate label"
    for ln in lines:
        m = re.match(r"s_(?:c?branch\w*)\s+(\S+)", ln)
        if m:
            assert m.group(1) in labels, ln
        m = re.match(r"s_waitcnt lgkmcnt\((\d+)\)", ln)
        if m:
            assert int(m.group(1)) <= 15
    # one barrier before the first tile and one per step body (6 unrolled steps)
    assert sum(ln == "s_barrier" for ln in lines) == 7
    # 16 MFMAs per pipelined step, two variants per step, plus the first
    # tile's 8 and the last step's 8 per step, and 8 in each of the three
    # out-of-line rescale blocks per step
    assert sum(ln.startswith("v_mfma") for ln in lines) == 8 + 6 * (16 + 16 + 8) + 6 * 3 * 8
    # the rescale blocks sit after the epilogue, hold no barrier and branch back
    tail = lines[lines.index("s_branch fwd_exit_%="):]
    assert "s_barrier" not in tail
    assert sum(ln.startswith("s_branch fwd_redo") for ln in tail) == 18


def test_program_hazard_distances_fwd():
    _check_hazard_distances(gen.program())


def test_program_hazard_distances_dkdv():
    _check_hazard_distances(gen_dkdv.program())


def test_program_hazard_distances_dq():
    _check_hazard_distances(gen_dq.program())


def _check_hazard_distances(lines):
    """Replays the straight-line stretches of the program and checks the
    distances the hardware leaves to software: a VALU/memory instruction
    after an MFMA that wrote one of its registers, and an MFMA after a VALU
    instruction that wrote one of its sources. Branches end a stretch (the
    generator assumes the worst at every label)."""
    reg = re.compile(r"v\[(\d+):(\d+)\]|v(\d+)")

    def regs(operands):
        out = []
        for m in reg.finditer(operands):
            if m.group(3) is not None:
                out.append(int(m.group(3)))
            else:
                out.extend(range(int(m.group(1)), int(m.group(2)) + 1))
        return out

    mfma_at, valu_at, slot = {}, {}, 0
    for ln in lines:
        if ln.endswith(":") or ln.startswith("."):
            mfma_at, valu_at = {}, {}
            continue
        op, _, rest = ln.partition(" ")
        if op == "s_nop":
            slot += int(rest) + 1
            continue
        rs = regs(rest)
        if op.startswith("v_mfma"):
            dst, srcs = rs[:16], rs[16:]
            for r in srcs:
                if r in valu_at:
                    assert slot - valu_at[r] >= gen.VALU_TO_MFMA_WAIT, ln
            for r in dst:
                mfma_at[r] = slot
                valu_at.pop(r, None)
        elif op.startswith(("v_", "ds_", "global_", "buffer_")):
            for r in rs:
                if r in mfma_at:
                    assert slot - mfma_at[r] >= gen.MFMA_RESULT_WAIT, ln
            if op.startswith(("v_", "ds_")) and rs and not op.startswith("v_cmp"):
                valu_at[rs[0]] = slot
                if op.startswith("ds_read"):
                    for r in rs[:4]:
                        valu_at[r] = slot
        slot += 1


@pytest.mark.parametrize("n_kt", [1, 2, 3, 5, 8, 16, 33])
def test_fwd_barriers_and_loads(n_kt):
    """Each wave meets one barrier before its first tile and one per key tile
    of the workgroup, whatever its last tile, and loads 4 rows' worth per tile."""
    lines = gen.program()
    for wave in range(4):
        for j_last in range(n_kt):
            bars, loads = Flow(lines, {"nkt": n_kt, "jlast": j_last, "wave": wave}).run()
            assert bars == n_kt + 1 and len(loads) == 4 * n_kt


def _dkdv_events(trace):
    ev = []
    for ln in trace:
        m = re.match(r"ds_read_b128 v\[128:131\], v156 offset:(\d+)", ln)
        if m:
            o = int(m.group(1)) - gen_dkdv.T_OFF
            ev.append(("p1", o // gen_dkdv.TSTAGE, (o % gen_dkdv.TSTAGE) // 1024))
        m = re.match(r"ds_read_b64_tr_b16 v\[\d+:\d+\], v152 offset:(\d+)", ln)
        if m and int(m.group(1)) >= gen_dkdv.G_OFF:
            o = int(m.group(1)) - gen_dkdv.G_OFF
            st, kc = o // gen_dkdv.STAGE, (o % gen_dkdv.STAGE) // 2048
            if kc % 2 == 0:
                ev.append(("p3", st, kc // 2))
        m = re.match(r"v_cmp_lt_i32_e64 \S+, (\d+), v171", ln)
        if m and int(m.group(1)) in (0, 32):
            ev.append(("mask", int(m.group(1))))
    return ev


@pytest.mark.parametrize("n_it", [1, 2, 3, 4, 5, 7, 12, 16])
def test_dkdv_schedule(n_it):
    """Per wave: n_it + 1 barriers; Q and dO rows of every tile (and the
    terms, waves 0 and 1); S/dP of halves from the wave's first (2 (w // 2))
    to one past the last, dV/dK of each of its halves once, in order, from the
    stage tile k // 2 occupies; the mask on the first two halves."""
    lines = gen_dkdv.program()
    for w in range(4):
        f = Flow(lines, {"nit": n_it, "wave": w})
        bars, loads = f.run()
        assert bars == n_it + 1
        assert len(loads) == 4 * n_it + (n_it if w < 2 else 0)
        ev = _dkdv_events(f.trace)
        first = 2 * (w // 2)
        if n_it == 1 and w >= 2:   # no keys of these waves fall inside T
            want1, want3, masks = [], [], []
        else:
            want1 = [("p1", (k // 2) % 3, k % 2) for k in range(first, 2 * n_it + 1)]
            want3 = [("p3", (k // 2) % 3, k % 2) for k in range(first, 2 * n_it)]
            masks = [0, 32]
        assert [e for e in ev if e[0] == "p1"] == want1
        assert [e for e in ev if e[0] == "p3"] == want3
        assert [e[1] for e in ev if e[0] == "mask"] == masks


@pytest.mark.parametrize("n_it", [1, 2, 3, 6, 13])
def test_dkdv_reads_between_publish_and_refill(n_it):
    """Tile t is published by barrier max(1, t + 1) and its stage refilled
    after barrier t + 3: every LDS read must map to exactly one tile inside
    that window."""
    lines = gen_dkdv.program()
    for w in range(4):
        f = Flow(lines, {"nit": n_it, "wave": w})
        f.run()
        nb = 0
        for ln in f.trace:
            if ln == "s_barrier":
                nb += 1
            elif ln.startswith("ds_read"):
                o = int(re.search(r"offset:(\d+)", ln).group(1))
                st = ((o - gen_dkdv.T_OFF) // gen_dkdv.TSTAGE if o >= gen_dkdv.T_OFF
                      else (o % gen_dkdv.G_OFF) // gen_dkdv.STAGE)
                cands = [t for t in range(n_it + 3)
                         if t % 3 == st and max(1, t + 1) <= nb < t + 3]
                assert len(cands) == 1, (w, nb, ln)


@pytest.mark.parametrize("n_kt", [1, 2, 3, 4, 7, 11])
def test_dq_schedule(n_kt):
    """Per wave, for every position of its diagonal half k1: n_kt + 1
    barriers and 4 tile-load instructions per tile; S/dP and dQ of halves
    0 .. k1 each once, in order, from the stage tile k // 2 occupies; one
    masked half; every LDS read between its tile's publication and refill."""
    lines = gen_dq.program()
    for k1 in range(2 * n_kt):
        f = Flow(lines, {"nkt": n_kt, "k1": k1})
        bars, loads = f.run()
        assert bars == n_kt + 1 and len(loads) == 4 * n_kt
        p1, p3, masks, nb = [], [], 0, 0
        for ln in f.trace:
            if ln == "s_barrier":
                nb += 1
                continue
            m = re.match(rf"ds_read_b128 v\[\d+:\d+\], v{gen_dq.ROFF} offset:(\d+)", ln)
            if m and int(m.group(1)) < gen_dq.V_OFF:
                o = int(m.group(1))
                p1.append((o // gen_dq.STAGE, (o % gen_dq.STAGE) // 4096))
            m = re.match(rf"ds_read_b64_tr_b16 v\[\d+:\d+\], v{gen_dq.TROFF} offset:(\d+)", ln)
            if m:
                o = int(m.group(1))
                st, kc = o // gen_dq.STAGE, (o % gen_dq.STAGE) // 2048
                if kc % 2 == 0:
                    p3.append((st, kc // 2))
            if re.match(rf"v_cmp_gt_i32_e64 \S+, 0, v{gen_dq.LIM}", ln):
                masks += 1
            if ln.startswith("ds_read"):
                o = int(re.search(r"offset:(\d+)", ln).group(1))
                st = (o % gen_dq.V_OFF) // gen_dq.STAGE
                cands = [t for t in range(n_kt + 3)
                         if t % 3 == st and max(1, t + 1) <= nb < t + 3]
                assert len(cands) == 1, (k1, nb, ln)
        want = [((k // 2) % 3, k % 2) for k in range(k1 + 1)]
        assert p1 == want and p3 == want and masks == 1
