"""The generator of the hand-scheduled forward program (CPU only): the
committed include matches the generator, the lane address arithmetic it
emits equals the tile layout's formulas, and the program's control flow and
wait counts are well formed."""

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_flash_attention_amd", "csrc")
sys.path.insert(0, CSRC)

import gen_attn_fwd_asm as gen  # noqa: E402


def swz(r):
    # the tile swizzle: chunk c of row r sits at chunk c ^ swz(r)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)


def test_include_is_current():
    res = subprocess.run([sys.executable, os.path.join(CSRC, "gen_attn_fwd_asm.py"), "--check"],
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
    # tile's 8 and the last step's 8 per step
    assert sum(ln.startswith("v_mfma") for ln in lines) == 8 + 6 * (16 + 16 + 8)


def test_program_hazard_distances():
    """Replays the straight-line stretches of the program and checks the
    distances the hardware leaves to software: a VALU/memory instruction
    after an MFMA that wrote one of its registers, and an MFMA after a VALU
    instruction that wrote one of its sources. Branches end a stretch (the
    generator assumes the worst at every label)."""
    lines = gen.program()
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
