"""A small interpreter of the scalar control flow of the generated kernel
programs (CPU only): it follows the SALU moves, adds, compares and branches,
counts the barriers a wave executes and the tile loads it issues, and treats
every other instruction as a no-op. Operands (%[name]) take the values given."""

import re

_SREG = re.compile(r"^s(\d+)$")


class Flow:
    def __init__(self, lines, operands, max_steps=2_000_000):
        self.lines = [ln.replace("_%=", "") for ln in lines]
        self.labels = {ln[:-1]: i for i, ln in enumerate(self.lines) if ln.endswith(":")}
        self.ops = operands
        self.max_steps = max_steps

    def _val(self, tok, sregs):
        tok = tok.strip()
        if tok.startswith("%["):
            return self.ops.get(tok[2:-1], 0) & 0xFFFFFFFF
        m = _SREG.match(tok)
        if m:
            return sregs.get(int(m.group(1)), 0)
        return int(tok, 0) & 0xFFFFFFFF

    def run(self):
        sregs, scc, pc = {}, 0, 0
        barriers, tile_loads, steps = 0, [], 0
        self.trace = []
        while pc < len(self.lines):
            steps += 1
            if steps > self.max_steps:
                raise RuntimeError("control flow does not terminate")
            ln = self.lines[pc]
            self.trace.append(ln)
            op, _, rest = ln.partition(" ")
            args = [a for a in rest.split(", ")] if rest else []
            nxt = pc + 1
            if op == "s_barrier":
                barriers += 1
            elif op in ("s_mov_b32",) and _SREG.match(args[0]):
                sregs[int(args[0][1:])] = self._val(args[1], sregs)
            elif op == "s_add_u32" and _SREG.match(args[0]):
                v = self._val(args[1], sregs) + self._val(args[2], sregs)
                sregs[int(args[0][1:])] = v & 0xFFFFFFFF
            elif op.startswith("s_cmp_"):
                a, b = self._val(args[0], sregs), self._val(args[1], sregs)
                kind = op[6:9].rstrip("_")
                scc = {"lt": a < b, "eq": a == b, "lg": a != b, "gt": a > b,
                       "ge": a >= b, "le": a <= b}[kind]
            elif op == "s_cbranch_scc0":
                if not scc:
                    nxt = self.labels[args[0]] + 1
            elif op == "s_cbranch_scc1":
                if scc:
                    nxt = self.labels[args[0]] + 1
            elif op == "s_branch":
                nxt = self.labels[args[0]] + 1
            elif op in ("buffer_load_dwordx4", "global_load_lds_dwordx4") and "lds" in ln:
                tile_loads.append(ln)
            pc = nxt
        return barriers, tile_loads
