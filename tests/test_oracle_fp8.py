"""Pins for the FP8 (MXFP8) attention oracle (no GPU).

Each pin checks oracle.fp8 against something other than itself: the OCP OFP8
E4M3 value table (published facts: largest finite 448, smallest normal 2^-6,
smallest subnormal 2^-9, NaN at S.1111.111, no infinities), brute-force
nearest rounding over the whole E4M3 grid, the defining inequality of the
block-scale rule, hand-built block examples, closed forms of the attention
(constant V, identical keys, T = 1) and a pure-Python brute force of the whole
forward. ``test_planted_mistakes_are_caught`` plants plausible mistakes in the
oracle and shows that each fails at least one pin.
"""

import math
from contextlib import ExitStack
from unittest import mock

import numpy as np
import pytest

import oracle.attention as A
import oracle.fp8 as F

RNG = np.random.default_rng(20241203)
LOG2E = 1.0 / math.log(2.0)


# ----------------------------------------------------------------------------
# Brute-force helpers, independent of oracle.fp8's algorithms: the grid is
# listed value by value, rounding is a nearest search, and the scale exponent
# is found by stepping e upward.
# ----------------------------------------------------------------------------

def _grid():
    """(value, code) of every non-negative finite E4M3 number, ascending."""
    out = [(m * 2.0 ** -9, m) for m in range(8)]                 # subnormals and 0
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue                                          # NaN
            out.append(((8 + m) * 2.0 ** (e - 10), (e << 3) | m))
    return out


GRID = _grid()
GRID_V = np.array([g[0] for g in GRID])
GRID_C = np.array([g[1] for g in GRID])


def _nearest_code(x):
    """Brute-force RNE: the grid value nearest |x|; on a tie the even code."""
    a = abs(x)
    d = np.abs(GRID_V - a)
    best = np.nonzero(d == d.min())[0]
    if len(best) > 1:
        best = [i for i in best if GRID_C[i] % 2 == 0]
    code = int(GRID_C[best[0]])
    return code | (0x80 if math.copysign(1.0, x) < 0 else 0)


def _nearest_value(x):
    i = int(np.argmin(np.abs(GRID_V - abs(x))))
    d = np.abs(GRID_V - abs(x))
    ties = np.nonzero(d == d.min())[0]
    if len(ties) > 1:
        i = [j for j in ties if GRID_C[j] % 2 == 0][0]
    return math.copysign(GRID_V[i], x)


def _scale_exp_search(amax):
    if amax == 0:
        return -127
    e = -127
    while e < 127 and amax > 448.0 * 2.0 ** e:
        e += 1
    return e


def _quant_list(vals):
    """Brute-force MX quantization of one block (a list of floats)."""
    e = _scale_exp_search(max(abs(v) for v in vals))
    return [_nearest_value(v / 2.0 ** e) * 2.0 ** e for v in vals], e


def _brute_forward(q, k, v):
    """Steps 1-7 in pure-Python loops from the brute-force helpers."""
    T, d = q.shape
    qd = np.zeros((T, d))
    kd = np.zeros((T, d))
    for t in range(T):
        for c0 in range(0, d, 32):
            qd[t, c0:c0 + 32] = _quant_list(list(q[t, c0:c0 + 32]))[0]
            kd[t, c0:c0 + 32] = _quant_list(list(k[t, c0:c0 + 32]))[0]
    Tp = -(-T // 32) * 32
    vd = np.zeros((Tp, d))
    vp = np.zeros((Tp, d))
    vp[:T] = v
    for c in range(d):
        for t0 in range(0, Tp, 32):
            vd[t0:t0 + 32, c] = _quant_list(list(vp[t0:t0 + 32, c]))[0]
    o = np.zeros((T, d))
    lse = np.zeros(T)
    for i in range(T):
        z = []
        for j in range(i + 1):
            s = 0.0
            for c in range(d):
                s += qd[i, c] * kd[j, c]
            z.append(s / math.sqrt(d) * LOG2E)
        m = math.ceil(max(z))
        w = [_nearest_value(2.0 ** (zz - m + 8)) * 2.0 ** -8 for zz in z]
        l = sum(w)
        for c in range(d):
            o[i, c] = sum(w[j] * vd[j, c] for j in range(i + 1)) / l
        lse[i] = math.log(2.0) * (m + math.log2(l))
    return o, lse


# ----------------------------------------------------------------------------
# Pins
# ----------------------------------------------------------------------------

def pin_e4m3_table(M):
    """OFP8 E4M3 facts: named codes, 254 finite codes, order and symmetry."""
    facts = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x30: 0.5, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0,
             0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    v = M.e4m3_decode(np.arange(256))
    for c, x in facts.items():
        assert v[c] == x, (hex(c), v[c], x)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isnan(v).sum() == 2
    assert math.copysign(1.0, v[0x80]) < 0 and v[0x80] == 0
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[0x80:0xFF], -pos)


def pin_e4m3_rounding(M):
    """Encoding equals brute-force nearest with ties to the even code, on grid
    values, exact midpoints, values beside them and random magnitudes."""
    xs = list(GRID_V)
    xs += [0.5 * (a + b) for a, b in zip(GRID_V[:-1], GRID_V[1:])]
    xs += [np.nextafter(0.5 * (a + b), 0.0) for a, b in zip(GRID_V[:-1], GRID_V[1:])]
    xs += [np.nextafter(0.5 * (a + b), 1e9) for a, b in zip(GRID_V[:-1], GRID_V[1:])]
    xs += list(np.exp2(RNG.uniform(-12, math.log2(448), 400)))
    xs = np.array(xs)
    xs = np.concatenate([xs, -xs[1:]])
    got = M.e4m3_encode(xs)
    want = np.array([_nearest_code(float(x)) for x in xs], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert len(bad) == 0, [(float(xs[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]
    # decode(encode(x)) is the nearest grid value
    dec = M.e4m3_decode(got)
    assert np.all(np.abs(dec - xs) <= np.abs(xs) * 2.0 ** -4 + 2.0 ** -10)


def pin_e4m3_range(M):
    """Arguments beyond +-448 or NaN are caller errors; +-448 encode exactly."""
    for bad in (448.5, -449.0, 1e9, float("nan"), float("inf")):
        try:
            M.e4m3_encode(np.array([bad]))
        except ValueError:
            continue
        raise AssertionError(f"encode accepted {bad}")
    assert M.e4m3_encode(np.array([448.0, -448.0])).tolist() == [0x7E, 0xFE]


def pin_scale_rule(M):
    """e is the smallest integer with amax <= 448 * 2^e (checked against a
    step-by-step search and the inequality), 0 gives -127."""
    a = np.concatenate([np.exp2(RNG.uniform(-100, 100, 300)),
                        [1.0, 1.75, 1.75 * (1 + 2 ** -52), 2.0, 3.5, 448.0, 449.0, 0.875]])
    e = M.mx_scale_exponent(a)
    for x, ee in zip(a, e):
        assert ee == _scale_exp_search(x), (x, ee)
        assert x <= 448.0 * 2.0 ** ee and x > 448.0 * 2.0 ** (ee - 1)
    assert M.mx_scale_exponent(np.array([0.0]))[0] == -127
    assert M.mx_scale_exponent(np.array([1e-45]))[0] == -127


def pin_blocks_hand_built(M):
    """Q blocks run along channels, V blocks along positions (T = 40 pads
    to 64 with zeros); codes and exponents worked out by hand."""
    T, d = 40, 64
    q = np.ones((T, d))
    q[:, 32:] = 0.0
    q[0, 5] = 3.0            # block (0, 0): amax 3 -> e = -7 (1.75 < 3 <= 3.5)
    k = np.ones((T, d))
    v = np.zeros((T, d))
    v[3, 7] = 1000.0         # V block (0, 7): 1000 = 1.95 * 2^9 -> e = 2; 250 -> 256 (0x78)
    v[35, 7] = 0.01          # V block (1, 7): 0.01 = 1.28 * 2^-7 -> e = -15; 327.68 -> 320 (0x7A)
    v[35, 8] = 1000.0        # same position, next channel: would crush 0.01 into the
                             # subnormals if the blocks ran along channels
    r = M.quantize_head(q, k, v)
    assert r["q_exp"].shape == (T, 2) and r["v_exp"].shape == (2, d)
    assert r["v_codes"].shape == (64, d)
    assert r["q_exp"][0, 0] == -7 and r["q_exp"][0, 1] == -127 and r["q_exp"][1, 0] == -8
    assert r["q_codes"][0, 5] == 0x7C          # 3 * 2^7 = 384 = 1.5 * 2^8
    assert r["q_codes"][0, 0] == 0x70          # 2^7
    assert r["q_codes"][1, 0] == 0x78          # 1 * 2^8 = 256
    assert r["v_exp"][0, 7] == 2 and r["v_codes"][3, 7] == 0x78
    assert r["v_exp"][1, 7] == -15 and r["v_codes"][35, 7] == 0x7A
    assert r["v_exp"][0, 6] == -127 and r["v_exp"][1, 9] == -127 and r["v_exp"][1, 8] == 2
    assert np.all(r["v_codes"][40:] == 0)
    assert r["v"].shape == (T, d)
    assert r["v"][3, 7] == 1024.0 and r["v"][35, 7] == 320.0 * 2.0 ** -15


def pin_constant_v(M):
    """Every row of V equal: each output row is that (quantized) row exactly,
    since the weights are normalised by their own sum."""
    T, d = 50, 64
    q, k = RNG.standard_normal((2, T, d))
    w = RNG.standard_normal(d)
    v = np.tile(w, (T, 1))
    o, _ = M.head_forward_fp8(q, k, v)
    wq = np.array([_quant_list([w[c]] * 32)[0][0] for c in range(d)])
    assert np.allclose(o, wq[None, :], rtol=1e-14, atol=0), np.abs(o - wq).max()


def pin_t1(M):
    """T = 1: O = V^_0; LSE = ln 2 (m + log2 P^) with m = ceil(z), worked
    out from brute-force quantization."""
    for _ in range(5):
        q, k, v = RNG.standard_normal((3, 1, 64)) * RNG.uniform(0.2, 4)
        o, lse = M.head_forward_fp8(q, k, v)
        qd = np.concatenate([_quant_list(list(q[0, :32]))[0], _quant_list(list(q[0, 32:]))[0]])
        kd = np.concatenate([_quant_list(list(k[0, :32]))[0], _quant_list(list(k[0, 32:]))[0]])
        vd = np.array([_quant_list([v[0, c]] + [0.0] * 31)[0][0] for c in range(64)])
        z = float(qd @ kd) / 8.0 * LOG2E
        m = math.ceil(z)
        p = _nearest_value(2.0 ** (z - m + 8)) * 2.0 ** -8
        assert np.allclose(o[0], vd, rtol=1e-15, atol=0)
        assert abs(lse[0] - math.log(2.0) * (m + math.log2(p))) < 1e-12


def pin_identical_keys(M):
    """All keys equal: row i's weights are equal, so O_i is the mean of
    V^_0..i and LSE_i = ln 2 (m_i + log2((i + 1) P^_i))."""
    T, d = 40, 64
    q = RNG.standard_normal((T, d))
    k = np.tile(RNG.standard_normal(d), (T, 1))
    v = RNG.standard_normal((T, d))
    o, lse, parts = M.head_forward_fp8(q, k, v, return_parts=True)
    Tp = 64
    vp = np.zeros((Tp, d))
    vp[:T] = v
    vq = np.zeros((Tp, d))
    for c in range(d):
        for t0 in (0, 32):
            vq[t0:t0 + 32, c] = _quant_list(list(vp[t0:t0 + 32, c]))[0]
    kq = np.concatenate([_quant_list(list(k[0, :32]))[0], _quant_list(list(k[0, 32:]))[0]])
    for i in range(T):
        qi = np.concatenate([_quant_list(list(q[i, :32]))[0], _quant_list(list(q[i, 32:]))[0]])
        z = float(qi @ kq) / 8.0 * LOG2E
        m = math.ceil(z)
        p = _nearest_value(2.0 ** (z - m + 8)) * 2.0 ** -8
        assert np.allclose(o[i], vq[:i + 1].mean(axis=0), rtol=1e-12, atol=1e-14)
        assert abs(lse[i] - math.log(2.0) * (m + math.log2((i + 1) * p))) < 1e-12


def pin_brute_force(M):
    """The whole forward against pure-Python loops on small heads."""
    for T, std in ((5, 1.0), (9, 3.0), (33, 0.5)):
        q, k, v = RNG.standard_normal((3, T, 64)) * std
        o, lse = M.head_forward_fp8(q, k, v)
        ob, lb = _brute_forward(q, k, v)
        assert np.allclose(o, ob, rtol=1e-12, atol=1e-13), np.abs(o - ob).max()
        assert np.allclose(lse, lb, rtol=1e-12, atol=1e-12)


def pin_near_exact_attention(M):
    """FP8 stays within a few percent of exact attention on the unquantized
    inputs (E4M3 keeps 4 significant bits: 2^-4 relative per element)."""
    T = 200
    q, k, v = RNG.standard_normal((3, T, 64))
    o, lse = M.head_forward_fp8(q, k, v)
    oe, le = A.head_forward(q, k, v)
    rel = np.linalg.norm(o - oe) / np.linalg.norm(oe)
    assert 0 < rel < 0.08, rel
    assert np.abs(lse - le).max() < 0.1


def pin_packed_layout(M):
    """forward_packed_fp8 reads [Q | K | V] blocks with head h at columns
    h*d .. h*d + d - 1 and writes out (B, T, C), lse (B, H, T)."""
    B, T, H, d = 2, 20, 3, 64
    C = H * d
    qkv = RNG.standard_normal((B, T, 3 * C))
    out, lse = M.forward_packed_fp8(qkv, H, d)
    for b in range(B):
        for h in range(H):
            q = qkv[b, :, h * d:(h + 1) * d]
            k = qkv[b, :, C + h * d:C + (h + 1) * d]
            v = qkv[b, :, 2 * C + h * d:2 * C + (h + 1) * d]
            ob, lb = _brute_forward(q, k, v)
            assert np.allclose(out[b, :, h * d:(h + 1) * d], ob, rtol=1e-12, atol=1e-13)
            assert np.allclose(lse[b, h], lb, rtol=1e-12, atol=1e-12)


def pin_rounding_slack(M):
    """Slack is zero when no weight is small or near a midpoint, and equals
    2^-17 |V^_0 - O_1| / (l_1 - 2^-17) for one tiny weight (hand derived)."""
    d = 64
    q = np.zeros((2, d))
    k = np.zeros((2, d))
    q[:, 0] = 1.0
    k[1, 0] = 1.0                  # z_11 = log2e/8, z_10 = 0, z_00 = 0
    v = RNG.standard_normal((2, d))
    _, _, parts = M.head_forward_fp8(q, k, v, return_parts=True)
    os_, ls_ = M.rounding_slack(parts)
    assert np.all(os_ == 0) and np.all(ls_ == 0)
    k[0, 0] = -150.0               # z_10 = -150 log2e / 8, about -27: a tiny weight
    _, _, parts = M.head_forward_fp8(q, k, v, return_parts=True)
    os_, ls_ = M.rounding_slack(parts)
    o1 = (parts["p_hat"][1] @ parts["v"]) / parts["l"][1]
    want = 2.0 ** -17 * np.abs(parts["v"][0] - o1).max() / (parts["l"][1] - 2.0 ** -17)
    assert os_[0] == 0 and abs(os_[1] - want) <= 1e-15 * want
    assert abs(ls_[1] - 2.0 ** -17 / (parts["l"][1] - 2.0 ** -17)) < 1e-18


def pin_rounding_slack_near_midpoint(M):
    """Branch (b) of the slack: a code whose argument lies within the
    kernel's error of an E4M3 rounding midpoint, worked by hand.

    T = 2, only channels 0 and 1 non-zero: q_0 = 0, q_1 = (1, 1);
    k_0 = (0.3125, -22), k_1 = 0; v_0 = (1, 0, ...), v_1 = 0. Every value has
    at most four significant bits, so each MX block holds it exactly
    (k_0's block takes e = -4: 5 and -352 are E4M3 codes).

    Row 1: z_11 = 0 and z_10 = (0.3125 - 22) log2(e) / 8 = -3.9115, so the
    reference is m_1 = ceil(0) = 0 and the arguments 2^(z - m + 8) are
    x_11 = 256 (a grid value) and x_10 = 17.01746, just above the midpoint 17
    between the E4M3 neighbours 16 and 18 (it rounds to 18: P^_10 = 18/256,
    l_1 = 274/256). The pair's largest product is |k_0,1 q_1,1| = 22, so the
    allowed relative error of x is 2^-11 * 22 / 8 + 2^-20 = 1.3437e-3, and
    |x_10 - 17| / x_10 = 1.0261e-3 lies inside it: that code may move by one
    grid step, 2 / 256. With the moved weight w = 2^-7:
      lse_slack_1 = w / (l_1 - w) = (2/256) / (272/256) = 1/136,
      O_1 = (18/256 v_0) / l_1 = 18/274 v_0, spread max_c |v_0c - O_1c| =
      256/274, so o_slack_1 = w * 256/274 / (272/256) = 512 / (274 * 272).
    Row 0 (one key, x = 256) and code x_11 are on the grid: no slack.

    A second head with k_0 = (0.34375, -22) puts x_10 = 17.08407 at
    4.92e-3 relative from the midpoint, 3.7 times the allowed error: no
    slack anywhere. (The earlier sum-scaled model, 2^-13 * 22.3125 / 8, would
    allow only 3.41e-4 in the first case, and a bound without the 1/sqrt(d)
    would take in the second.)"""
    d = 64

    def slack(k01):
        q = np.zeros((2, d))
        k = np.zeros((2, d))
        v = np.zeros((2, d))
        q[1, 0] = q[1, 1] = 1.0
        k[0, 0], k[0, 1] = k01, -22.0
        v[0, 0] = 1.0
        _, _, parts = M.head_forward_fp8(q, k, v, return_parts=True)
        assert parts["p_hat"][1, 0] == 18.0 / 256.0 and parts["p_hat"][1, 1] == 1.0
        return M.rounding_slack(parts)

    os_, ls_ = slack(0.3125)
    assert os_[0] == 0 and ls_[0] == 0
    assert abs(ls_[1] - 1.0 / 136.0) <= 1e-15
    assert abs(os_[1] - 512.0 / (274.0 * 272.0)) <= 1e-15
    os_, ls_ = slack(0.34375)
    assert np.all(os_ == 0) and np.all(ls_ == 0)


def _brute_backward(q, k, v, g, o, lse):
    """FP8 backward steps B1-B6 in pure-Python loops from the brute-force
    quantizers."""
    T, d = q.shape
    Tp = -(-T // 32) * 32

    def chan(x):
        out = np.zeros((T, d))
        for t in range(T):
            for c0 in range(0, d, 32):
                out[t, c0:c0 + 32] = _quant_list(list(x[t, c0:c0 + 32]))[0]
        return out

    def pos(x):
        pad = np.zeros((Tp, d))
        pad[:T] = x
        out = np.zeros((Tp, d))
        for c in range(d):
            for t0 in range(0, Tp, 32):
                out[t0:t0 + 32, c] = _quant_list(list(pad[t0:t0 + 32, c]))[0]
        return out[:T]

    qc, kc, vc, gc = chan(q), chan(k), chan(v), chan(g)
    qp, kp, gp = pos(q), pos(k), pos(g)
    p = np.zeros((T, T))
    ph = np.zeros((T, T))
    ds = np.zeros((T, T))
    for i in range(T):
        dd = sum(g[i, c] * o[i, c] for c in range(d))
        for j in range(i + 1):
            z = sum(qc[i, c] * kc[j, c] for c in range(d)) / math.sqrt(d) * LOG2E
            p[i, j] = 2.0 ** (z - lse[i] * LOG2E)
            ph[i, j] = _nearest_value(p[i, j] * 256.0) / 256.0
            dp = sum(gc[i, c] * vc[j, c] for c in range(d))
            ds[i, j] = p[i, j] * (dp - dd)
    dsq = np.zeros((Tp, Tp))   # blocks of 32 queries of one key
    dsk = np.zeros((Tp, Tp))   # blocks of 32 keys of one query
    pad = np.zeros((Tp, Tp))
    pad[:T, :T] = ds
    for a in range(Tp):
        for b0 in range(0, Tp, 32):
            dsq[b0:b0 + 32, a] = _quant_list(list(pad[b0:b0 + 32, a]))[0]
            dsk[a, b0:b0 + 32] = _quant_list(list(pad[a, b0:b0 + 32]))[0]
    dv = np.zeros((T, d))
    dk = np.zeros((T, d))
    dq = np.zeros((T, d))
    for j in range(T):
        for c in range(d):
            dv[j, c] = sum(ph[i, j] * gp[i, c] for i in range(j, T))
            dk[j, c] = sum(dsq[i, j] * qp[i, c] for i in range(j, T)) / math.sqrt(d)
    for i in range(T):
        for c in range(d):
            dq[i, c] = sum(dsk[i, j] * kp[j, c] for j in range(i + 1)) / math.sqrt(d)
    return dq, dk, dv


def pin_backward_brute_force(M):
    """The FP8 backward against pure-Python loops (forward outputs from the
    brute force too)."""
    cases = [RNG.standard_normal((4, T, 64)) * std for T, std in ((5, 1.0), (9, 2.0), (33, 0.7))]
    # elements spread over 2^-10 .. 2^10 (Q and K less, to keep the scores
    # moderate): block scales then differ between channel and position blocks
    wide = RNG.standard_normal((4, 20, 64)) * np.exp2(RNG.integers(-10, 11, (4, 20, 64)))
    wide[:2] *= 2.0 ** -8
    cases.append(wide)
    for q, k, v, g in cases:
        o, lse = _brute_forward(q, k, v)
        dq, dk, dv = M.head_backward_fp8(q, k, v, g, o, lse)
        bq, bk, bv = _brute_backward(q, k, v, g, o, lse)
        for a, b, name in ((dq, bq, "dq"), (dk, bk, "dk"), (dv, bv, "dv")):
            assert np.allclose(a, b, rtol=1e-10, atol=1e-12), (name, np.abs(a - b).max())


def pin_backward_zero_upstream(M):
    """dO = 0: every gradient is exactly zero."""
    T = 20
    q, k, v = RNG.standard_normal((3, T, 64))
    o, lse = M.head_forward_fp8(q, k, v)
    for x in M.head_backward_fp8(q, k, v, np.zeros((T, 64)), o, lse):
        assert np.all(x == 0)


def pin_backward_near_exact(M):
    """The FP8 backward stays within about 2^-3 (relative L2) of the exact
    gradients on the unquantized inputs."""
    T = 150
    q, k, v, g = RNG.standard_normal((4, T, 64))
    o, lse = M.head_forward_fp8(q, k, v)
    got = M.head_backward_fp8(q, k, v, g, o, lse)
    ref = A.head_backward(q, k, v, g)
    for a, b in zip(got, ref):
        rel = np.linalg.norm(a - b) / np.linalg.norm(b)
        assert 0 < rel < 0.12, rel


PINS = [
    pin_e4m3_table,
    pin_e4m3_rounding,
    pin_e4m3_range,
    pin_scale_rule,
    pin_blocks_hand_built,
    pin_constant_v,
    pin_t1,
    pin_identical_keys,
    pin_brute_force,
    pin_near_exact_attention,
    pin_packed_layout,
    pin_rounding_slack,
    pin_rounding_slack_near_midpoint,
    pin_backward_brute_force,
    pin_backward_zero_upstream,
    pin_backward_near_exact,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_fp8_oracle_pin(pin):
    pin(F)


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------

_orig = {name: getattr(F, name) for name in
         ("e4m3_decode", "e4m3_encode", "mx_scale_exponent", "quantize_head", "_logits",
          "_probabilities", "head_forward_fp8", "_dot_error_bound", "_e4m3_neighbours")}


def _dot_error_sum_scaled(q, k, dot_max_err):
    """The slack's earlier error model: 2^-13 of the sum of the products'
    magnitudes."""
    return 2.0 ** -13 * (np.abs(q) @ np.abs(k).T)


def _dot_error_no_sqrt_d(q, k, dot_max_err):
    """The right bound on the dot product taken as the bound on the logit
    (the 1/sqrt(d) forgotten)."""
    return _orig["_dot_error_bound"](q, k, dot_max_err) * math.sqrt(q.shape[1])


def _neighbours_from_code(x):
    """The grid neighbours taken as the rounded value and the next one up,
    whichever side of x the rounded value lies."""
    code = F.e4m3_encode(x).astype(np.int64)
    return F.e4m3_decode(code), F.e4m3_decode(np.minimum(code + 1, 0x7E))


def _decode_bias8(codes):
    c = np.asarray(codes, dtype=np.int64)
    return _orig["e4m3_decode"](c) * 0.5


def _encode_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    out = _orig["e4m3_encode"](x)
    dec = _orig["e4m3_decode"](out)
    over = np.abs(dec) > np.abs(x)
    return np.where(over & ((out & 0x7F) > 0), out - 1, out).astype(np.uint8)


def _encode_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    out = _orig["e4m3_encode"](x).astype(np.int64)
    dec = _orig["e4m3_decode"](out)
    up = _orig["e4m3_decode"](np.minimum((out & 0x7F) + 1, 0x7E) | (out & 0x80))
    down = _orig["e4m3_decode"](np.maximum((out & 0x7F) - 1, 0) | (out & 0x80))
    tie_up = np.abs(np.abs(up) - np.abs(x)) == np.abs(np.abs(dec) - np.abs(x))
    tie_dn = np.abs(np.abs(down) - np.abs(x)) == np.abs(np.abs(dec) - np.abs(x))
    bump = tie_up & (np.abs(up) > np.abs(dec)) & (np.abs(dec) != np.abs(x))
    out = np.where(bump, out + 1, out)
    out = np.where(tie_dn & (np.abs(down) > np.abs(dec)), out - 1, out)
    return out.astype(np.uint8)


def _scale_floor_rule(amax):
    a = np.asarray(amax, dtype=np.float64)
    fr, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.where(a > 0, ex - 1 - 8, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def _quantize_v_along_channels(q, k, v):
    r = _orig["quantize_head"](q, k, v)
    vc, ve, vd = F.quantize_blocks(np.asarray(v, dtype=np.float64), axis=1)
    r["v"] = vd
    return r


def _logits_natural(qd, kd):
    return _orig["_logits"](qd, kd) / LOG2E


def _logits_k_q(qd, kd):
    return _orig["_logits"](kd, qd).T.copy() if qd.shape[0] == 1 else _orig["_logits"](kd, qd)


def _logits_no_mask(qd, kd):
    T, d = qd.shape
    return (LOG2E / math.sqrt(d)) * (qd @ kd.T)


def _probabilities_m_max(z):
    m = z.max(axis=1, keepdims=True)
    x = np.exp2(z - m + 8)
    return m[:, 0], F.e4m3_decode(F.e4m3_encode(x)) * 2.0 ** -8


def _probabilities_unquantized(z):
    m = np.ceil(z.max(axis=1, keepdims=True))
    return m[:, 0], np.exp2(z - m)


def _forward_variant(kind):
    def f(q, k, v, return_parts=False):
        qz = F.quantize_head(q, k, v)
        z = F._logits(qz["q"], qz["k"])
        m, p_hat = F._probabilities(z)
        l = p_hat.sum(axis=1)
        if kind == "l_unquantized":
            l = np.exp2(z - m[:, None]).sum(axis=1)
        o = (p_hat @ qz["v"]) / l[:, None]
        lse = math.log(2.0) * (m + np.log2(l))
        if kind == "lse_natural_m":
            lse = m + np.log(l)
        if kind == "lse_no_shift_undo":
            lse = math.log(2.0) * (m + np.log2(l * 256.0))
        if return_parts:
            parts = dict(qz)
            parts.update({"z": z, "m": m, "p_hat": p_hat, "l": l})
            return o, lse, parts
        return o, lse
    return f


def _backward_variant(kind):
    def f(q, k, v, g, o, lse, return_parts=False):
        q, k, v, g, o = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, o))
        T, d = q.shape
        qc, kc, vc, gc = (F.quantize_blocks(a, axis=1)[2] for a in (q, k, v, g))
        qp, kp, gp = (F.quantize_positions(a)[2] for a in (q, k, g))
        if kind == "dk_q_channel_blocks":
            qp = qc
        if kind == "dv_g_channel_blocks":
            gp = gc
        z = F._logits(qc, kc)
        p = np.exp2(z - LOG2E * np.asarray(lse)[:, None])
        p_hat = F.e4m3_decode(F.e4m3_encode(p * 256.0)) / 256.0
        dv = (p if kind == "dv_unquantized_p" else p_hat).T @ gp
        dp = gc @ vc.T
        dd = (g * o).sum(axis=1)
        ds = (p_hat if kind == "ds_quantized_p" else p) * (dp - dd[:, None])
        if kind == "ds_no_d":
            ds = p * dp
        sc = 1.0 / math.sqrt(d)
        ax_k, ax_q = (1, 0) if kind == "ds_blocks_swapped" else (0, 1)
        dk = sc * (F._quantize_rows_along(ds, axis=ax_k).T @ qp)
        dq = sc * (F._quantize_rows_along(ds, axis=ax_q) @ kp)
        if kind == "dq_no_scale":
            dq = dq / sc
        return dq, dk, dv
    return f


MUTANTS = {
    "bwd_dv_unquantized_p": {"head_backward_fp8": _backward_variant("dv_unquantized_p")},
    "bwd_ds_from_quantized_p": {"head_backward_fp8": _backward_variant("ds_quantized_p")},
    "bwd_ds_without_d": {"head_backward_fp8": _backward_variant("ds_no_d")},
    "bwd_ds_blocks_swapped": {"head_backward_fp8": _backward_variant("ds_blocks_swapped")},
    "bwd_dk_q_channel_blocks": {"head_backward_fp8": _backward_variant("dk_q_channel_blocks")},
    "bwd_dv_g_channel_blocks": {"head_backward_fp8": _backward_variant("dv_g_channel_blocks")},
    "bwd_dq_no_scale": {"head_backward_fp8": _backward_variant("dq_no_scale")},
    "decode_bias_8": {"e4m3_decode": _decode_bias8},
    "encode_truncates": {"e4m3_encode": _encode_truncate},
    "encode_ties_away": {"e4m3_encode": _encode_ties_away},
    "scale_floor_rule": {"mx_scale_exponent": _scale_floor_rule},
    "v_blocks_along_channels": {"quantize_head": _quantize_v_along_channels},
    "logits_natural_base": {"_logits": _logits_natural},
    "logits_k_q_swapped": {"_logits": _logits_k_q},
    "logits_no_mask": {"_logits": _logits_no_mask},
    "reference_not_integer": {"_probabilities": _probabilities_m_max},
    "p_not_quantized": {"_probabilities": _probabilities_unquantized},
    "l_from_unquantized_p": {"head_forward_fp8": _forward_variant("l_unquantized")},
    "lse_natural_m": {"head_forward_fp8": _forward_variant("lse_natural_m")},
    "lse_keeps_2^8": {"head_forward_fp8": _forward_variant("lse_no_shift_undo")},
    "slack_sum_scaled_error": {"_dot_error_bound": _dot_error_sum_scaled},
    "slack_without_sqrt_d": {"_dot_error_bound": _dot_error_no_sqrt_d},
    "slack_wrong_neighbour": {"_e4m3_neighbours": _neighbours_from_code},
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name):
    failed = []
    with ExitStack() as stack:
        for attr, repl in MUTANTS[name].items():
            stack.enter_context(mock.patch.object(F, attr, repl))
        for pin in PINS:
            try:
                with np.errstate(all="ignore"):
                    pin(F)
            except (AssertionError, ValueError, FloatingPointError, IndexError):
                failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
