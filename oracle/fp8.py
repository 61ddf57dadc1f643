"""CPU float64 oracle of the FP8 (MXFP8) causal attention forward.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import or call this module; the product
path never does, and it imports nothing from the product.

Why an FP8 variant
------------------
The llm.c page ("Réimplémenter à bas coût le modèle GPT-2 avec llm.c", FAQ)
states that training runs in BF16 and that FP8 support is planned, and says
nothing more about it. The FP8 variant built here is therefore defined by this
module, from two published formats and the attention definition of
``oracle.attention``:

* OCP 8-bit floating point (OFP8) E4M3: sign, 4 exponent bits (bias 7),
  3 mantissa bits; subnormals at exponent field 0 (m/8 * 2^-6); 0x7F and 0xFF
  are NaN; no infinities; largest finite 448. Conversion rounds to nearest,
  ties to even.
* OCP Microscaling (MX) v1.0: 32 consecutive elements share one E8M0 scale
  2^e (stored as the byte e + 127), element value = code value * 2^e.

The variant, step by step (one head, T positions, d = 64 channels):

1. Block scales. For a block with largest magnitude a, e is the smallest
   integer with a <= 448 * 2^e, clamped to [-127, 127]; a block of zeros takes
   e = -127. So no scaled element exceeds 448 and none saturates. (The MX
   document's own suggestion, floor(log2 a) - 8, can leave elements above 448
   that must then be clamped; this policy avoids that at the cost of at most
   one binade of range.)
2. Blocks. Q and K: per position, channels [0, 32) and [32, 64) (the blocks
   run along the contraction of Q K^T). V: per channel, positions
   [32j, 32j + 32) with positions at or past T read as zero (the blocks run
   along the contraction of P V).
3. Elements: code = E4M3(x / 2^e); the dequantized value is code * 2^e.
4. Base-2 logits of the dequantized operands: z_ij = log2(e) * Q^_i . K^_j /
   sqrt(d) for j <= i (keys after the query are excluded).
5. Row reference m_i = ceil(max_j z_ij), an integer.
6. Probabilities on the FP8 grid: P^_ij = E4M3(2^(z_ij - m_i + 8)) * 2^-8.
   The argument lies in (0, 256], so the code never saturates.
7. l_i = sum_j P^_ij;  O_i = sum_j P^_ij V^_j / l_i;
   LSE_i = ln 2 * (m_i + log2 l_i), the log-normaliser of the weights that O
   actually uses.

Step 5 makes every rescale between two integer references an exact power of
two, and E4M3 rounding commutes with powers of two in its normal range, so a
streaming kernel whose running reference only grows reaches the same P^ as
step 6 except (a) for probabilities below 2^-13 (E4M3 subnormals at one of
the two references) and (b) where the kernel's logit, computed with rounding
error, puts 2^(z - m + 8) on the other side of a rounding midpoint.
``rounding_slack`` bounds what those two cases can change, given a bound on
that rounding error.

The backward (head_backward_fp8) keeps the same formats: every product runs
on MXFP8 operands blocked along that product's own contraction (channels for
Q K^T and dO V^T, positions for P^T dO, dS^T Q and dS K), the probabilities
on the forward's fixed 2^-8 grid and dS on the block-scale rule of step 1.

Pins: tests/test_oracle_fp8.py checks the encoding against the OFP8 table and
brute-force nearest rounding, the scale rule against its defining inequality,
the blocks against hand-built examples, and the attention against closed forms
(constant V, identical keys, T = 1) and a pure-Python brute force, and shows
that planted mistakes fail at least one of them.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "E4M3_MAX",
    "MX_BLOCK",
    "e4m3_decode",
    "e4m3_encode",
    "mx_scale_exponent",
    "quantize_blocks",
    "quantize_head",
    "head_forward_fp8",
    "forward_packed_fp8",
    "quantize_positions",
    "head_backward_fp8",
    "backward_packed_fp8",
    "rounding_slack",
]

E4M3_MAX = 448.0
MX_BLOCK = 32
P_SHIFT = 8          # step 6: probabilities are encoded as 2^8 * p
LOG2E = 1.0 / math.log(2.0)


def e4m3_decode(codes) -> np.ndarray:
    """Values of E4M3 codes (OFP8): float64, NaN for 0x7F / 0xFF."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """E4M3 codes of x, round to nearest, ties to even (uint8).

    |x| must not exceed 448 and x must not be NaN: the block-scale policy never
    produces such an argument, so one is a caller error (ValueError).
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or (np.abs(x) > E4M3_MAX).any():
        raise ValueError("E4M3 argument outside [-448, 448]")
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.abs(x)
    # Normal range: a = f * 2^E with f in [1, 2); 8 f rounded (ties to even by
    # np.rint) gives 8 + mantissa, or 16 when it rounds up into the next binade.
    fr, ex = np.frexp(np.where(a > 0, a, 1.0))      # a = fr * 2^ex, fr in [0.5, 1)
    E = ex - 1
    n = np.rint(fr * 16.0).astype(np.int64)         # 8 f in [8, 16]
    E = np.where(n == 16, E + 1, E)
    n = np.where(n == 16, 8, n)
    normal = ((E + 7) << 3) | (n - 8)
    # Subnormal range (a < 2^-6): multiples of 2^-9, ties to even; 8 * 2^-9
    # is the smallest normal, whose code (0x08) follows on.
    sub = np.rint(a * 2.0 ** 9).astype(np.int64)
    code = np.where(a < 2.0 ** -6, sub, normal)
    return (sign | code).astype(np.uint8)


def mx_scale_exponent(amax) -> np.ndarray:
    """Step 1: the smallest integer e with amax <= 448 * 2^e, in [-127, 127].

    amax = 0 gives -127. Exact: with amax = f * 2^E, f in [1, 2),
    448 * 2^(E - 8) = 1.75 * 2^E, so e = E - 8 when f <= 1.75, else E - 7.
    """
    a = np.asarray(amax, dtype=np.float64)
    fr, ex = np.frexp(np.where(a > 0, a, 1.0))      # fr in [0.5, 1)
    E = ex - 1
    e = np.where(2.0 * fr <= 1.75, E - 8, E - 7)
    e = np.where(a > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_blocks(x: np.ndarray, axis: int):
    """MX quantization of x in blocks of 32 along ``axis`` (a multiple of 32).

    Returns (codes uint8 shaped like x, exponents int64 with ``axis`` divided
    by 32, dequantized float64 shaped like x).
    """
    x = np.asarray(x, dtype=np.float64)
    xm = np.moveaxis(x, axis, -1)
    n = xm.shape[-1]
    if n % MX_BLOCK:
        raise ValueError("blocked axis must be a multiple of 32")
    blocks = xm.reshape(xm.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    e = mx_scale_exponent(np.abs(blocks).max(axis=-1))
    scale = np.exp2(e.astype(np.float64))[..., None]
    codes = e4m3_encode(blocks / scale)
    deq = e4m3_decode(codes) * scale
    codes = np.moveaxis(codes.reshape(xm.shape), -1, axis)
    deq = np.moveaxis(deq.reshape(xm.shape), -1, axis)
    e = np.moveaxis(e, -1, axis)
    return codes, e, deq


def quantize_head(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    """Steps 2-3 for one head: q, k, v are (T, d) with d a multiple of 32.

    Returns a dict with codes and exponents: q_codes, k_codes (T, d) and
    q_exp, k_exp (T, d/32) blocked along channels; v_codes (Tp, d) and
    v_exp (Tp/32, d) blocked along positions, with Tp = round_up(T, 32) and
    the padding positions zero; and the dequantized q, k (T, d), v (T, d).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, d = q.shape
    qc, qe, qd = quantize_blocks(q, axis=1)
    kc, ke, kd = quantize_blocks(k, axis=1)
    Tp = -(-T // MX_BLOCK) * MX_BLOCK
    vpad = np.zeros((Tp, d))
    vpad[:T] = v
    vc, ve, vd = quantize_blocks(vpad, axis=0)
    return {"q_codes": qc, "q_exp": qe, "k_codes": kc, "k_exp": ke,
            "v_codes": vc, "v_exp": ve, "q": qd, "k": kd, "v": vd[:T]}


def _logits(qd: np.ndarray, kd: np.ndarray) -> np.ndarray:
    """Step 4: base-2 causal logits, -inf for keys after the query."""
    T, d = qd.shape
    z = (LOG2E / math.sqrt(d)) * (qd @ kd.T)
    z[np.triu(np.ones((T, T), dtype=bool), k=1)] = -np.inf
    return z


def _probabilities(z: np.ndarray):
    """Steps 5-6: integer row references and the FP8-grid probabilities."""
    m = np.ceil(z.max(axis=1, keepdims=True))        # finite: key i <= i
    x = np.exp2(z - m + P_SHIFT)                      # in (0, 256], 0 above the diagonal
    p_hat = e4m3_decode(e4m3_encode(x)) * 2.0 ** -P_SHIFT
    return m[:, 0], p_hat


def head_forward_fp8(q: np.ndarray, k: np.ndarray, v: np.ndarray, return_parts: bool = False):
    """Steps 1-7 for one head: q, k, v (T, d) float -> (O (T, d), LSE (T,)).

    With ``return_parts`` also returns a dict of the intermediate arrays
    (quantized operands, z, m, P^, l).
    """
    qz = quantize_head(q, k, v)
    z = _logits(qz["q"], qz["k"])
    m, p_hat = _probabilities(z)
    l = p_hat.sum(axis=1)
    o = (p_hat @ qz["v"]) / l[:, None]
    lse = math.log(2.0) * (m + np.log2(l))
    if return_parts:
        parts = dict(qz)
        parts.update({"z": z, "m": m, "p_hat": p_hat, "l": l})
        return o, lse, parts
    return o, lse


def quantize_positions(x: np.ndarray):
    """Blocks of 32 aligned positions per channel (zero past T): the blocking
    of an operand whose product contracts over positions. x (T, d) ->
    (codes (Tp, d), exps (Tp/32, d), dequantized (T, d)), Tp = round_up(T, 32)."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    Tp = -(-T // MX_BLOCK) * MX_BLOCK
    pad = np.zeros((Tp, d))
    pad[:T] = x
    c, e, deq = quantize_blocks(pad, axis=0)
    return c, e, deq[:T]


def _quantize_rows_along(x: np.ndarray, axis: int):
    """MX quantization of a T x T matrix in blocks of 32 along ``axis``,
    padded with zeros to a multiple of 32 there; returns the dequantized
    T x T values."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    Tp = -(-T // MX_BLOCK) * MX_BLOCK
    pad = np.zeros((Tp, Tp))
    pad[:T, :T] = x
    return quantize_blocks(pad, axis=axis)[2][:T, :T]


def head_backward_fp8(q, k, v, g, o, lse, return_parts: bool = False):
    """FP8 backward of one head: gradients of L = sum(G * O) with every
    product on MXFP8 operands, each blocked along its own contraction.

    q, k, v, g (= dL/dO), o (the forward's O) are (T, d); lse (T,) is the
    forward's natural-log LSE. Steps:
      B1. Q, K, V, G blocked along channels (for the products over d) and
          Q, K, G along positions (for the products over T).
      B2. z = log2(e) Q^ K^T / sqrt(d) (channel blocks, causal);
          P = 2^(z - lse log2 e), 0 above the diagonal.
      B3. P^ = E4M3(2^8 P) 2^-8 (the forward's fixed grid; P <= 1.75).
      B4. dV = P^T G^ (G blocked along positions).
      B5. dP = G^ V^T (channel blocks); D = rowsum(G * O) on the unquantized
          G and O; dS = P * (dP - D), with the unrounded P.
      B6. dS quantized along queries (blocks of 32 queries of one key):
          dK = dS_q^T Q^ / sqrt(d) (Q blocked along positions); along keys
          (blocks of 32 keys of one query): dQ = dS_k K^ / sqrt(d).
    Returns (dQ, dK, dV).
    """
    q, k, v, g, o = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, o))
    lse = np.asarray(lse, dtype=np.float64)
    T, d = q.shape
    qc = quantize_blocks(q, axis=1)[2]
    kc = quantize_blocks(k, axis=1)[2]
    vc = quantize_blocks(v, axis=1)[2]
    gc = quantize_blocks(g, axis=1)[2]
    qp = quantize_positions(q)[2]
    kp = quantize_positions(k)[2]
    gp = quantize_positions(g)[2]
    z = _logits(qc, kc)
    p = np.exp2(z - LOG2E * lse[:, None])
    if np.any(p > 1.75):
        raise ValueError("lse below the row's scores: P exceeds the E4M3 grid of step B3")
    p_hat = e4m3_decode(e4m3_encode(p * 2.0 ** P_SHIFT)) * 2.0 ** -P_SHIFT
    dv = p_hat.T @ gp
    dp = gc @ vc.T
    dd = (g * o).sum(axis=1)
    ds = p * (dp - dd[:, None])
    scale = 1.0 / math.sqrt(d)
    dk = scale * (_quantize_rows_along(ds, axis=0).T @ qp)
    dq = scale * (_quantize_rows_along(ds, axis=1) @ kp)
    if return_parts:
        return dq, dk, dv, {"p": p, "p_hat": p_hat, "dp": dp, "d": dd, "ds": ds}
    return dq, dk, dv


def backward_packed_fp8(dout, qkv, out, lse, n_head: int, head_dim: int,
                        heads: Optional[Sequence[Tuple[int, int]]] = None):
    """FP8 backward over packed arrays: dout, out (B, T, C), qkv (B, T, 3C),
    lse (B, H, T) -> dqkv (B, T, 3C), float64; heads not listed stay NaN."""
    qkv = np.asarray(qkv, dtype=np.float64)
    B, T, C3 = qkv.shape
    C = n_head * head_dim
    dqkv = np.full((B, T, 3 * C), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(n_head)]
    for b, h in pairs:
        q, k, v = _split(qkv, b, h, n_head, head_dim)
        lo = h * head_dim
        g = np.asarray(dout, dtype=np.float64)[b, :, lo:lo + head_dim]
        oo = np.asarray(out, dtype=np.float64)[b, :, lo:lo + head_dim]
        dq, dk, dv = head_backward_fp8(q, k, v, g, oo, np.asarray(lse, dtype=np.float64)[b, h])
        dqkv[b, :, lo:lo + head_dim] = dq
        dqkv[b, :, C + lo:C + lo + head_dim] = dk
        dqkv[b, :, 2 * C + lo:2 * C + lo + head_dim] = dv
    return dqkv


def _split(qkv: np.ndarray, b: int, h: int, n_head: int, head_dim: int):
    C = n_head * head_dim
    lo = h * head_dim
    return (qkv[b, :, lo:lo + head_dim], qkv[b, :, C + lo:C + lo + head_dim],
            qkv[b, :, 2 * C + lo:2 * C + lo + head_dim])


def forward_packed_fp8(qkv: np.ndarray, n_head: int, head_dim: int,
                       heads: Optional[Sequence[Tuple[int, int]]] = None):
    """FP8 forward over a packed (B, T, 3C) array ([Q | K | V], head h at
    columns h*d .. h*d + d - 1 of each block). Returns out (B, T, C) and lse
    (B, n_head, T), float64; heads not listed in ``heads`` stay NaN."""
    qkv = np.asarray(qkv, dtype=np.float64)
    B, T, C3 = qkv.shape
    C = n_head * head_dim
    if C3 != 3 * C:
        raise ValueError("last axis of qkv must be 3 * n_head * head_dim")
    out = np.full((B, T, C), np.nan)
    lse = np.full((B, n_head, T), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(n_head)]
    for b, h in pairs:
        q, k, v = _split(qkv, b, h, n_head, head_dim)
        o, l = head_forward_fp8(q, k, v)
        out[b, :, h * head_dim:(h + 1) * head_dim] = o
        lse[b, h, :] = l
    return out, lse


def _e4m3_neighbours(x: np.ndarray):
    """For x in (0, 448]: the E4M3 values just below and above the rounding
    decision of x (lo <= x <= hi, adjacent on the grid)."""
    code = e4m3_encode(x).astype(np.int64)
    val = e4m3_decode(code)
    below = val > x
    lo_code = np.where(below, code - 1, code)
    lo = e4m3_decode(np.maximum(lo_code, 0))
    hi = e4m3_decode(np.minimum(lo_code + 1, 0x7E))
    return lo, hi


def _dot_error_bound(q: np.ndarray, k: np.ndarray, dot_max_err: float) -> np.ndarray:
    """(T, T) bound on the error of the dot products Q^_i . K^_j as the FP8
    matrix unit forms them: dot_max_err times the largest magnitude among the
    d exact products |Q^_ic K^_jc| of each pair."""
    qa, ka = np.abs(q), np.abs(k)
    dot_max = np.empty((qa.shape[0], ka.shape[0]))
    for r0 in range(0, qa.shape[0], 64):
        dot_max[r0:r0 + 64] = (qa[r0:r0 + 64, None, :] * ka[None, :, :]).max(axis=2)
    return dot_max_err * dot_max


def rounding_slack(parts: dict, dot_max_err: float = 2.0 ** -11, x_rel_err: float = 2.0 ** -20):
    """Per-row bounds on what a streaming kernel may legitimately differ from
    head_forward_fp8 by, through the two cases named in the module docstring:
    (a) probabilities 2^(z - m) below 2^-13, whose codes depend on the
    reference in use (each may move by at most 2^-17 after the final
    rescale), and (b) codes whose argument x = 2^(z - m + 8) lies within the
    kernel's error of x from a rounding midpoint (each may move by one grid
    step). That error is taken as a dot-product error of at most
    ``dot_max_err`` * max_c |Q^_ic K^_jc| (the largest magnitude among the
    exact products: a matrix unit that aligns its products to the largest one
    before adding them loses bits in proportion to it, however small the
    others are), which moves z by that / sqrt(d) * log2(e) and x by ln 2
    times as much, relatively, plus ``x_rel_err`` for the scale, one fused
    multiply-add and exp2 in float32.

    The default dot_max_err = 2^-11 is empirical, not derived: it is the
    scaled FP8 matrix unit's worst observed error relative to its largest
    product (2^-11.2 over 2^21 random outputs of an in-bounds probe), rounded
    up to a power of two. A bound on an earlier model (2^-13 of the sum of
    the products' magnitudes) was broken by a wide-range row with one
    dominant weight, which is why the error is scaled by the largest product.

    Returns (o_slack (T,), lse_slack (T,)): |dO_i| <= o_slack_i per channel
    and |dLSE_i| <= lse_slack_i, to first order in the moved weights.
    """
    z, m, p_hat, l = parts["z"], parts["m"], parts["p_hat"], parts["l"]
    v = parts["v"]
    d = v.shape[1]
    o = (p_hat @ v) / l[:, None]
    x = np.exp2(z - m[:, None] + P_SHIFT)
    live = x > 0
    small = live & (x < 2.0 ** (P_SHIFT - 13))
    move = np.where(small, 2.0 ** -17, 0.0)
    xs = np.where(live, np.minimum(x, E4M3_MAX), 1.0)
    lo, hi = _e4m3_neighbours(xs)
    mid = 0.5 * (lo + hi)
    dot_err = _dot_error_bound(parts["q"], parts["k"], dot_max_err)
    rel = dot_err / math.sqrt(d) + x_rel_err   # ln 2 * log2(e) = 1
    if np.any(live & (rel > 2.0 ** -6)):
        # A logit error that large can move a code by several grid steps and
        # the row reference by more than one: the bound below would not hold.
        raise ValueError("rounding_slack needs logit errors below 2^-6 (relative to x)")
    near = live & ~small & (np.abs(xs - mid) <= rel * xs)
    move = move + np.where(near, (hi - lo) * 2.0 ** -P_SHIFT, 0.0)
    # |d(sum_j w_j v_j / sum_j w_j)| <= sum_j |dw_j| |v_j - O_i| / (l_i - sum_j |dw_j|)
    T = v.shape[0]
    spread = np.empty((T, T))
    for r0 in range(0, T, 64):
        spread[r0:r0 + 64] = np.abs(v[None, :, :] - o[r0:r0 + 64, None, :]).max(axis=2)
    tot = move.sum(axis=1)
    denom = np.maximum(l - tot, 1e-300)
    o_slack = (move * spread).sum(axis=1) / denom
    lse_slack = tot / denom
    return o_slack, lse_slack
