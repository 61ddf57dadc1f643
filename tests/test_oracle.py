"""Pins for the CPU float64 oracle (no GPU).

Each pin checks the oracle against something other than itself: a closed form,
a hand-derived worked example, brute force in pure-Python loops, central finite
differences, gradient identities, causality, key-shift invariance or torch's
CPU float64 scaled_dot_product_attention. ``test_planted_mistakes_are_caught``
then plants plausible mistakes in the oracle (a dropped scale, a shifted mask,
a transposed operand, a missing term) and shows that every one of them fails
at least one pin.
"""

import json
import math
import os
from contextlib import ExitStack
from unittest import mock

import numpy as np
import pytest

import oracle.attention as A

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng(20240901)


def _rand(*shape, std=1.0):
    return RNG.standard_normal(shape) * std


# ----------------------------------------------------------------------------
# Pins. Each takes the oracle module (possibly with a planted mistake) and
# raises AssertionError when the module disagrees with the pin.
# ----------------------------------------------------------------------------

def pin_t1_closed_form(M):
    """T = 1: the only visible key is the query's own, so O = V, LSE = s*q.k;
    backward: dV = G and dQ = dK = 0 (softmax of one logit is constant)."""
    for d in (1, 8, 64):
        q, k, v, g = (_rand(1, d) for _ in range(4))
        s = 1.0 / math.sqrt(d)
        o, lse = M.head_forward(q, k, v, s)
        np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse, [s * float(q[0] @ k[0])], rtol=1e-14, atol=1e-14)
        dq, dk, dv = M.head_backward(q, k, v, g, s)
        np.testing.assert_allclose(dv, g, rtol=0, atol=1e-15)
        np.testing.assert_allclose(dq, 0.0, atol=1e-15)
        np.testing.assert_allclose(dk, 0.0, atol=1e-15)


def pin_identical_keys_prefix_mean(M):
    """All keys equal: every visible logit in row i is the same, so P is
    uniform over keys 0..i, O[i] is the mean of V[0..i] and
    LSE[i] = s*q_i.k + ln(i + 1)."""
    T, d = 9, 16
    s = 1.0 / math.sqrt(d)
    q, v = _rand(T, d), _rand(T, d)
    k = np.tile(_rand(1, d), (T, 1))
    o, lse = M.head_forward(q, k, v, s)
    prefix_mean = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(o, prefix_mean, rtol=1e-13, atol=1e-13)
    expect_lse = s * (q @ k[0]) + np.log(np.arange(1, T + 1))
    np.testing.assert_allclose(lse, expect_lse, rtol=1e-13, atol=1e-13)


def pin_probability_rows(M):
    """Rows of P sum to 1, P is 0 above the diagonal and positive on and
    below it, and O = P V."""
    T, d = 12, 8
    q, k, v = _rand(T, d), _rand(T, d), _rand(T, d)
    o, _lse, p = M.head_forward(q, k, v, 1.0 / math.sqrt(d), return_probs=True)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(p[np.triu_indices(T, 1)] == 0.0)
    assert np.all(p[np.tril_indices(T)] > 0.0)
    np.testing.assert_allclose(o, p @ v, rtol=1e-13, atol=1e-13)


def pin_causality(M):
    """Changing tokens >= t leaves rows < t of O, LSE and dQ bitwise equal; with
    G also zero at rows >= t, rows < t of dK and dV are bitwise equal too."""
    T, d, t = 10, 8, 6
    s = 1.0 / math.sqrt(d)
    q, k, v, g = (_rand(T, d) for _ in range(4))
    g[t:] = 0.0
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[t:] += _rand(T - t, d)
    k2[t:] += _rand(T - t, d)
    v2[t:] += _rand(T - t, d)
    o1, l1 = M.head_forward(q, k, v, s)
    o2, l2 = M.head_forward(q2, k2, v2, s)
    assert np.array_equal(o1[:t], o2[:t]) and np.array_equal(l1[:t], l2[:t])
    assert not np.array_equal(o1[t:], o2[t:])
    b1 = M.head_backward(q, k, v, g, s)
    b2 = M.head_backward(q2, k2, v2, g, s)
    for x1, x2 in zip(b1, b2):
        assert np.array_equal(x1[:t], x2[:t])


def _loss(M, q, k, v, g, s):
    o, _ = M.head_forward(q, k, v, s)
    return float((g * o).sum())


def pin_finite_differences(M):
    """Central differences of L = sum(G * O) agree with the analytic gradients."""
    T, d, h = 5, 3, 1e-6
    s = 0.7  # a scale other than 1/sqrt(d) also exercises where it enters
    q, k, v, g = (_rand(T, d) for _ in range(4))
    dq, dk, dv = M.head_backward(q, k, v, g, s)
    for x, dx in ((q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(M, q, k, v, g, s)
            x[idx] = old - h
            lm = _loss(M, q, k, v, g, s)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(dx, fd, rtol=1e-6, atol=1e-8)


def pin_gradient_sums(M):
    """Rows of dS sum to 0, so sum_j dK_j = 0; rows of P sum to 1, so
    sum_j dV_j = sum_i G_i."""
    T, d = 11, 8
    q, k, v, g = (_rand(T, d) for _ in range(4))
    _dq, dk, dv = M.head_backward(q, k, v, g, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-13)
    np.testing.assert_allclose(dv.sum(axis=0), g.sum(axis=0), rtol=1e-13, atol=1e-13)


def pin_key_shift(M):
    """Adding one vector c to every key adds q_i.c to every logit of row i,
    which the row softmax cancels: O and dQ are unchanged."""
    T, d = 8, 8
    s = 1.0 / math.sqrt(d)
    q, k, v, g = (_rand(T, d) for _ in range(4))
    k2 = k + _rand(1, d) * 3.0
    o1, _ = M.head_forward(q, k, v, s)
    o2, _ = M.head_forward(q, k2, v, s)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    dq1 = M.head_backward(q, k, v, g, s)[0]
    dq2 = M.head_backward(q, k2, v, g, s)[0]
    np.testing.assert_allclose(dq1, dq2, rtol=1e-11, atol=1e-11)


def pin_worked_example(M):
    """The hand-derived T = 2 example in tests/golden/worked_example_t2.json."""
    with open(os.path.join(HERE, "golden", "worked_example_t2.json")) as f:
        ex = json.load(f)
    q, k, v, g = (np.array(ex[n], dtype=np.float64) for n in ("q", "k", "v", "g"))
    s = ex["scale"]
    e = ex["expected"]
    o, lse, p = M.head_forward(q, k, v, s, return_probs=True)
    np.testing.assert_allclose(o, e["o"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse, e["lse"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(p, e["p"], rtol=1e-14, atol=1e-14)
    dq, dk, dv = M.head_backward(q, k, v, g, s)
    np.testing.assert_allclose(dq, e["dq"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(dk, e["dk"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(dv, e["dv"], rtol=1e-14, atol=1e-14)


def _brute_force(q, k, v, g, s):
    """Pure-Python loops over the definition, with math.exp/math.log."""
    T, d = len(q), len(q[0])
    o = [[0.0] * d for _ in range(T)]
    lse = [0.0] * T
    P = [[0.0] * T for _ in range(T)]
    for i in range(T):
        logits = [s * sum(q[i][c] * k[j][c] for c in range(d)) for j in range(i + 1)]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        tot = sum(w)
        lse[i] = mx + math.log(tot)
        for j in range(i + 1):
            P[i][j] = w[j] / tot
            for c in range(d):
                o[i][c] += P[i][j] * v[j][c]
    dq = [[0.0] * d for _ in range(T)]
    dk = [[0.0] * d for _ in range(T)]
    dv = [[0.0] * d for _ in range(T)]
    for i in range(T):
        Di = sum(g[i][c] * o[i][c] for c in range(d))
        for j in range(i + 1):
            dpij = sum(g[i][c] * v[j][c] for c in range(d))
            dsij = P[i][j] * (dpij - Di)
            for c in range(d):
                dv[j][c] += P[i][j] * g[i][c]
                dq[i][c] += s * dsij * k[j][c]
                dk[j][c] += s * dsij * q[i][c]
    return o, lse, dq, dk, dv


def pin_brute_force(M):
    """Pure-Python loops over the definition agree with the oracle."""
    T, d = 6, 3
    s = 1.0 / math.sqrt(d)
    q, k, v, g = (_rand(T, d) for _ in range(4))
    bo, blse, bdq, bdk, bdv = _brute_force(q.tolist(), k.tolist(), v.tolist(), g.tolist(), s)
    o, lse = M.head_forward(q, k, v, s)
    dq, dk, dv = M.head_backward(q, k, v, g, s)
    for got, want in ((o, bo), (lse, blse), (dq, bdq), (dk, bdk), (dv, bdv)):
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def pin_torch_sdpa(M):
    """torch's CPU float64 scaled_dot_product_attention (is_causal=True) and
    its autograd gradients agree with the oracle."""
    torch = pytest.importorskip("torch")
    T, d = 17, 64
    q, k, v, g = (_rand(T, d) for _ in range(4))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None], is_causal=True)[0, 0]
    to.backward(torch.tensor(g, dtype=torch.float64))
    o, _ = M.head_forward(q, k, v)
    dq, dk, dv = M.head_backward(q, k, v, g)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-12)


def pin_packed_layout(M):
    """Packed (B, T, 3C) qkv is [Q | K | V] with head h at columns h*d..h*d+d-1
    of each block; out, lse and dqkv follow. Checked through a reshape to
    (B, T, 3, H, d), an indexing independent of the oracle's slicing, and at
    T = 1 through the closed form."""
    B, T, H, d = 2, 7, 3, 4
    C = H * d
    qkv = _rand(B, T, 3 * C)
    dout = _rand(B, T, C)
    out, lse = M.forward_packed(qkv, H, d)
    dqkv = M.backward_packed(dout, qkv, H, d)
    r = qkv.reshape(B, T, 3, H, d)
    rg = dout.reshape(B, T, H, d)
    ro = out.reshape(B, T, H, d)
    rd = dqkv.reshape(B, T, 3, H, d)
    for b in range(B):
        for h in range(H):
            o, l = M.head_forward(r[b, :, 0, h], r[b, :, 1, h], r[b, :, 2, h])
            np.testing.assert_allclose(ro[b, :, h], o, rtol=1e-14, atol=1e-14)
            np.testing.assert_allclose(lse[b, h], l, rtol=1e-14, atol=1e-14)
            grads = M.head_backward(r[b, :, 0, h], r[b, :, 1, h], r[b, :, 2, h], rg[b, :, h])
            for which in range(3):
                np.testing.assert_allclose(rd[b, :, which, h], grads[which], rtol=1e-14, atol=1e-14)
    # T = 1: out is the V block, the dV block is dout, the dQ and dK blocks are 0
    qkv1 = _rand(B, 1, 3 * C)
    dout1 = _rand(B, 1, C)
    out1, lse1 = M.forward_packed(qkv1, H, d)
    np.testing.assert_allclose(out1, qkv1[:, :, 2 * C:], atol=1e-15)
    r1 = qkv1.reshape(B, 1, 3, H, d)
    np.testing.assert_allclose(
        lse1[:, :, 0], (r1[:, 0, 0] * r1[:, 0, 1]).sum(-1) / math.sqrt(d), rtol=1e-14, atol=1e-14)
    d1 = M.backward_packed(dout1, qkv1, H, d)
    np.testing.assert_allclose(d1[:, :, 2 * C:], dout1, atol=1e-15)
    np.testing.assert_allclose(d1[:, :, :2 * C], 0.0, atol=1e-15)


def pin_sampled_heads(M):
    """Computing a subset of heads gives the same values as computing all."""
    B, T, H, d = 2, 5, 2, 4
    qkv = _rand(B, T, 3 * H * d)
    dout = _rand(B, T, H * d)
    out, lse = M.forward_packed(qkv, H, d)
    outs, lses = M.forward_packed(qkv, H, d, heads=[(1, 0)])
    np.testing.assert_array_equal(outs[1, :, 0:d], out[1, :, 0:d])
    np.testing.assert_array_equal(lses[1, 0], lse[1, 0])
    assert np.isnan(outs[0]).all()
    dq = M.backward_packed(dout, qkv, H, d)
    dqs = M.backward_packed(dout, qkv, H, d, heads=[(1, 0)])
    r, rs = dq.reshape(B, T, 3, H, d), dqs.reshape(B, T, 3, H, d)
    np.testing.assert_array_equal(rs[1, :, :, 0], r[1, :, :, 0])


PINS = [
    pin_t1_closed_form,
    pin_identical_keys_prefix_mean,
    pin_probability_rows,
    pin_causality,
    pin_finite_differences,
    pin_gradient_sums,
    pin_key_shift,
    pin_worked_example,
    pin_brute_force,
    pin_torch_sdpa,
    pin_packed_layout,
    pin_sampled_heads,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(A)


# ----------------------------------------------------------------------------
# Planted mistakes. Each mutant replaces one oracle function by a copy with a
# single plausible error; at least one pin must fail for every mutant.
# ----------------------------------------------------------------------------

_orig_scores = A._causal_scores
_orig_forward = A.head_forward
_orig_backward = A.head_backward
_orig_split = A.split_packed_head


def _scores_no_scale(q, k, scale):
    return _orig_scores(q, k, 1.0)


def _scores_scale_1_over_d(q, k, scale):
    return _orig_scores(q, k, scale * scale)


def _scores_strict_mask(q, k, scale):
    s = _orig_scores(q, k, scale)
    T = q.shape[0]
    if T > 1:
        s[np.diag_indices(T)] = -np.inf
        s[0, 0] = scale * float(q[0] @ k[0])  # keep row 0 finite
    return s


def _scores_anticausal(q, k, scale):
    T = q.shape[0]
    s = scale * (q @ k.T)
    s[np.tril(np.ones((T, T), dtype=bool), k=-1)] = -np.inf
    return s


def _scores_no_mask(q, k, scale):
    return scale * (q @ k.T)


def _scores_k_transposed_roles(q, k, scale):
    return _orig_scores(k, q, scale)


def _forward_variant(kind):
    def f(q, k, v, scale=None, return_probs=False):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        if scale is None:
            scale = A.default_scale(q.shape[1])
        s = A._causal_scores(q, k, scale)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        if kind == "column_norm":
            l = e.sum(axis=0, keepdims=True)
            p = e / l
            lse = m[:, 0] + np.log(e.sum(axis=1))
        else:
            l = e.sum(axis=1, keepdims=True)
            p = e / l
            lse = m[:, 0] + np.log(l[:, 0])
        if kind == "lse_no_max":
            lse = np.log(l[:, 0])
        if kind == "lse_base2":
            lse = (m[:, 0] + np.log(l[:, 0])) / math.log(2.0)
        o = p.T @ v if kind == "pt_v" else p @ v
        if kind == "swap_kv":
            s2 = A._causal_scores(q, v, scale)
            m2 = s2.max(axis=1, keepdims=True)
            e2 = np.exp(s2 - m2)
            p = e2 / e2.sum(axis=1, keepdims=True)
            o = p @ k
            lse = m2[:, 0] + np.log(e2.sum(axis=1))
        if return_probs:
            return o, lse, p
        return o, lse
    return f


def _backward_variant(kind):
    def f(q, k, v, g, scale=None):
        q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g))
        if scale is None:
            scale = A.default_scale(q.shape[1])
        o, _lse, p = A.head_forward(q, k, v, scale, return_probs=True)
        dv = p @ g if kind == "dv_no_transpose" else p.T @ g
        dp = g @ v.T
        d_row = (g * o).sum(axis=1)
        if kind == "d_from_dp":
            d_row = dp.sum(axis=1)
        ds = p * (dp - d_row[:, None])
        if kind == "ds_no_d":
            ds = p * dp
        dq = scale * (ds @ k)
        dk = scale * (ds.T @ q)
        if kind == "dk_no_transpose":
            dk = scale * (ds @ q)
        if kind == "dq_transposed":
            dq = scale * (ds.T @ k)
        if kind == "dq_no_scale":
            dq = ds @ k
        if kind == "dk_no_scale":
            dk = ds.T @ q
        if kind == "dq_uses_v":
            dq = scale * (ds @ v)
        return dq, dk, dv
    return f


def _split_swap_kv(qkv, b, h, n_head, head_dim):
    q, k, v = _orig_split(qkv, b, h, n_head, head_dim)
    return q, v, k


def _split_head_stride_3d(qkv, b, h, n_head, head_dim):
    # interleaved-per-head reading of the packing: [q_h | k_h | v_h] per head
    lo = 3 * h * head_dim
    return (qkv[b, :, lo:lo + head_dim], qkv[b, :, lo + head_dim:lo + 2 * head_dim],
            qkv[b, :, lo + 2 * head_dim:lo + 3 * head_dim])


MUTANTS = {
    "scores_no_scale": {"_causal_scores": _scores_no_scale},
    "scores_scale_1_over_d": {"_causal_scores": _scores_scale_1_over_d},
    "mask_hides_diagonal": {"_causal_scores": _scores_strict_mask},
    "mask_anticausal": {"_causal_scores": _scores_anticausal},
    "mask_missing": {"_causal_scores": _scores_no_mask},
    "scores_q_k_swapped": {"_causal_scores": _scores_k_transposed_roles},
    "softmax_column_normalised": {"head_forward": _forward_variant("column_norm")},
    "lse_without_max": {"head_forward": _forward_variant("lse_no_max")},
    "lse_base2": {"head_forward": _forward_variant("lse_base2")},
    "o_uses_p_transposed": {"head_forward": _forward_variant("pt_v")},
    "k_and_v_swapped": {"head_forward": _forward_variant("swap_kv")},
    "dv_no_transpose": {"head_backward": _backward_variant("dv_no_transpose")},
    "d_from_dp": {"head_backward": _backward_variant("d_from_dp")},
    "ds_without_d": {"head_backward": _backward_variant("ds_no_d")},
    "dk_no_transpose": {"head_backward": _backward_variant("dk_no_transpose")},
    "dq_transposed": {"head_backward": _backward_variant("dq_transposed")},
    "dq_no_scale": {"head_backward": _backward_variant("dq_no_scale")},
    "dk_no_scale": {"head_backward": _backward_variant("dk_no_scale")},
    "dq_uses_v": {"head_backward": _backward_variant("dq_uses_v")},
    "packing_k_v_swapped": {"split_packed_head": _split_swap_kv},
    "packing_interleaved_per_head": {"split_packed_head": _split_head_stride_3d},
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name):
    failed = []
    with ExitStack() as stack:
        for attr, repl in MUTANTS[name].items():
            stack.enter_context(mock.patch.object(A, attr, repl))
        for pin in PINS:
            try:
                with np.errstate(all="ignore"):
                    pin(A)
            except (AssertionError, ValueError, FloatingPointError, IndexError):
                failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
