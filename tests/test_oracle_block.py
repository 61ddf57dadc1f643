"""Pins for the attention-block oracle (c_attn, attention, c_proj; no GPU).

Each pin checks oracle.block against something other than itself: torch's
CPU float64 autograd of the same layer (linear maps and
scaled_dot_product_attention), central finite differences, the reduction to
plain attention when both maps are identities, and the exact shift of y by
a change of b_proj. ``test_planted_mistakes_are_caught`` plants plausible
mistakes and shows that each fails at least one pin.
"""

from contextlib import ExitStack
from unittest import mock

import numpy as np
import pytest

import oracle.attention as A
import oracle.block as K

RNG = np.random.default_rng(20241204)
D = 64


def _params(C, std=0.05):
    return (RNG.standard_normal((C, 3 * C)) * std, RNG.standard_normal(3 * C) * std,
            RNG.standard_normal((C, C)) * std, RNG.standard_normal(C) * std)


def _all(M, x, dy, H, p):
    wa, ba, wp, bp = p
    f = M.block_forward(x, wa, ba, wp, bp, H, D)
    g = M.block_backward(dy, x, wa, wp, f, H, D)
    return f, g


def pin_torch_autograd(M):
    """The whole layer against torch CPU float64 autograd."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    for B, T, H in ((2, 7, 2), (1, 33, 1)):
        C = H * D
        x = RNG.standard_normal((B, T, C))
        dy = RNG.standard_normal((B, T, C))
        p = _params(C, std=0.1)
        f, g = _all(M, x, dy, H, p)
        xt = torch.tensor(x, requires_grad=True)
        wa, ba, wp, bp = (torch.tensor(a, requires_grad=True) for a in p)
        qkv = xt @ wa + ba
        q, k, v = (t.reshape(B, T, H, D).transpose(1, 2) for t in qkv.split(C, dim=2))
        att = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        att = att.transpose(1, 2).reshape(B, T, C)
        y = att @ wp + bp
        (y * torch.tensor(dy)).sum().backward()
        assert np.allclose(f["y"], y.detach().numpy(), rtol=1e-10, atol=1e-12)
        assert np.allclose(f["qkv"], qkv.detach().numpy(), rtol=1e-12, atol=1e-14)
        for name, t in (("dx", xt), ("dw_attn", wa), ("db_attn", ba), ("dw_proj", wp),
                        ("db_proj", bp)):
            assert np.allclose(g[name], t.grad.numpy(), rtol=1e-9, atol=1e-11), name


def pin_identity_maps(M):
    """W_attn = [I | I | I], W_proj = I, zero biases: the block is plain
    attention with Q = K = V = x, and dx = dQ + dK + dV of that attention."""
    B, T, H = 2, 9, 2
    C = H * D
    x = RNG.standard_normal((B, T, C))
    dy = RNG.standard_normal((B, T, C))
    eye = np.eye(C)
    p = (np.concatenate([eye, eye, eye], axis=1), np.zeros(3 * C), eye, np.zeros(C))
    f, g = _all(M, x, dy, H, p)
    packed = np.concatenate([x, x, x], axis=2)
    out, _ = A.forward_packed(packed, H, D)
    assert np.allclose(f["y"], out, rtol=1e-12, atol=1e-14)
    dq = A.backward_packed(dy, packed, H, D)
    assert np.allclose(g["dx"], dq[..., :C] + dq[..., C:2 * C] + dq[..., 2 * C:],
                       rtol=1e-10, atol=1e-12)


def pin_bias_shift(M):
    """Adding delta to b_proj adds delta to every row of y; adding it to the
    V third of b_attn adds delta W_proj to every row (softmax rows sum to 1)."""
    B, T, H = 1, 6, 2
    C = H * D
    x = RNG.standard_normal((B, T, C))
    wa, ba, wp, bp = _params(C)
    delta = RNG.standard_normal(C)
    y0 = M.block_forward(x, wa, ba, wp, bp, H, D)["y"]
    y1 = M.block_forward(x, wa, ba, wp, bp + delta, H, D)["y"]
    assert np.allclose(y1 - y0, np.broadcast_to(delta, y0.shape), rtol=1e-10, atol=1e-12)
    ba2 = ba.copy()
    ba2[2 * C:] += delta
    y2 = M.block_forward(x, wa, ba2, wp, bp, H, D)["y"]
    assert np.allclose(y2 - y0, np.broadcast_to(delta @ wp, y0.shape), rtol=1e-9, atol=1e-11)


def pin_finite_differences(M):
    """Central differences of L = sum(dy * y) on random coordinates of every
    input and parameter."""
    B, T, H = 1, 5, 2
    C = H * D
    x = RNG.standard_normal((B, T, C))
    dy = RNG.standard_normal((B, T, C))
    p = list(_params(C, std=0.2))
    f, g = _all(M, x, dy, H, p)

    def loss(xx, pp):
        return float((M.block_forward(xx, *pp, H, D)["y"] * dy).sum())

    h = 1e-6
    targets = [("dx", None), ("dw_attn", 0), ("db_attn", 1), ("dw_proj", 2), ("db_proj", 3)]
    for name, idx in targets:
        arr = x if idx is None else p[idx]
        for _ in range(4):
            pos = tuple(int(RNG.integers(0, s)) for s in arr.shape)
            old = arr[pos]
            arr[pos] = old + h
            lp = loss(x, p)
            arr[pos] = old - h
            lm = loss(x, p)
            arr[pos] = old
            fd = (lp - lm) / (2 * h)
            an = g[name][pos]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, pos, fd, an)


PINS = [pin_torch_autograd, pin_identity_maps, pin_bias_shift, pin_finite_differences]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_block_oracle_pin(pin):
    pin(K)


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------

_orig_fwd = K.block_forward
_orig_bwd = K.block_backward


def _fwd_variant(kind):
    def f(x, w_attn, b_attn, w_proj, b_proj, n_head, head_dim=64):
        x = np.asarray(x, dtype=np.float64)
        qkv = x @ w_attn + (0.0 if kind == "no_b_attn" else b_attn)
        att, lse = K._attention_forward(qkv, n_head, head_dim)
        wp = w_proj.T if kind == "w_proj_transposed" else w_proj
        y = att @ wp + (0.0 if kind == "no_b_proj" else b_proj)
        return {"qkv": qkv, "att": att, "lse": lse, "y": y}
    return f


def _bwd_variant(kind):
    def f(dy, x, w_attn, w_proj, fwd, n_head, head_dim=64):
        dy = np.asarray(dy, dtype=np.float64)
        B, T, C = x.shape
        att, qkv = fwd["att"], fwd["qkv"]
        datt = dy @ (w_proj if kind == "datt_no_transpose" else w_proj.T)
        if kind == "dw_proj_transposed":
            dw_proj = dy.reshape(B * T, C).T @ att.reshape(B * T, C)
        else:
            dw_proj = att.reshape(B * T, C).T @ dy.reshape(B * T, C)
        db_proj = dy.reshape(B * T, C).sum(axis=0)
        if kind == "db_proj_mean":
            db_proj = db_proj / (B * T)
        dqkv = K._attention_backward(dy if kind == "skip_c_proj" else datt, qkv, n_head, head_dim)
        dx = dqkv @ w_attn.T
        dw_attn = x.reshape(B * T, C).T @ dqkv.reshape(B * T, 3 * C)
        db_attn = dqkv.reshape(B * T, 3 * C).sum(axis=0)
        if kind == "db_attn_qk_only":
            db_attn[2 * C:] = 0.0
        return {"datt": datt, "dqkv": dqkv, "dx": dx, "dw_attn": dw_attn, "db_attn": db_attn,
                "dw_proj": dw_proj, "db_proj": db_proj}
    return f


MUTANTS = {
    "no_b_attn": {"block_forward": _fwd_variant("no_b_attn")},
    "no_b_proj": {"block_forward": _fwd_variant("no_b_proj")},
    "w_proj_transposed": {"block_forward": _fwd_variant("w_proj_transposed")},
    "datt_no_transpose": {"block_backward": _bwd_variant("datt_no_transpose")},
    "dw_proj_transposed": {"block_backward": _bwd_variant("dw_proj_transposed")},
    "db_proj_mean": {"block_backward": _bwd_variant("db_proj_mean")},
    "skip_c_proj_in_backward": {"block_backward": _bwd_variant("skip_c_proj")},
    "db_attn_qk_only": {"block_backward": _bwd_variant("db_attn_qk_only")},
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name):
    failed = []
    with ExitStack() as stack:
        for attr, repl in MUTANTS[name].items():
            stack.enter_context(mock.patch.object(K, attr, repl))
        for pin in PINS:
            try:
                with np.errstate(all="ignore"):
                    pin(K)
            except (AssertionError, ValueError, FloatingPointError, IndexError):
                failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
