"""CPU float64 oracle of the attention block: c_attn, causal attention, c_proj.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import or call this module; the product
path never does, and it imports nothing from the product.

What it computes
----------------
The attention layer of GPT-2 as the pages build it ("Let's reproduce GPT-2
(124M)", chapter list, 00:13:47 implementing GPT-2 as an nn.Module; the
kernel-fusion and flash-attention chapters 01:48:15 and 02:00:18 speed up
exactly this layer): one linear map (c_attn) turns each token's C channels
into the packed [Q | K | V] row, causal attention mixes the tokens per head,
and a second linear map (c_proj) mixes the heads back into C channels:

    qkv = x W_attn + b_attn          x (N, C), W_attn (C, 3C), b_attn (3C,)
    att, lse = attention(qkv)        oracle.attention, packed layout
    y = att W_proj + b_proj          W_proj (C, C), b_proj (C,)

with N = B * T token rows and the weights stored (in, out), the GPT-2
checkpoint's Conv1D orientation. For an upstream gradient dy:

    datt = dy W_proj^T;  dW_proj = att^T dy;  db_proj = sum over rows of dy
    dqkv = attention backward(datt)
    dx = dqkv W_attn^T;  dW_attn = x^T dqkv;  db_attn = sum over rows of dqkv

Every step is a library matmul or sum in float64, with no rounding between
them (the GPU path stores qkv, att, datt and dqkv in bf16; the tests derive
their bound from that).

Pins: tests/test_oracle_block.py checks this module against torch's CPU
float64 autograd of the same layer, central finite differences, the
reduction to plain attention when both maps are identities, the bias
gradient identities, and shows that planted mistakes fail at least one pin.
"""

from __future__ import annotations

import numpy as np

from . import attention as A

__all__ = ["block_forward", "block_backward"]


def _attention_forward(qkv: np.ndarray, n_head: int, head_dim: int):
    return A.forward_packed(qkv, n_head, head_dim)


def _attention_backward(datt, qkv, n_head, head_dim):
    return A.backward_packed(datt, qkv, n_head, head_dim)


def block_forward(x, w_attn, b_attn, w_proj, b_proj, n_head: int, head_dim: int = 64):
    """x (B, T, C) -> dict with qkv (B, T, 3C), att (B, T, C), lse (B, H, T),
    y (B, T, C), all float64."""
    x = np.asarray(x, dtype=np.float64)
    B, T, C = x.shape
    if C != n_head * head_dim:
        raise ValueError("x's last axis must be n_head * head_dim")
    qkv = x @ np.asarray(w_attn, dtype=np.float64) + np.asarray(b_attn, dtype=np.float64)
    att, lse = _attention_forward(qkv, n_head, head_dim)
    y = att @ np.asarray(w_proj, dtype=np.float64) + np.asarray(b_proj, dtype=np.float64)
    return {"qkv": qkv, "att": att, "lse": lse, "y": y}


def block_backward(dy, x, w_attn, w_proj, fwd: dict, n_head: int, head_dim: int = 64):
    """Gradients of L = sum(dy * y) for the forward `fwd` of block_forward.

    Returns a dict with datt, dqkv (as the layer passes them on), dx, dw_attn,
    db_attn, dw_proj, db_proj, float64.
    """
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    w_attn = np.asarray(w_attn, dtype=np.float64)
    w_proj = np.asarray(w_proj, dtype=np.float64)
    B, T, C = x.shape
    att, qkv = fwd["att"], fwd["qkv"]
    datt = dy @ w_proj.T
    dw_proj = att.reshape(B * T, C).T @ dy.reshape(B * T, C)
    db_proj = dy.reshape(B * T, C).sum(axis=0)
    dqkv = _attention_backward(datt, qkv, n_head, head_dim)
    dx = dqkv @ w_attn.T
    dw_attn = x.reshape(B * T, C).T @ dqkv.reshape(B * T, 3 * C)
    db_attn = dqkv.reshape(B * T, 3 * C).sum(axis=0)
    return {"datt": datt, "dqkv": dqkv, "dx": dx, "dw_attn": dw_attn, "db_attn": db_attn,
            "dw_proj": dw_proj, "db_proj": db_proj}
