"""CPU float64 oracle for causal multi-head self-attention, forward and backward.

TEST INFRASTRUCTURE. This module exists to check the HIP library. Only the test
suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or call it; the product path (the C-ABI library and its Python
binding) never does, and it imports nothing from the product.

What it computes
----------------
The pages describe flash attention as attention that gives the same result as
the ordinary computation while never keeping the full T x T attention matrix in
GPU memory (theprofessional.online summary of "Let's reproduce GPT-2 (124M)",
glossary table, row "flash attention"; "Andrej Karpathy - Lets reproduce GPT 2
124M", chapter list, 02:00:18 "flash attention"). Since the fused method reaches
the plain result up to rounding order, this oracle is the plain definition
written out, materialising the T x T matrix on purpose:

    S = scale * Q K^T, with S[i, j] = -inf where j > i   (causal, next-token
        model: "Let's reproduce GPT-2 (124M)" chapter list, 00:13:47 and
        00:31:00; the loss row of the glossary table; scaled dot-product
        attention of "Attention is All You Need", linked from the same page)
    P = softmax(S) row by row
    O = P V
    LSE[i] = log sum_j exp(S[i, j])            (natural log, scaled logits)

and its analytic gradients for an upstream gradient G = dL/dO:

    dV = P^T G
    dP = G V^T
    D[i] = sum_k G[i, k] O[i, k]
    dS = P * (dP - D[:, None])
    dQ = scale * dS K
    dK = scale * dS^T Q

The pages give no formula, so these readings are adopted where they are
silent: the diagonal is visible (query i sees keys j <= i); the scale is
1/sqrt(head_dim) applied before the softmax; qkv is packed as (B, T, 3C) with
[Q | K | V] along the last axis and head h at columns h*d .. h*d+d-1 of each
block; out is (B, T, C) with the same head placement; lse is (B, H, T); dqkv
mirrors qkv. Every step is one library primitive (a matmul, an exp, a sum) in
float64 with no blocking, fusion or reordering.

Pins: tests/test_oracle.py checks this module against closed forms (T = 1,
identical keys), a hand-derived worked example (tests/golden/), brute force in
pure-Python loops, central finite differences, gradient-sum identities,
causality, key-shift invariance and torch's CPU float64
scaled_dot_product_attention with autograd, and shows that planted mistakes
fail at least one of them.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "default_scale",
    "head_forward",
    "head_backward",
    "forward_packed",
    "backward_packed",
    "split_packed_head",
]


def default_scale(head_dim: int) -> float:
    """1/sqrt(head_dim): the scaled dot-product temperature."""
    return 1.0 / math.sqrt(head_dim)


def _causal_scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T with every entry above the diagonal set to -inf."""
    T = q.shape[0]
    s = scale * (q @ k.T)
    above = np.triu(np.ones((T, T), dtype=bool), k=1)  # key index j > query i
    s[above] = -np.inf
    return s


def head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                 scale: Optional[float] = None,
                 return_probs: bool = False):
    """Causal attention of one head.

    q, k, v: (T, d) float64. Returns (O (T, d), LSE (T,)) and, if asked, P.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = default_scale(q.shape[1])
    s = _causal_scores(q, k, scale)
    m = s.max(axis=1, keepdims=True)       # finite: j = i is always visible
    e = np.exp(s - m)                       # exactly 0 above the diagonal
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    o = p @ v
    lse = m[:, 0] + np.log(l[:, 0])
    if return_probs:
        return o, lse, p
    return o, lse


def head_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray,
                  scale: Optional[float] = None):
    """Gradients of L = sum(G * O) for one head.

    q, k, v, g: (T, d) float64, g = dL/dO. Returns (dQ, dK, dV), each (T, d).
    D is taken from this oracle's own float64 O.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    if scale is None:
        scale = default_scale(q.shape[1])
    o, _lse, p = head_forward(q, k, v, scale, return_probs=True)
    dv = p.T @ g
    dp = g @ v.T
    d_row = (g * o).sum(axis=1)
    ds = p * (dp - d_row[:, None])          # zero where P is zero (j > i)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def split_packed_head(qkv: np.ndarray, b: int, h: int, n_head: int,
                      head_dim: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Views of Q, K, V of head h in batch row b of a packed (B, T, 3C) array."""
    C = n_head * head_dim
    lo = h * head_dim
    q = qkv[b, :, lo:lo + head_dim]
    k = qkv[b, :, C + lo:C + lo + head_dim]
    v = qkv[b, :, 2 * C + lo:2 * C + lo + head_dim]
    return q, k, v


def _heads(B: int, n_head: int, heads: Optional[Iterable[Tuple[int, int]]]):
    if heads is None:
        return [(b, h) for b in range(B) for h in range(n_head)]
    return list(heads)


def forward_packed(qkv: np.ndarray, n_head: int, head_dim: int,
                   scale: Optional[float] = None,
                   heads: Optional[Sequence[Tuple[int, int]]] = None):
    """Forward over a packed (B, T, 3C) array.

    Returns out (B, T, C) and lse (B, n_head, T), float64. If ``heads`` lists
    (b, h) pairs, only those heads are computed; the rest stay NaN.
    """
    qkv = np.asarray(qkv, dtype=np.float64)
    B, T, C3 = qkv.shape
    C = n_head * head_dim
    if C3 != 3 * C:
        raise ValueError("last axis of qkv must be 3 * n_head * head_dim")
    out = np.full((B, T, C), np.nan)
    lse = np.full((B, n_head, T), np.nan)
    for b, h in _heads(B, n_head, heads):
        q, k, v = split_packed_head(qkv, b, h, n_head, head_dim)
        o, l = head_forward(q, k, v, scale)
        out[b, :, h * head_dim:(h + 1) * head_dim] = o
        lse[b, h, :] = l
    return out, lse


def backward_packed(dout: np.ndarray, qkv: np.ndarray, n_head: int,
                    head_dim: int, scale: Optional[float] = None,
                    heads: Optional[Sequence[Tuple[int, int]]] = None):
    """Backward over packed arrays: dout (B, T, C) -> dqkv (B, T, 3C), float64.

    If ``heads`` lists (b, h) pairs, only those heads are computed; the rest
    stay NaN.
    """
    qkv = np.asarray(qkv, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, T, C3 = qkv.shape
    C = n_head * head_dim
    if C3 != 3 * C or dout.shape != (B, T, C):
        raise ValueError("dout must be (B, T, C) and qkv (B, T, 3C)")
    dqkv = np.full((B, T, 3 * C), np.nan)
    for b, h in _heads(B, n_head, heads):
        q, k, v = split_packed_head(qkv, b, h, n_head, head_dim)
        lo = h * head_dim
        g = dout[b, :, lo:lo + head_dim]
        dq, dk, dv = head_backward(q, k, v, g, scale)
        dqkv[b, :, lo:lo + head_dim] = dq
        dqkv[b, :, C + lo:C + lo + head_dim] = dk
        dqkv[b, :, 2 * C + lo:2 * C + lo + head_dim] = dv
    return dqkv
