"""Where the workloads' bars stop holding for any implementation (no GPU):
the flat bf16 bar on O against output magnitude, and the fp32 bar against
logit size.

A bf16 value of magnitude in [4, 8) is a multiple of 2^-5, so even the
correctly rounded exact output can lie 2^-6 = 0.0156 from it. The
workloads' outputs stay small enough for the flat bar. A larger shape from
the same generator does not: at B=2, T=1613, 5 heads, seed 10254, query 1 of
head (0, 0) has an output of magnitude 4.05 whose correctly rounded bf16
value misses the exact one by more than 1e-2. No bf16 output can meet the
flat bar there, so the GPU test of that shape holds O to the
magnitude-relative bar 2^-7 max|O| (tests/helpers.bf16_o_bound)."""

import numpy as np

from causal_flash_attention_amd import inputs as I
from oracle import attention as A

D = 64
CASE = (2, 1613, 5, 10254)  # B, T, n_head, seed


def _exact_out_first_rows(n_rows: int):
    B, T, H, seed = CASE
    qkv, _ = I.attention_inputs(B, T, H, D, "bf16", 1.0, 0.01, seed=seed)
    q64 = I.to_float64(qkv, "bf16")[:, :n_rows]  # causal: rows < n_rows see only themselves
    out, _ = A.forward_packed(q64, H, D, heads=[(0, 0)])
    return out[0, :, :D]


def test_correctly_rounded_bf16_output_misses_the_flat_bar():
    o = _exact_out_first_rows(4)
    rounded = I.bf16_bits_to_f32(I.f32_to_bf16_bits(o.astype(np.float32))).astype(np.float64)
    err = np.abs(rounded - o)
    t, d = np.unravel_index(err.argmax(), err.shape)
    assert (t, d) == (1, 27)
    assert 4.0 <= abs(o[t, d]) < 8.0
    assert err[t, d] > 1e-2           # the flat bar is out of reach here ...
    assert err[t, d] <= 2.0 ** -6     # ... by at most half a bf16 step at this magnitude
    assert err[t, d] <= 2.0 ** -7 * np.abs(o).max()  # and within the relative bar


def test_plain_fp32_misses_the_fp32_bar_at_large_logits():
    """The fp32 bar 1e-5 * max|ref| is the tiny workload's; it does not hold
    for logits far beyond the workloads'. With Q and K scaled by 4 (B=1,
    T=600, 3 heads, seed 80011; logits up to about 87), a straightforward
    float32 backward misses it on dQ, since the logits' own float32 rounding
    grows with their size. No committed fp32 GPU test uses such inputs."""
    import oracle
    from test_parity_gpu import _scale_qk
    B, T, H = 1, 600, 3
    qkv, dout = I.attention_inputs(B, T, H, D, "f32", 1.0, 1.0, seed=80011)
    qkv = _scale_qk(qkv, "f32", H, 4.0)
    q64, g64 = I.to_float64(qkv, "f32"), I.to_float64(dout, "f32")
    ref = oracle.backward_packed(g64, q64, H, D)
    C = H * D
    f32 = np.float32
    worst, refmax = 0.0, float(np.abs(ref[0, :, :C]).max())
    mask = np.triu(np.ones((T, T), bool), 1)
    for h in range(H):
        q, k, v = (q64[0, :, o + h * D:o + (h + 1) * D].astype(f32) for o in (0, C, 2 * C))
        g = g64[0, :, h * D:(h + 1) * D].astype(f32)
        s = (q @ k.T) * f32(0.125)
        s[mask] = -np.inf
        p = np.exp(s - s.max(1, keepdims=True))
        p = (p / p.sum(1, keepdims=True)).astype(f32)
        o = p @ v
        ds = p * (g @ v.T - (g * o).sum(1, keepdims=True))
        dq = (ds @ k) * f32(0.125)
        worst = max(worst, float(np.abs(dq - ref[0, :, h * D:(h + 1) * D]).max()))
    assert worst > 1e-5 * refmax
