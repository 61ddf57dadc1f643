"""The materialising attention path (attn_fwd_unfused / attn_bwd_unfused)
against the CPU float64 oracle, and its probability matrix (needs a GPU).

Same seeded inputs and comparison as the fused path's parity tests. The
gradient and LSE bars are the same. The O bar is the one derived from this
method's arithmetic: it rounds the normalised probabilities to bf16 before
P V (as a framework's bf16 matrix product does), which adds up to 2^-9 |O|
to the 2^-9 |O| of O's own rounding, so O is held to max(1e-2, 2^-7 max|O|).
"""

import numpy as np
import pytest

import oracle
from causal_flash_attention_amd import binding
from causal_flash_attention_amd import inputs as I

from helpers import (assert_parity, bf16_o_bound, compare, log, run_library, sample_heads,
                     to_device, to_host64)

pytestmark = pytest.mark.gpu

D = 64


def run_unfused(qd, gd, H):
    import torch
    B, T = int(qd.shape[0]), int(qd.shape[1])
    C = H * D
    out = torch.empty((B, T, C), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    probs = torch.empty((B, H, T, binding.unfused_row_stride(T)), dtype=torch.bfloat16,
                        device="cuda")
    # Every workspace byte 0xff (a NaN in every float): a kernel that reads a
    # workspace element its producer never wrote (the padding columns of S and
    # dP when T % 8 != 0) turns the whole row into NaN instead of passing by luck.
    ws = torch.full((binding.unfused_workspace_bytes(B, T, H),), 255, dtype=torch.uint8,
                    device="cuda")
    dqkv = torch.full_like(qd, float("nan"))
    binding.attn_fwd_unfused(qd, out, lse, probs, ws, H)
    binding.attn_bwd_unfused(gd, qd, probs, dqkv, ws, H)
    torch.cuda.synchronize()
    return out, lse, probs, dqkv


def _check(B, T, H, seed, heads=None, label="unfused"):
    log(f"[case] {label} B={B} T={T} H={H} seed={seed}")
    qkv, dout = I.attention_inputs(B, T, H, D, "bf16", 1.0, 0.01, seed=seed)
    q64, g64 = I.to_float64(qkv, "bf16"), I.to_float64(dout, "bf16")
    qd, gd = to_device(qkv, "bf16"), to_device(dout, "bf16")
    out, lse, probs, dqkv = run_unfused(qd, gd, H)
    gpu = {"out": to_host64(out), "lse": to_host64(lse), "dqkv": to_host64(dqkv)}
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    ref_out, ref_lse = oracle.forward_packed(q64, H, D, heads=heads)
    ref_dqkv = oracle.backward_packed(g64, q64, H, D, heads=heads)
    m = compare(gpu, {"out": ref_out, "lse": ref_lse, "dqkv": ref_dqkv}, heads, H, D)
    for k in ("out", "lse", "dqkv"):
        assert np.all(np.isfinite(gpu[k])), (label, k)
    assert_parity(m, "bf16", f"{label} B={B} T={T} H={H}", bf16_o_bound(m["o_refmax"]))
    return qd, gd, probs, gpu


@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (1, 2, 1), (1, 64, 2), (1, 65, 1), (2, 200, 3),
                                   (2, 485, 3),
                                   (3, 129, 2), (1, 1000, 2), (2, 257, 25), (1, 2047, 1),
                                   (1, 4096, 1)])
def test_unfused_parity(B, T, H):
    _, _, probs, _ = _check(B, T, H, seed=100 + T)
    # P: exactly zero above the diagonal and in the padding columns; each row
    # sums to 1 up to the bf16 rounding of its entries (relative 2^-9 each).
    p = to_host64(probs)
    assert np.all(p[..., T:] == 0.0)
    p = p[..., :T]
    iu = np.triu_indices(T, 1)
    assert np.all(p[:, :, iu[0], iu[1]] == 0.0)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=3e-3)


def test_unfused_headline_shape_and_fused_agreement():
    """GPT-2 124M layer shape on sampled heads, and the fused path on the same
    inputs: both meet the oracle's bars, so they agree to within twice them."""
    B, T, H = 16, 1024, 12
    qd, gd, _, gpu = _check(B, T, H, seed=0, heads=sample_heads(B, H, 8, seed=3),
                            label="unfused headline")
    out, lse, dqkv = run_library(qd, gd, H)
    fused = {"out": to_host64(out), "lse": to_host64(lse), "dqkv": to_host64(dqkv)}
    assert np.max(np.abs(fused["out"] - gpu["out"])) <= 2e-2
    assert np.max(np.abs(fused["lse"] - gpu["lse"])) <= 2e-3
    rel = np.linalg.norm(fused["dqkv"] - gpu["dqkv"]) / np.linalg.norm(gpu["dqkv"])
    assert rel <= 4e-2, rel
