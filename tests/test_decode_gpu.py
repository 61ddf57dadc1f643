"""Decode attention (attn_decode) against the CPU float64 oracle (needs a GPU).

The decode of position T-1 is the last row of causal attention over the first
T positions, so the oracle's full forward on the same seeded qkv gives the
expected O and LSE. Two cache layouts: the packed qkv itself (strided views),
and separate (B, T_max, C) caches whose rows past T hold NaN (any read of
them would show in the result).
"""

import numpy as np
import pytest

import oracle
from causal_flash_attention_amd import binding
from causal_flash_attention_amd import inputs as I

from helpers import BF16_LSE_MAXABS, BF16_O_MAXABS, log, to_device, to_host64

pytestmark = pytest.mark.gpu

D = 64


def _run(q, k, v, T, H):
    import torch
    B, C = int(q.shape[0]), H * D
    out = torch.full((B, C), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((max(1, binding.decode_workspace_floats(B, T, H)),), float("nan"),
                    device="cuda")
    binding.attn_decode(q, k, v, out, lse, ws, T, H)
    torch.cuda.synchronize()
    return to_host64(out), to_host64(lse)


@pytest.mark.parametrize("layout", ["packed", "separate"])
@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (2, 63, 2), (1, 64, 1), (3, 65, 2), (2, 1000, 3),
                                   (1, 4096, 2), (2, 257, 25)])
def test_decode_parity(B, T, H, layout):
    import torch
    log(f"[case] decode {layout} B={B} T={T} H={H}")
    C = H * D
    qkv, _ = I.attention_inputs(B, T, H, D, "bf16", 1.0, 0.01, seed=500 + T)
    ref_out, ref_lse = oracle.forward_packed(I.to_float64(qkv, "bf16"), H, D)
    qd = to_device(qkv, "bf16")
    q = qd[:, T - 1, :C]
    if layout == "packed":
        k, v = qd[:, :, C:2 * C], qd[:, :, 2 * C:]
    else:
        T_max = T + 37
        k = torch.full((B, T_max, C), float("nan"), dtype=torch.bfloat16, device="cuda")
        v = torch.full_like(k, float("nan"))
        k[:, :T] = qd[:, :, C:2 * C]
        v[:, :T] = qd[:, :, 2 * C:]
        q = q.contiguous()
    out, lse = _run(q, k, v, T, H)
    o_err = float(np.max(np.abs(out - ref_out[:, T - 1, :])))
    l_err = float(np.max(np.abs(lse - ref_lse[:, :, T - 1])))
    log(f"[parity] decode {layout} B={B} T={T} H={H}: o_maxabs={o_err:.3e} lse_maxabs={l_err:.3e}")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert o_err <= BF16_O_MAXABS and l_err <= BF16_LSE_MAXABS


def test_decode_matches_the_fused_forward_and_is_deterministic():
    """At the GPT-2 124M layer shape the decode of the last position agrees
    with the last row of attn_fwd, and two runs agree bit for bit."""
    B, T, H = 16, 1024, 12
    C = H * D
    qkv, _ = I.attention_inputs(B, T, H, D, "bf16", 1.0, 0.01, seed=7)
    qd = to_device(qkv, "bf16")
    out_f, lse_f = binding.forward(qd, H)
    q, k, v = qd[:, T - 1, :C], qd[:, :, C:2 * C], qd[:, :, 2 * C:]
    o1, l1 = _run(q, k, v, T, H)
    o2, l2 = _run(q, k, v, T, H)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.max(np.abs(o1 - to_host64(out_f)[:, T - 1, :])) <= 2 * BF16_O_MAXABS
    assert np.max(np.abs(l1 - to_host64(lse_f)[:, :, T - 1])) <= 2 * BF16_LSE_MAXABS
