"""attn_bwd_noalloc, the backward whose workspace is the library's own
per-GPU array, against attn_bwd with a caller workspace (needs a GPU): the
same dqkv bit for bit, on two calls in a row, the second smaller (so it runs
on what the first left in the array), and on a shape at the array's limit."""

import pytest

from causal_flash_attention_amd import binding
from causal_flash_attention_amd import inputs as I

from helpers import log, to_device

pytestmark = pytest.mark.gpu

D = 64


def _case(B, T, H, seed):
    import torch
    log(f"[case] noalloc B={B} T={T} H={H} seed={seed}")
    qkv, dout = I.attention_inputs(B, T, H, D, "bf16", 1.0, 0.01, seed=seed)
    qd, gd = to_device(qkv, "bf16"), to_device(dout, "bf16")
    out, lse = binding.forward(qd, H)
    ref = torch.full_like(qd, float("nan"))
    ws = torch.full((binding.workspace_floats(B, T, H),), float("nan"), dtype=torch.float32,
                    device="cuda")
    binding.attn_bwd(gd, qd, out, lse, ref, ws, H)
    got = torch.full_like(qd, float("nan"))
    binding.attn_bwd_noalloc(gd, qd, out, lse, got, H)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (B, T, H)
    assert torch.isfinite(got.float()).all()


def test_noalloc_matches_attn_bwd_twice():
    _case(3, 700, 5, seed=901)     # fills part of the array
    _case(2, 130, 3, seed=902)     # smaller: runs over the first call's leftovers


def test_noalloc_at_limit_and_beyond():
    import torch
    # 10 * 16 * 12 * 1024 floats: the GPT-2 124M layer shape fits.
    _case(16, 1024, 12, seed=903)
    B, T, H = 64, 1089, 12  # 10 * 64 * 12 * 1152 floats: over the limit
    assert binding.workspace_floats(B, T, H) > binding.noalloc_max_floats()
    qd = torch.zeros((1, 1, 3 * H * D), dtype=torch.bfloat16, device="cuda")
    st = binding.lib().attn_bwd_noalloc(qd.data_ptr(), qd.data_ptr(), qd.data_ptr(),
                                        qd.data_ptr(), qd.data_ptr(), B, T, H, D, None)
    assert st == -4  # ATTN_ERR_TOO_LARGE, before any launch
