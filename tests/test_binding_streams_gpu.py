"""The allocating wrappers of the binding on a stream other than torch's
current one (needs a GPU): forward, backward, forward_fp8 and backward_fp8
launched on a side stream give the same bits as on the default stream, and
their scratch buffers, allocated on that stream, are not handed to other
work while its kernels may still read them."""

import numpy as np
import pytest

from causal_flash_attention_amd import binding
from causal_flash_attention_amd import inputs as I

from helpers import log, to_device

pytestmark = pytest.mark.gpu

D = 64


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_wrappers_on_side_stream():
    import torch
    B, T, H = 2, 333, 3
    log(f"[case] side stream B={B} T={T} H={H}")
    qkv, dout = I.attention_inputs(B, T, H, D, "bf16", 1.0, 0.01, seed=4321)
    qd, gd = to_device(qkv, "bf16"), to_device(dout, "bf16")
    ref_o, ref_l = binding.forward(qd, H)
    ref_g = binding.backward(gd, qd, ref_o, ref_l, H)
    ref_o8, ref_l8 = binding.forward_fp8(qd, H)
    ref_g8 = binding.backward_fp8(gd, qd, ref_o8, ref_l8, H)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        o, l = binding.forward(qd, H, stream=side)
        g = binding.backward(gd, qd, o, l, H, stream=side)
        o8, l8 = binding.forward_fp8(qd, H, stream=side)
        g8 = binding.backward_fp8(gd, qd, o8, l8, H, stream=side)
        # Work on the default stream meanwhile, allocating and freeing
        # memory of the same sizes as the wrappers' scratch buffers.
        for _ in range(4):
            junk = torch.full((binding.workspace_floats(B, T, H),), float("nan"), device="cuda")
            junk8 = torch.full((binding.fp8_bwd_buffer_bytes(B, T, H),), 0xAB, dtype=torch.uint8,
                               device="cuda")
            del junk, junk8
        side.synchronize()
        for name, a, b in (("out", o, ref_o), ("lse", l, ref_l), ("dqkv", g, ref_g),
                           ("out fp8", o8, ref_o8), ("lse fp8", l8, ref_l8), ("dqkv fp8", g8, ref_g8)):
            assert torch.equal(_bits(a), _bits(b)), (rep, name)
    assert np.isfinite(ref_g.float().cpu().numpy()).all()
