"""The measurement probes (attn_peak_mfma, attn_peak_copy) do the work they
are credited with (needs a GPU).

attn_peak_mfma: every wave multiplies the same operands `iters` times into
eight accumulators, so each lane's output is 8 * iters times the sum of its
sixteen elements of one 32x32x16 product, computed here in float64 from the
operand values and the MFMA's lane layout (A: lane l holds row l % 32 and k
8 (l / 32) .. +7; B: lane l holds column l % 32 and the same k; C: lane l
holds column l % 32, rows 8 (i / 4) + 4 (l / 32) + i % 4). attn_peak_copy:
the copy is bit-exact and writes nothing past its end. attn_peak_read: the
XOR of its per-workgroup outputs is the XOR of every 32-bit word read.
"""

import numpy as np
import pytest

from causal_flash_attention_amd import binding

from helpers import log

pytestmark = pytest.mark.gpu


def _operands():
    lanes = np.arange(64)
    x = 1.0 + (lanes & 7) / 128.0
    y = ((lanes >> 3) + 1) / 1024.0
    A = np.zeros((32, 16))
    Bm = np.zeros((16, 32))
    for l in range(64):
        r, h = l % 32, l // 32
        for e in range(8):
            A[r, 8 * h + e] = x[l] if e % 2 == 0 else y[l]
            Bm[8 * h + e, r] = y[l] if e % 2 == 0 else x[l]
    return A @ Bm


def test_peak_mfma_computes_its_products():
    import torch
    n_wg, iters = 8, 16
    log(f"[case] peak mfma n_wg={n_wg} iters={iters}")
    out = torch.full((256 * n_wg,), float("nan"), dtype=torch.float32, device="cuda")
    ticks = torch.zeros(2 * n_wg, dtype=torch.int64, device="cuda")
    binding.attn_peak_mfma(out, ticks, n_wg, iters)
    torch.cuda.synchronize()
    C = _operands()
    want = np.zeros(64)
    for l in range(64):
        rows = [8 * (i // 4) + 4 * (l // 32) + i % 4 for i in range(16)]
        want[l] = 8 * iters * C[rows, l % 32].sum()
    got = out.cpu().numpy().astype(np.float64).reshape(n_wg * 4, 64)
    assert np.allclose(got, want[None, :], rtol=1e-5, atol=0), np.abs(got - want).max()
    t = ticks.cpu().numpy().reshape(n_wg, 2)
    assert np.all(t > 0)
    ghz = t[:, 0] / t[:, 1] * 0.1
    log(f"[probe] clock under a short MFMA loop: {np.median(ghz):.2f} GHz")
    assert np.all((ghz > 0.3) & (ghz < 3.5))


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (8 << 20) + 48])
def test_peak_copy_is_exact(nbytes):
    import torch
    log(f"[case] peak copy {nbytes} bytes")
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.full((nbytes + 256,), 0xAB, dtype=torch.uint8, device="cuda")
    st = binding.lib().attn_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                                      torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xAB).all())


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (8 << 20) + 48])
def test_peak_read_reads_everything(nbytes):
    import torch
    log(f"[case] peak read {nbytes} bytes")
    g = torch.Generator(device="cpu").manual_seed(nbytes + 1)
    words = torch.randint(0, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    src = words.cuda()
    out = torch.zeros(binding.lib().attn_peak_read_slots(), dtype=torch.int32, device="cuda")
    binding.attn_peak_read(src, out)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(words.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == want
