"""FP8 (MXFP8) attention backward against the CPU float64 FP8 oracle (needs a
GPU).

The backward buffer is integer work plus two float rows: every code and
exponent byte (padding included) must equal the oracle's quantization bit for
bit; LSE * log2(e) must equal its float32 product exactly; D must match its
float64 value to float32 rounding. The gradients are compared with
oracle.fp8.head_backward_fp8 at the attention backward's bar (relative L2
<= 2e-2 on each of dQ, dK, dV). Both sides take the same forward results,
made by the oracle alone: the FP8 oracle's O rounded to bf16 and its LSE
rounded to float32, so no input of the oracle comes from the GPU (heads that
are not compared take the GPU forward's values, as inputs of the GPU
backward only). The
kernel's probabilities and dS differ from the oracle's only by the FP8
matrix cores' accumulation (about 14 bits) and float32 arithmetic, which can
move single E4M3 codes across a rounding midpoint, not by any rounding of
the definition.
"""

import numpy as np
import pytest

import oracle
import oracle.fp8 as F
from causal_flash_attention_amd import binding
from causal_flash_attention_amd import inputs as I

from helpers import BF16_GRAD_REL_L2, log, sample_heads, to_device, to_host64

pytestmark = pytest.mark.gpu

D = 64
LOG2E32 = np.float32(1.4426950408889634)


def _unpack_bwd(buf, B, T, H):
    BH, Tp = B * H, (T + 63) // 64 * 64
    NT = Tp // 64
    n = BH * Tp * 64
    vc = buf[:n].reshape(BH, Tp, 64)
    gc = buf[n:2 * n].reshape(BH, Tp, 64)
    qp = buf[2 * n:3 * n].reshape(BH, 64, Tp)
    kp = buf[3 * n:4 * n].reshape(BH, 64, Tp)
    gp = buf[4 * n:5 * n].reshape(BH, 64, Tp)
    side = buf[5 * n:5 * n + BH * NT * 1152].reshape(BH, NT, 1152)
    ex = {"v": side[:, :, 0:128].reshape(BH, Tp, 2), "kp": side[:, :, 128:256].reshape(BH, 2 * NT, 64),
          "g": side[:, :, 256:384].reshape(BH, Tp, 2), "qp": side[:, :, 384:512].reshape(BH, 2 * NT, 64),
          "gp": side[:, :, 512:640].reshape(BH, 2 * NT, 64)}
    lse2 = np.ascontiguousarray(side[:, :, 640:896]).view(np.float32).reshape(BH, Tp)
    dd = np.ascontiguousarray(side[:, :, 896:1152]).view(np.float32).reshape(BH, Tp)
    return vc, gc, qp, kp, gp, ex, lse2, dd


def _inputs(B, T, H, std, seed):
    qkv, dout = I.attention_inputs(B, T, H, D, "bf16", std, 1.0, seed=seed)
    return qkv, dout


def _forward(qkv_dev, H):
    import torch
    out, lse = binding.forward_fp8(qkv_dev, H)
    torch.cuda.synchronize()
    return out, lse


def _check_grads(dqkv, qkv64, dout64, out64, lse64, H, heads, tag):
    C = H * D
    errs = {"dq": [0.0, 0.0], "dk": [0.0, 0.0], "dv": [0.0, 0.0]}
    for b, h in heads:
        q, k, v = oracle.split_packed_head(qkv64, b, h, H, D)
        lo = h * D
        g, o = dout64[b, :, lo:lo + D], out64[b, :, lo:lo + D]
        rq, rk, rv = F.head_backward_fp8(q, k, v, g, o, lse64[b, h])
        got = (dqkv[b, :, lo:lo + D], dqkv[b, :, C + lo:C + lo + D], dqkv[b, :, 2 * C + lo:2 * C + lo + D])
        for name, a, r in zip(("dq", "dk", "dv"), got, (rq, rk, rv)):
            errs[name][0] += float(((a - r) ** 2).sum())
            errs[name][1] += float((r ** 2).sum())
    rel = {k: (v[0] / max(v[1], 1e-300)) ** 0.5 for k, v in errs.items()}
    log(f"[parity] fp8 bwd {tag}: rel-L2 dQ {rel['dq']:.2e} dK {rel['dk']:.2e} dV {rel['dv']:.2e}")
    for k, v in rel.items():
        assert v <= BF16_GRAD_REL_L2, (tag, k, v)
    return rel


def _oracle_forward(qkv, qd, B, T, H, heads):
    """O (bf16 bits) and LSE (float32) for the backward: the FP8 oracle's
    forward on the listed heads; the other heads (never compared) keep the
    GPU forward's values."""
    import torch
    q64 = I.to_float64(qkv, "bf16")
    if len(heads) < B * H:
        out_d, lse_d = _forward(qd, H)
        out_bits = out_d.view(torch.int16).cpu().numpy().view(np.uint16).copy()
        lse32 = lse_d.cpu().numpy().copy()
    else:
        out_bits = np.zeros((B, T, H * D), dtype=np.uint16)
        lse32 = np.zeros((B, H, T), dtype=np.float32)
    ref_o, ref_l = F.forward_packed_fp8(q64, H, D, heads=heads)
    for b, h in heads:
        sl = slice(h * D, (h + 1) * D)
        out_bits[b, :, sl] = I.f32_to_bf16_bits(ref_o[b, :, sl].astype(np.float32))
        lse32[b, h] = ref_l[b, h].astype(np.float32)
    return out_bits, lse32


def _run_bwd(qkv, dout, B, T, H, heads=None):
    """GPU FP8 backward on the oracle's forward results; returns the float64
    O and LSE both sides use and the GPU's dqkv."""
    import torch
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    qd, gd = to_device(qkv, "bf16"), to_device(dout, "bf16")
    out_bits, lse32 = _oracle_forward(qkv, qd, B, T, H, heads)
    out, lse = to_device(out_bits, "bf16"), torch.from_numpy(lse32).to("cuda")
    dqkv = binding.backward_fp8(gd, qd, out, lse, H)
    torch.cuda.synchronize()
    o64 = I.bf16_bits_to_f32(out_bits).astype(np.float64)
    return o64, lse32.astype(np.float64), to_host64(dqkv), (qd, gd, out, lse)


@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (2, 63, 2), (2, 65, 3), (1, 200, 2)])
def test_fp8_bwd_buffer(B, T, H):
    """Backward buffer: codes and exponents bit-exact, padding zero, LSE2 and D."""
    import torch
    log(f"[case] fp8 bwd buffer B={B} T={T} H={H}")
    qkv, dout = _inputs(B, T, H, 1.0, 2100 + T)
    qd, gd = to_device(qkv, "bf16"), to_device(dout, "bf16")
    out_bits, lse32 = _oracle_forward(qkv, qd, B, T, H, [(b, h) for b in range(B) for h in range(H)])
    out, lse = to_device(out_bits, "bf16"), torch.from_numpy(lse32).to("cuda")
    buf = torch.full((binding.fp8_bwd_buffer_bytes(B, T, H),), 0xAB, dtype=torch.uint8, device="cuda")
    binding.attn_quantize_bwd_fp8(gd, qd, out, lse, buf, H)
    torch.cuda.synchronize()
    vc, gc, qp, kp, gp, ex, lse2, dd = _unpack_bwd(buf.cpu().numpy(), B, T, H)
    q64, g64 = I.to_float64(qkv, "bf16"), I.to_float64(dout, "bf16")
    o64 = I.bf16_bits_to_f32(out_bits).astype(np.float64)
    C = H * D
    T32 = -(-T // 32) * 32
    for b in range(B):
        for h in range(H):
            bh = b * H + h
            q, k, v = oracle.split_packed_head(q64, b, h, H, D)
            g = g64[b, :, h * D:(h + 1) * D]
            for name, codes, exps, x in (("v", vc, "v", v), ("g", gc, "g", g)):
                c, e, _ = F.quantize_blocks(x, axis=1)
                assert np.array_equal(codes[bh, :T], c), f"{name} codes (channel blocks) head {b, h}"
                assert np.array_equal(ex[exps][bh, :T], e + 127), f"{name} exponents head {b, h}"
                assert not codes[bh, T:].any() and not ex[exps][bh, T:].any()
            for name, codes, exps, x in (("q", qp, "qp", q), ("k", kp, "kp", k), ("g", gp, "gp", g)):
                c, e, _ = F.quantize_positions(x)
                assert np.array_equal(codes[bh].T[:T32], c), f"{name} codes (position blocks) head {b, h}"
                assert np.array_equal(ex[exps][bh, :T32 // 32], e + 127), f"{name} exps head {b, h}"
                assert not codes[bh, :, T32:].any() and not ex[exps][bh, T32 // 32:].any()
            want = (lse32[b, h] * LOG2E32).astype(np.float32)
            assert np.array_equal(lse2[bh, :T], want), f"LSE2 head {b, h}"
            assert np.all(np.isinf(lse2[bh, T:])) and np.all(lse2[bh, T:] > 0)
            ref_d = (g * o64[b, :, h * D:(h + 1) * D]).sum(axis=1)
            assert np.allclose(dd[bh, :T], ref_d, rtol=1e-5, atol=1e-6), f"D head {b, h}"
            assert not dd[bh, T:].any()
    del C


@pytest.mark.parametrize("B,T,H,std", [(1, 1, 1, 1.0), (2, 63, 2, 1.0), (1, 64, 1, 1.0),
                                       (2, 65, 3, 1.0), (1, 200, 2, 1.0), (2, 512, 2, 1.0),
                                       (1, 1024, 2, 1.0), (1, 300, 2, 3.0)])
def test_fp8_bwd_parity(B, T, H, std):
    log(f"[case] fp8 bwd B={B} T={T} H={H} std={std}")
    qkv, dout = _inputs(B, T, H, std, 2300 + T)
    out64, lse64, dqkv, _ = _run_bwd(qkv, dout, B, T, H)
    _check_grads(dqkv, I.to_float64(qkv, "bf16"), I.to_float64(dout, "bf16"), out64, lse64, H,
                 [(b, h) for b in range(B) for h in range(H)], f"B={B} T={T} H={H} std={std}")


def test_fp8_bwd_headline_sampled():
    """GPT-2 124M layer shape (B 16, T 1024, 12 heads) on sampled heads."""
    B, T, H = 16, 1024, 12
    log(f"[case] fp8 bwd headline B={B} T={T} H={H}")
    qkv, dout = _inputs(B, T, H, 1.0, 2024)
    heads = sample_heads(B, H, 4, seed=5)
    out64, lse64, dqkv, _ = _run_bwd(qkv, dout, B, T, H, heads)
    _check_grads(dqkv, I.to_float64(qkv, "bf16"), I.to_float64(dout, "bf16"), out64, lse64, H,
                 heads, "headline")


def test_fp8_bwd_deterministic_and_close_to_exact():
    """Two runs agree bit for bit; the whole FP8 chain (the GPU's FP8 forward,
    then its backward) stays within about 2^-3 (relative L2) of the exact
    gradients of the unquantized inputs."""
    import torch
    B, T, H = 2, 256, 2
    qkv, dout = _inputs(B, T, H, 1.0, 77)
    qd, gd = to_device(qkv, "bf16"), to_device(dout, "bf16")
    out, lse = _forward(qd, H)
    a = binding.backward_fp8(gd, qd, out, lse, H)
    b = binding.backward_fp8(gd, qd, out, lse, H)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle.backward_packed(I.to_float64(dout, "bf16"), I.to_float64(qkv, "bf16"), H, D)
    got = to_host64(a)
    C = H * D
    for s, name in ((slice(0, C), "dQ"), (slice(C, 2 * C), "dK"), (slice(2 * C, 3 * C), "dV")):
        rel = np.linalg.norm(got[..., s] - ref[..., s]) / np.linalg.norm(ref[..., s])
        log(f"[accuracy] fp8 bwd {name} vs exact: rel-L2 {rel:.4f}")
        assert rel < 0.12
