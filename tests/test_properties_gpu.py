"""Properties of the HIP library that hold at any size (needs a GPU).

Bitwise causality and run-to-run determinism of every output, the stage
entry points against attn_bwd, the backward workspace contents, sentinel
guard bands around ragged outputs, element offsets beyond 2^31, empty
problems, and the gradient-sum identities at the full GPT-2 124M shape.
"""

import numpy as np
import pytest

import oracle
from causal_flash_attention_amd import binding
from causal_flash_attention_amd import inputs as I

from helpers import (BF16_GRAD_REL_L2, BF16_LSE_MAXABS, BF16_O_MAXABS, compare, log,
                     run_library, to_device, to_host64)

pytestmark = pytest.mark.gpu

D = 64


def _inputs(B, T, H, dtype, seed, dout_std=None):
    if dout_std is None:
        dout_std = 0.01 if dtype == "bf16" else 1.0
    qkv, dout = I.attention_inputs(B, T, H, D, dtype, 1.0, dout_std, seed=seed)
    return qkv, dout


def _bits(t):
    import torch
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causality_is_bitwise(dtype):
    B, T, H, t = 2, 300, 3, 173
    log(f"[case] causality {dtype} B={B} T={T} H={H} t={t}")
    qkv, dout = _inputs(B, T, H, dtype, seed=21)
    dout_a = dout.copy()
    dout_a[:, t:] = 0  # later queries then feed exact zeros into dK, dV
    qkv_b = qkv.copy()
    noise = _inputs(B, T, H, dtype, seed=22)[0]
    qkv_b[:, t:] = noise[:, t:]
    ra = run_library(to_device(qkv, dtype), to_device(dout_a, dtype), H)
    rb = run_library(to_device(qkv_b, dtype), to_device(dout_a, dtype), H)
    oa, la, ga = (_bits(x) for x in ra)
    ob, lb, gb = (_bits(x) for x in rb)
    assert np.array_equal(oa[:, :t], ob[:, :t])
    assert np.array_equal(la[:, :, :t], lb[:, :, :t])
    assert np.array_equal(ga[:, :t], gb[:, :t])  # dQ, dK and dV of earlier rows
    assert not np.array_equal(oa[:, t:], ob[:, t:])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causality_is_bitwise_when_later_rows_rescale(dtype):
    """As above, but the later tokens get Q and K scaled by 8, so their rows
    take the forward's rescale path on almost every tile while the earlier
    rows of the same waves (t = 173 falls inside the 32-row wave 160-191)
    do not: a row that did not ask for a rescale must come out the same."""
    B, T, H, t = 2, 300, 3, 173
    C = H * D
    log(f"[case] causality with rescales {dtype} B={B} T={T} H={H} t={t}")
    qkv, dout = _inputs(B, T, H, dtype, seed=23)
    dout_a = dout.copy()
    dout_a[:, t:] = 0
    noise = _inputs(B, T, H, dtype, seed=24)[0]
    x = I.bf16_bits_to_f32(noise) if dtype == "bf16" else noise.copy()
    x[..., :2 * C] *= np.float32(8.0)  # a power of two: exact in bf16 and f32
    noise = I.f32_to_bf16_bits(x) if dtype == "bf16" else x
    qkv_b = qkv.copy()
    qkv_b[:, t:] = noise[:, t:]
    ra = run_library(to_device(qkv, dtype), to_device(dout_a, dtype), H)
    rb = run_library(to_device(qkv_b, dtype), to_device(dout_a, dtype), H)
    oa, la, ga = (_bits(x) for x in ra)
    ob, lb, gb = (_bits(x) for x in rb)
    assert np.array_equal(oa[:, :t], ob[:, :t])
    assert np.array_equal(la[:, :, :t], lb[:, :, :t])
    assert np.array_equal(ga[:, :t], gb[:, :t])
    assert not np.array_equal(oa[:, t:], ob[:, t:])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_runs_are_bitwise_identical(dtype):
    B, T, H = 2, 1000, 3
    log(f"[case] determinism {dtype}")
    qkv, dout = _inputs(B, T, H, dtype, seed=31)
    qd, gd = to_device(qkv, dtype), to_device(dout, dtype)
    r1 = [_bits(x) for x in run_library(qd, gd, H)]
    r2 = [_bits(x) for x in run_library(qd, gd, H)]
    for a, b in zip(r1, r2):
        assert np.array_equal(a, b)


def test_stage_entry_points_match_attn_bwd():
    import torch
    B, T, H = 3, 257, 5
    log("[case] stage entry points")
    qkv, dout = _inputs(B, T, H, "bf16", seed=41)
    qd, gd = to_device(qkv, "bf16"), to_device(dout, "bf16")
    out, lse = binding.forward(qd, H)
    nws = binding.workspace_floats(B, T, H)
    ws_a = torch.full((nws,), float("nan"), device="cuda")
    dqkv_a = torch.full_like(qd, float("nan"))
    binding.attn_bwd(gd, qd, out, lse, dqkv_a, ws_a, H)
    # three stages: preprocess, then dQ and dK/dV in either order
    ws = torch.full((nws,), float("nan"), device="cuda")
    dqkv_b = torch.full_like(qd, float("nan"))
    binding.attn_bwd_preprocess(gd, out, lse, ws, H)
    binding.attn_bwd_dq(gd, qd, ws, dqkv_b, H)
    binding.attn_bwd_dkdv(gd, qd, ws, dqkv_b, H)
    # the fused first stage, then dK/dV
    ws_c = torch.full((nws,), float("nan"), device="cuda")
    dqkv_c = torch.full_like(qd, float("nan"))
    binding.attn_bwd_dq_preprocess(gd, qd, out, lse, dqkv_c, ws_c, H)
    binding.attn_bwd_dkdv(gd, qd, ws_c, dqkv_c, H)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dqkv_a), _bits(dqkv_b))
    assert np.array_equal(_bits(dqkv_a), _bits(dqkv_c))
    for w_ in (ws_a, ws_c):
        assert np.array_equal(w_.cpu().numpy().view(np.uint32), ws.cpu().numpy().view(np.uint32))
    # workspace: D = rowsum(dout * out) in float32, then LSE * log2(e); padding
    Tp = (T + 63) // 64 * 64
    R = B * H * Tp
    w_all = ws.cpu().numpy()
    assert w_all.size == 10 * R
    w = w_all[:2 * R].reshape(2, B, H, Tp)
    g64 = I.to_float64(dout, "bf16").reshape(B, T, H, D)
    o64 = to_host64(out).reshape(B, T, H, D)
    d_ref = np.einsum("bthk,bthk->bht", g64, o64)
    np.testing.assert_allclose(w[0, :, :, :T], d_ref, rtol=1e-5, atol=1e-7)
    assert np.all(w[0, :, :, T:] == 0.0)
    l_ref = lse.cpu().numpy().astype(np.float64) * np.log2(np.e)
    np.testing.assert_allclose(w[1, :, :, :T], l_ref, rtol=1e-6, atol=1e-6)
    assert np.all(np.isposinf(w[1, :, :, T:]))
    # then 32 bytes per row in groups of 32 rows (the group's m chunks, then
    # its D chunks): bf16 terms [m1 m2 m3 0 0 0 0 0] and [d1 d2 d3 0 0 0 0 0]
    # summing to m = 8 * LSE and to D; rows past T: m1 = largest finite bf16
    grouped = w_all[2 * R:].view(np.uint16).reshape(B, H, Tp // 32, 2, 32, 8)
    bits = grouped.transpose(0, 1, 2, 4, 3, 5).reshape(B, H, Tp, 2, 8)
    terms = I.bf16_bits_to_f32(bits).astype(np.float64)
    assert np.all(bits[..., 3:] == 0)
    m_sum = terms[:, :, :, 0, :3].sum(-1)
    d_sum = terms[:, :, :, 1, :3].sum(-1)
    m_ref = (np.float32(8.0) * lse.cpu().numpy()).astype(np.float64)
    np.testing.assert_allclose(m_sum[:, :, :T], m_ref, rtol=1e-7, atol=1e-30)
    np.testing.assert_allclose(d_sum[:, :, :T], w[0, :, :, :T].astype(np.float64), rtol=1e-7, atol=1e-30)
    assert np.all(bits[:, :, T:, 0, 0] == 0x7F7F) and np.all(bits[:, :, T:, 0, 1:] == 0)
    assert np.all(bits[:, :, T:, 1, :] == 0)


@pytest.mark.parametrize("dtype,T", [("bf16", 129), ("bf16", 1000), ("f32", 65)])
def test_guard_bands_untouched(dtype, T):
    import torch
    B, H = 2, 3
    C = H * D
    log(f"[case] guard bands {dtype} T={T}")
    qkv, dout = _inputs(B, T, H, dtype, seed=51)
    qd, gd = to_device(qkv, dtype), to_device(dout, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    pad = 64  # elements on each side; keeps 16-byte alignment for both dtypes

    def guarded(n, dt):
        buf = torch.empty(n + 2 * pad, dtype=dt, device="cuda")
        if dt == torch.bfloat16:
            buf.view(torch.int16).fill_(0x7FC1)  # a NaN pattern
        else:
            buf.view(torch.int32).fill_(0x7FC00001)
        return buf, buf[pad:pad + n]

    out_b, out = guarded(B * T * C, tdt)
    lse_b, lse = guarded(B * H * T, torch.float32)
    dq_b, dqkv = guarded(B * T * 3 * C, tdt)
    ws_b, ws = guarded(binding.workspace_floats(B, T, H), torch.float32)
    before = [_bits(x).copy() for x in (out_b, lse_b, dq_b, ws_b)]
    binding.attn_fwd(qd, out.view(B, T, C), lse.view(B, H, T), H)
    binding.attn_bwd(gd, qd, out.view(B, T, C), lse.view(B, H, T), dqkv.view(B, T, 3 * C), ws, H)
    torch.cuda.synchronize()
    for b0, x in zip(before, (out_b, lse_b, dq_b, ws_b)):
        after = _bits(x)
        assert np.array_equal(after[:pad], b0[:pad])
        assert np.array_equal(after[-pad:], b0[-pad:])
    for x in (out, lse, dqkv):
        assert np.all(np.isfinite(x.float().cpu().numpy()))


def test_element_offsets_beyond_2_31():
    """B = 1024 at the GPT-2 124M layer shape: qkv holds 2.4e9 elements, so
    the last batch rows sit past 2^31 elements. Rows repeat two seeded rows;
    heads of the first and last batch rows are checked against the oracle."""
    import torch
    B, T, H = 1024, 1024, 12
    C = H * D
    log(f"[case] offsets beyond 2^31: B={B} T={T} H={H}")
    qkv2, dout2 = _inputs(2, T, H, "bf16", seed=61)
    q2, g2 = to_device(qkv2, "bf16"), to_device(dout2, "bf16")
    qkv = q2.repeat(B // 2, 1, 1)
    dout = g2.repeat(B // 2, 1, 1)
    assert qkv.numel() > 2 ** 31
    out, lse, dqkv = run_library(qkv, dout, H)
    q64, g64 = I.to_float64(qkv2, "bf16"), I.to_float64(dout2, "bf16")
    for b in (0, B - 1):
        src = b % 2
        heads = [(src, 0), (src, H - 1)]
        ref_o, ref_l = oracle.forward_packed(q64, H, D, heads=heads)
        ref_d = oracle.backward_packed(g64, q64, H, D, heads=heads)
        gpu = {"out": to_host64(out[b:b + 1]), "lse": to_host64(lse[b:b + 1]),
               "dqkv": to_host64(dqkv[b:b + 1])}
        ref = {"out": ref_o[src:src + 1], "lse": ref_l[src:src + 1], "dqkv": ref_d[src:src + 1]}
        m = compare(gpu, ref, [(0, 0), (0, H - 1)], H, D)
        log(f"[parity] offsets b={b}: {m}")
        assert m["o_maxabs"] <= BF16_O_MAXABS and m["lse_maxabs"] <= BF16_LSE_MAXABS
        for k in ("dq", "dk", "dv"):
            assert m[f"{k}_rel_l2"] <= BF16_GRAD_REL_L2
    del qkv, dout, out, lse, dqkv
    torch.cuda.empty_cache()


def test_empty_problems_on_gpu():
    import torch
    for B, T in ((0, 64), (2, 0)):
        qkv = torch.empty(B, T, 3 * 2 * D, dtype=torch.bfloat16, device="cuda")
        out, lse = binding.forward(qkv, 2)
        dqkv = binding.backward(torch.empty(B, T, 2 * D, dtype=torch.bfloat16, device="cuda"),
                                qkv, out, lse, 2)
        torch.cuda.synchronize()
        assert out.numel() == 0 and dqkv.numel() == 0


def test_gradient_sums_at_headline_shape():
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i for every (b, h) of the
    GPT-2 124M layer (B=16, T=1024, H=12), within bf16 rounding of the
    summed terms."""
    import torch
    B, T, H = 16, 1024, 12
    log("[case] gradient sums at the headline shape")
    qkv, dout = _inputs(B, T, H, "bf16", seed=0)
    qd, gd = to_device(qkv, "bf16"), to_device(dout, "bf16")
    _out, _lse, dqkv = run_library(qd, gd, H)
    g = dqkv.float().view(B, T, 3, H, D)
    dk, dv = g[:, :, 1], g[:, :, 2]
    go = gd.float().view(B, T, H, D)
    sum_dk = dk.sum(1)                       # (B, H, D)
    scale_dk = dk.abs().sum(1)
    assert float((sum_dk.abs() / scale_dk.clamp_min(1e-30)).max()) < 2e-2
    err_dv = (dv.sum(1) - go.sum(1)).abs()
    assert float((err_dv / dv.abs().sum(1).clamp_min(1e-30)).max()) < 2e-2
