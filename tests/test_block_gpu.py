"""The attention block (attn_block_fwd / attn_block_bwd) against the CPU
float64 oracle of the same layer (needs a GPU).

The GPU path stores qkv, att, datt and dqkv in bf16 between its kernels
(fp32 inside each), the oracle nothing. Each of those roundings is at most
2^-9 relative per element and the maps between them are well conditioned
at these scales, so the outputs are held to relative L2 bars: 2e-2 on every
gradient (the attention backward's own bar), 1e-2 on y and 4e-3 on qkv (one
rounding after an fp32 product). LSE moves with the rounding of q and k
themselves (up to 2^-9 relative each, so a score q.k / 8 moves by up to
2^-8 |q| |k| / 8): its bound per row is 1e-3 plus that for the row's query
and its largest visible key. Inputs follow GPT-2's initialisation scale:
x ~ N(0, 1), weights and biases ~ N(0, 0.02^2), dy ~ N(0, 1), drawn from the
shared seeded generator.
"""

import numpy as np
import pytest

import oracle.block as K
from causal_flash_attention_amd import binding
from causal_flash_attention_amd import inputs as I

from helpers import log, to_device, to_host64

pytestmark = pytest.mark.gpu

D = 64
GRAD_REL = 2e-2
Y_REL = 1e-2
QKV_REL = 4e-3


def _draw(B, T, H, seed):
    C = H * D
    shapes = {"x": ((B, T, C), 1.0), "w_attn": ((C, 3 * C), 0.02), "b_attn": ((3 * C,), 0.02),
              "w_proj": ((C, C), 0.02), "b_proj": ((C,), 0.02), "dy": ((B, T, C), 1.0)}
    return {k: I.normal(s, std, seed, 10 + i, "bf16") for i, (k, (s, std)) in enumerate(shapes.items())}


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _run(B, T, H, seed):
    import torch
    C = H * D
    h = _draw(B, T, H, seed)
    d = {k: to_device(v, "bf16") for k, v in h.items()}
    bf, f32 = torch.bfloat16, torch.float32
    dev = "cuda"
    qkv = torch.full((B, T, 3 * C), float("nan"), dtype=bf, device=dev)
    att = torch.full((B, T, C), float("nan"), dtype=bf, device=dev)
    lse = torch.full((B, H, T), float("nan"), dtype=f32, device=dev)
    y = torch.full((B, T, C), float("nan"), dtype=bf, device=dev)
    binding.attn_block_fwd(d["x"], d["w_attn"], d["b_attn"], d["w_proj"], d["b_proj"], qkv, att,
                           lse, y, H)
    datt = torch.full((B, T, C), float("nan"), dtype=bf, device=dev)
    dqkv = torch.full((B, T, 3 * C), float("nan"), dtype=bf, device=dev)
    dx = torch.full((B, T, C), float("nan"), dtype=bf, device=dev)
    g = {"dw_attn": torch.full((C, 3 * C), float("nan"), device=dev),
         "db_attn": torch.full((3 * C,), float("nan"), device=dev),
         "dw_proj": torch.full((C, C), float("nan"), device=dev),
         "db_proj": torch.full((C,), float("nan"), device=dev)}
    ws = torch.full((binding.block_workspace_bytes(B, T, H) // 4,), float("nan"), device=dev)
    binding.attn_block_bwd(d["dy"], d["x"], d["w_attn"], d["w_proj"], qkv, att, lse, datt, dqkv,
                           dx, g["dw_attn"], g["db_attn"], g["dw_proj"], g["db_proj"], ws, H)
    torch.cuda.synchronize()
    got = {"qkv": qkv, "att": att, "lse": lse, "y": y, "datt": datt, "dqkv": dqkv, "dx": dx, **g}
    return h, {k: to_host64(v) for k, v in got.items()}


def _check(B, T, H, seed, tag):
    h, got = _run(B, T, H, seed)
    f64 = {k: I.to_float64(v, "bf16") for k, v in h.items()}
    ref_f = K.block_forward(f64["x"], f64["w_attn"], f64["b_attn"], f64["w_proj"], f64["b_proj"],
                            H, D)
    ref_b = K.block_backward(f64["dy"], f64["x"], f64["w_attn"], f64["w_proj"], ref_f, H, D)
    for k, v in got.items():
        assert np.all(np.isfinite(v)), f"{tag}: {k} has non-finite values"
    C = H * D
    qkv = ref_f["qkv"]
    qn = np.linalg.norm(qkv[..., :C].reshape(B, T, H, D), axis=3)          # (B, T, H)
    kn = np.linalg.norm(qkv[..., C:2 * C].reshape(B, T, H, D), axis=3)
    kmax = np.maximum.accumulate(kn, axis=1)                               # over keys <= t
    lse_bound = 1e-3 + 2.0 ** -8 * qn * kmax / np.sqrt(D)                  # (B, T, H)
    lse_ratio = float((np.abs(got["lse"] - ref_f["lse"]) / lse_bound.transpose(0, 2, 1)).max())
    errs = {"qkv": _rel(got["qkv"], ref_f["qkv"]), "y": _rel(got["y"], ref_f["y"]),
            "lse": float(np.abs(got["lse"] - ref_f["lse"]).max()), "lse/bound": lse_ratio}
    for k in ("datt", "dqkv", "dx", "dw_attn", "db_attn", "dw_proj", "db_proj"):
        errs[k] = _rel(got[k], ref_b[k])
    log(f"[parity] block {tag}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert errs["qkv"] <= QKV_REL and errs["y"] <= Y_REL and errs["lse/bound"] <= 1.0, errs
    for k in ("datt", "dqkv", "dx", "dw_attn", "db_attn", "dw_proj", "db_proj"):
        assert errs[k] <= GRAD_REL, (k, errs[k])


# (4, 130, 4) and (3, 1000, 4) split the weight gradients' K = B * T unevenly
# (last chunks of 200 and 120 rows; 10 chunks for the second).
@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (1, 64, 2), (2, 100, 3), (4, 130, 4), (2, 256, 12),
                                   (3, 1000, 4)])
def test_block_parity(B, T, H):
    log(f"[case] block B={B} T={T} H={H}")
    _check(B, T, H, seed=40 + T, tag=f"B={B} T={T} H={H}")


def test_block_headline():
    """GPT-2 124M layer shape, B 16, T 1024, 12 heads: every output of the
    layer against the oracle (the weight gradients run split over K here)."""
    log("[case] block headline B=16 T=1024 H=12")
    _check(16, 1024, 12, seed=7, tag="headline")


def test_block_deterministic():
    B, T, H = 2, 192, 4
    _, a = _run(B, T, H, seed=3)
    _, b = _run(B, T, H, seed=3)
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{k} differs between runs"
