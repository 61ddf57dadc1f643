"""Shared helpers of the GPU tests: move seeded inputs to the device, run the
library through its binding, bring results back as float64, and compare them
with the CPU oracle on chosen heads."""

from __future__ import annotations

import sys

import numpy as np

from causal_flash_attention_amd import binding
from causal_flash_attention_amd import inputs as I

# Parity bars. bf16: max-abs 1e-2 on O, relative L2 2e-2 on each of dQ, dK,
# dV (each over all compared heads); LSE max-abs 1e-3 is an extra gate.
# float32: a flat max-abs 1e-5 on O, LSE, dQ, dK, dV for the tiny workload
# (B 1, T 64, 2 heads); longer float32 sequences scale that bound by the
# largest magnitude of the reference tensor (sums of up to T terms).
BF16_O_MAXABS = 1e-2
BF16_GRAD_REL_L2 = 2e-2
BF16_LSE_MAXABS = 1e-3
F32_MAXABS = 1e-5


# Every parity check of the session, in order: (label, dtype, metrics, bars).
# tests/conftest.py prints them after the run, so the numbers survive a
# quiet (-q) pytest run.
PARITY_RECORDS = []


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to("cuda")


def to_host64(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        u = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return I.bf16_bits_to_f32(u).astype(np.float64)
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_library(qkv_dev, dout_dev, n_head: int):
    """One forward and one backward through the C ABI; returns device tensors.
    The outputs and the backward workspace start as NaN, so an element a
    kernel leaves unwritten, or a workspace element read before it is
    written, shows up as a non-finite result instead of passing by luck."""
    import torch
    B, T, C3 = (int(x) for x in qkv_dev.shape)
    C = C3 // 3
    nan = float("nan")
    out = torch.full((B, T, C), nan, dtype=qkv_dev.dtype, device=qkv_dev.device)
    lse = torch.full((B, n_head, T), nan, dtype=torch.float32, device=qkv_dev.device)
    dqkv = torch.full_like(qkv_dev, nan)
    ws = torch.full((max(1, binding.workspace_floats(B, T, n_head)),), nan, dtype=torch.float32,
                    device=qkv_dev.device)
    binding.attn_fwd(qkv_dev, out, lse, n_head)  # bf16 or float32 by the tensors' dtype
    binding.attn_bwd(dout_dev, qkv_dev, out, lse, dqkv, ws, n_head)
    torch.cuda.synchronize()
    return out, lse, dqkv


def sample_heads(B: int, H: int, n: int, seed: int = 0):
    """n distinct (b, h) pairs including the first and the last head."""
    all_heads = [(b, h) for b in range(B) for h in range(H)]
    if n >= len(all_heads):
        return all_heads
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(len(all_heads), size=n - 2, replace=False).tolist())
    pick |= {0, len(all_heads) - 1}
    return [all_heads[i] for i in sorted(pick)]


def head_slices(x: np.ndarray, heads, n_head: int, head_dim: int, which: str):
    """Concatenate the per-head slices of a packed array for the given heads.

    which: 'out' for (B, T, C) arrays, 'q'/'k'/'v' for blocks of (B, T, 3C),
    'lse' for (B, H, T)."""
    C = n_head * head_dim
    parts = []
    for b, h in heads:
        lo = h * head_dim
        if which == "lse":
            parts.append(x[b, h, :])
        elif which == "out":
            parts.append(x[b, :, lo:lo + head_dim])
        else:
            off = {"q": 0, "k": C, "v": 2 * C}[which]
            parts.append(x[b, :, off + lo:off + lo + head_dim])
    return np.concatenate([p.ravel() for p in parts])


def compare(gpu: dict, ref: dict, heads, n_head: int, head_dim: int = 64) -> dict:
    """Error metrics of GPU results against the oracle over the given heads."""
    m = {}
    for key, which in (("o", "out"), ("lse", "lse")):
        src = "out" if key == "o" else "lse"
        g = head_slices(gpu[src], heads, n_head, head_dim, which)
        r = head_slices(ref[src], heads, n_head, head_dim, which)
        m[f"{key}_maxabs"] = float(np.max(np.abs(g - r))) if g.size else 0.0
        m[f"{key}_refmax"] = float(np.max(np.abs(r))) if r.size else 0.0
    for key in ("q", "k", "v"):
        g = head_slices(gpu["dqkv"], heads, n_head, head_dim, key)
        r = head_slices(ref["dqkv"], heads, n_head, head_dim, key)
        m[f"d{key}_maxabs"] = float(np.max(np.abs(g - r))) if g.size else 0.0
        m[f"d{key}_refmax"] = float(np.max(np.abs(r))) if r.size else 0.0
        nr = float(np.linalg.norm(r))
        m[f"d{key}_rel_l2"] = float(np.linalg.norm(g - r)) / nr if nr > 0 else float(np.linalg.norm(g))
    return m


def bf16_o_bound(o_refmax: float) -> float:
    """O bar for bf16 stress inputs whose outputs exceed the unit scale of the
    workloads: a near one-hot softmax makes O one V row, whose error is then
    its output rounding (<= |O| 2^-9) plus the rounding of the dominant bf16
    weight (<= |O| 2^-9), so 2^-7 |O|max leaves a factor 2 of headroom. It
    never drops below the workloads' 1e-2."""
    return max(BF16_O_MAXABS, o_refmax * 2.0 ** -7)


def parity_bars(m: dict, dtype: str, o_bound: float = BF16_O_MAXABS,
                f32_flat: bool = False) -> dict:
    """The bar each metric of `m` is held to: bf16 max-abs on O and LSE and
    relative L2 on the gradients; float32 max-abs on every tensor, flat 1e-5
    when f32_flat (the tiny workload) and otherwise 1e-5 times the largest
    reference magnitude (at least 1)."""
    if dtype == "bf16":
        return {"o_maxabs": o_bound, "lse_maxabs": BF16_LSE_MAXABS,
                "dq_rel_l2": BF16_GRAD_REL_L2, "dk_rel_l2": BF16_GRAD_REL_L2,
                "dv_rel_l2": BF16_GRAD_REL_L2}
    return {f"{k}_maxabs": F32_MAXABS * (1.0 if f32_flat else max(1.0, m[f"{k}_refmax"]))
            for k in ("o", "lse", "dq", "dk", "dv")}


def assert_parity(m: dict, dtype: str, label: str, o_bound: float = BF16_O_MAXABS,
                  f32_flat: bool = False) -> None:
    bars = parity_bars(m, dtype, o_bound, f32_flat)
    PARITY_RECORDS.append((label, dtype, dict(m), bars))
    log(f"[parity] {label}: " + ", ".join(f"{k}={v:.3e}" for k, v in sorted(m.items())))
    for k, bound in bars.items():
        assert m[k] <= bound, (label, k, m[k], bound, m)
