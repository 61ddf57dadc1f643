"""The C-ABI library on a machine without a GPU: it loads, exports every
declared symbol, and rejects bad arguments before any HIP call."""

import ctypes
import os
import re

import pytest

from causal_flash_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "causal_attn.h")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# Fake device addresses are passed below only to calls whose validation must
# fail before any launch; never run them where a GPU could execute a kernel.
no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="uses fake device addresses")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("library not built")
    return binding.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:long\s+long|\w+)\**\s+\**(attn_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("attn_fwd", "attn_bwd", "attn_fwd_f32", "attn_bwd_f32", "attn_bwd_preprocess",
              "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_dq_preprocess", "attn_bwd_workspace_floats",
              "attn_bwd_noalloc", "attn_bwd_noalloc_max_floats",
              "attn_fwd_unfused", "attn_bwd_unfused", "attn_unfused_workspace_bytes",
              "attn_decode", "attn_decode_workspace_floats",
              "attn_fp8_buffer_bytes", "attn_quantize_fp8", "attn_fwd_fp8",
              "attn_block_fwd", "attn_block_bwd", "attn_block_workspace_bytes",
              "attn_fp8_bwd_buffer_bytes", "attn_quantize_bwd_fp8", "attn_bwd_fp8",
              "attn_peak_mfma_flops", "attn_peak_mfma", "attn_peak_copy", "attn_peak_read",
              "attn_peak_read_slots",
              "attn_status_string", "attn_last_error", "attn_version"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(binding.SIGNATURES)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, name in binding.STATUS_NAMES.items():
        assert L.attn_status_string(code).decode() == name
    assert L.attn_status_string(12345).decode() == "ATTN_ERR_UNKNOWN"
    assert L.attn_version() == 10000


Q, O, LS, G, DQ, DL = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000, 0x60000000


@no_gpu_only
@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_f32"])
def test_forward_validation(L, fn):
    f = getattr(L, fn)
    ok = (1, 64, 2, 64)
    assert f(None, O, LS, *ok, None) == -1
    assert f(Q, None, LS, *ok, None) == -1
    assert f(Q, O, None, *ok, None) == -1
    assert f(Q, O, LS, -1, 64, 2, 64, None) == -2
    assert f(Q, O, LS, 1, -5, 2, 64, None) == -2
    assert f(Q, O, LS, 1, 64, -2, 64, None) == -2
    assert f(Q, O, LS, 1, 64, 2, 0, None) == -2
    assert f(Q, O, LS, 1, 64, 2, 128, None) == -3
    assert f(Q, O, LS, 1, 64, 2, 32, None) == -3
    assert f(Q, O, LS, 2**31 - 1, 2**31 - 1, 2**20, 64, None) == -4
    assert f(Q, O, LS, 1, 2**31 - 1, 2**20, 64, None) == -4
    assert f(Q, O, LS, 1, 64, 2**17 + 1, 64, None) == -4   # n_head*head_dim > 2^23
    assert f(Q + 8, O, LS, *ok, None) == -5
    assert f(Q, O + 4, LS, *ok, None) == -5
    assert f(Q, O, LS + 2, *ok, None) == -5
    assert f(Q, Q + 16, LS, *ok, None) == -6   # out inside qkv
    assert f(Q, O, O + 16, *ok, None) == -6     # lse inside out
    assert f(Q, O, Q - 4, *ok, None) == -6      # lse runs into qkv
    assert "overlaps" in L.attn_last_error().decode()


@no_gpu_only
@pytest.mark.parametrize("fn", ["attn_bwd", "attn_bwd_f32"])
def test_backward_validation(L, fn):
    f = getattr(L, fn)
    ok = (1, 64, 2, 64)
    args = [G, Q, O, LS, DQ, DL]
    for i in range(6):
        a = list(args)
        a[i] = None
        assert f(*a, *ok, None) == -1, i
    assert f(*args, 1, 64, 2, 63, None) == -3
    assert f(*args, 0 - 1, 64, 2, 64, None) == -2
    assert f(G + 4, Q, O, LS, DQ, DL, *ok, None) == -5
    assert f(G, Q, O, LS, DQ + 2, DL, *ok, None) == -5
    assert f(G, Q, O, LS, Q, DL, *ok, None) == -6      # dqkv aliases qkv
    assert f(G, Q, O, LS, DQ, LS, *ok, None) == -6     # delta aliases lse
    assert f(G, Q, O, LS, DQ, DQ + 64, *ok, None) == -6  # delta inside dqkv


@no_gpu_only
def test_stage_validation(L):
    ok = (1, 64, 2, 64)
    assert L.attn_bwd_preprocess(G, O, LS, None, *ok, None) == -1
    assert L.attn_bwd_preprocess(G, O, None, DL, *ok, None) == -1
    assert L.attn_bwd_preprocess(G, O, LS, O, *ok, None) == -6      # workspace is out
    assert L.attn_bwd_preprocess(G, O, LS, DL + 4, *ok, None) == -5  # workspace misaligned
    assert L.attn_bwd_dkdv(G, Q, DL, None, *ok, None) == -1
    assert L.attn_bwd_dkdv(G, Q, DL, DQ, 1, 64, 2, 16, None) == -3
    assert L.attn_bwd_dq(G, Q, DL, Q, *ok, None) == -6
    assert L.attn_bwd_dq(G, Q, DQ + 32, DQ, *ok, None) == -6  # workspace read inside dqkv
    assert L.attn_bwd_dq_preprocess(G, Q, O, LS, DQ, None, *ok, None) == -1
    assert L.attn_bwd_dq_preprocess(G, Q, None, LS, DQ, DL, *ok, None) == -1   # needs out
    assert L.attn_bwd_dq_preprocess(G, Q, O, LS, DQ, DQ + 64, *ok, None) == -6  # delta in dqkv
    assert L.attn_bwd_dq_preprocess(G, Q, O, LS, DQ, DL + 4, *ok, None) == -5


@no_gpu_only
def test_unfused_validation(L):
    ok = (1, 64, 2, 64)
    P, W = 0x70000000, 0x80000000
    f, g = L.attn_fwd_unfused, L.attn_bwd_unfused
    assert f(Q, O, LS, P, None, *ok, None) == -1
    assert f(Q, O, LS, None, W, *ok, None) == -1
    assert f(Q, O, LS, P, W, 1, 4097, 2, 64, None) == -3       # T above 4096
    assert f(Q, O, LS, P, W, 300, 64, 300, 64, None) == -4     # B * n_head above 65535
    assert f(Q, O, LS, P, W, 1, 64, 2, 32, None) == -3
    assert f(Q, O, LS, P + 8, W, *ok, None) == -5
    assert f(Q, O, LS, Q + 64, W, *ok, None) == -6             # probs inside qkv
    assert f(Q, O, LS, P, P + 64, *ok, None) == -6             # ws inside probs
    assert g(G, Q, P, DQ, None, *ok, None) == -1
    assert g(G, Q, P, DQ, W + 4, *ok, None) == -5
    assert g(G, Q, P, P + 32, W, *ok, None) == -6              # dqkv overlaps probs
    assert g(G, Q, P, DQ, W, 1, 5000, 1, 64, None) == -3
    for fn in (f, g):
        assert fn(None, None, None, None, None, 0, 64, 2, 64, None) == 0


def test_unfused_workspace_size(L):
    assert L.attn_unfused_workspace_bytes(16, 1024, 12) == 6 * 16 * 12 * 1024 * 1024
    assert L.attn_unfused_workspace_bytes(1, 1, 1) == 6 * 8         # rows padded to 8
    assert L.attn_unfused_workspace_bytes(2, 13, 3) == 6 * 2 * 3 * 13 * 16
    assert L.attn_unfused_workspace_bytes(-1, 1, 1) == -1


@no_gpu_only
def test_decode_validation(L):
    f = L.attn_decode
    K, V, W = 0x70000000, 0x80000000, 0x90000000
    C = 128                                   # n_head 2, head_dim 64
    assert f(None, C, K, V, 3 * C, 64 * 3 * C, O, LS, W, 1, 64, 2, 64, None) == -1
    assert f(Q, C, K, V, 3 * C, 64 * 3 * C, O, LS, None, 1, 64, 2, 64, None) == -1
    assert f(Q, C, K, V, 3 * C, 64 * 3 * C, O, LS, W, 1, 64, 2, 32, None) == -3
    assert f(Q, C, K, V, 3 * C, 64 * 3 * C, O, LS, W, 300, 64, 300, 64, None) == -4
    assert f(Q, C - 8, K, V, 3 * C, 64 * 3 * C, O, LS, W, 2, 64, 2, 64, None) == -2   # q stride < C
    assert f(Q, C, K, V, C - 8, 64 * 3 * C, O, LS, W, 2, 64, 2, 64, None) == -2       # row stride < C
    assert f(Q, C, K, V, 3 * C, 3 * C, O, LS, W, 2, 64, 2, 64, None) == -2            # batch rows overlap
    assert f(Q, C, K, V, 3 * C + 4, 64 * 3 * C, O, LS, W, 1, 64, 2, 64, None) == -5   # stride not 8k
    assert f(Q + 8, C, K, V, 3 * C, 64 * 3 * C, O, LS, W, 1, 64, 2, 64, None) == -5
    assert f(Q, C, K, V, 3 * C, 64 * 3 * C, K + 64, LS, W, 1, 64, 2, 64, None) == -6  # out in cache
    assert f(Q, C, K, V, 3 * C, 64 * 3 * C, O, LS, O, 1, 64, 2, 64, None) == -6       # ws is out
    assert f(None, C, None, None, 3 * C, 0, None, None, None, 0, 64, 2, 64, None) == 0


def test_decode_workspace_size(L):
    assert L.attn_decode_workspace_floats(16, 1024, 12) > 0
    assert L.attn_decode_workspace_floats(1, 1, 1) == 66            # one split: m, l, 64 sums
    assert L.attn_decode_workspace_floats(0, 5, 2) == 0
    assert L.attn_decode_workspace_floats(1, -1, 2) == -1


@no_gpu_only
def test_fp8_validation(L):
    F8 = 0x70000000
    fq, ff = L.attn_quantize_fp8, L.attn_fwd_fp8
    ok = (1, 64, 2, 64)
    assert fq(Q, None, *ok, None) == -1
    assert fq(None, F8, *ok, None) == -1
    assert fq(Q, F8, 1, 64, 2, 32, None) == -3                 # head_dim 32
    assert fq(Q, F8 + 8, *ok, None) == -5
    assert fq(Q, Q + 64, *ok, None) == -6                      # buffer inside qkv
    assert fq(Q, F8, 1, 67108801, 1, 64, None) == -4           # round_up(T, 64) * 64 = 2^32
    assert ff(None, O, LS, *ok, None) == -1
    assert ff(F8, O, None, *ok, None) == -1
    assert ff(F8, O + 8, LS, *ok, None) == -5
    assert ff(F8, O, LS + 2, *ok, None) == -5
    assert ff(F8, F8 + 128, LS, *ok, None) == -6               # out inside the buffer
    assert ff(F8, O, O, *ok, None) == -6                       # lse is out
    assert ff(F8, O, LS, 1, 64, 2, 32, None) == -3
    for fn in (fq,):
        assert fn(None, None, 0, 64, 2, 64, None) == 0
    assert ff(None, None, None, 1, 0, 2, 64, None) == 0


@no_gpu_only
def test_block_validation(L):
    X, WA, BA, WP, BP = 0x70000000, 0x71000000, 0x72000000, 0x73000000, 0x74000000
    QK, AT, LSE, Y = 0x80000000, 0x81000000, 0x82000000, 0x83000000
    f = L.attn_block_fwd
    ok = (2, 64, 2, 64)
    assert f(X, WA, BA, WP, BP, QK, AT, LSE, None, *ok, None) == -1
    assert f(X, WA, BA, WP, BP, QK, AT, LSE, Y, 2, 64, 2, 32, None) == -3
    assert f(X + 8, WA, BA, WP, BP, QK, AT, LSE, Y, *ok, None) == -5
    assert f(X, WA, BA + 1, WP, BP, QK, AT, LSE, Y, *ok, None) == -5
    assert f(X, WA, BA, WP, BP, X + 64, AT, LSE, Y, *ok, None) == -6     # qkv inside x
    assert f(X, WA, BA, WP, BP, QK, AT, LSE, QK + 128, *ok, None) == -6  # y inside qkv
    assert f(X, WA, BA, WP, BP, QK, AT, LSE, Y, 65536, 256, 1, 64, None) == -4  # B*T too large
    assert f(None, None, None, None, None, None, None, None, None, 0, 64, 2, 64, None) == 0
    g = L.attn_block_bwd
    D8 = [0x90000000 + i * 0x1000000 for i in range(8)]       # datt .. ws
    args = [0x60000000, X, WA, WP, QK, AT, LSE] + D8
    assert g(*args, *ok, None) != -1
    bad = list(args)
    bad[14] = None                                            # ws
    assert g(*bad, *ok, None) == -1
    bad = list(args)
    bad[7] = D8[0] + 8                                        # datt misaligned
    assert g(*bad, *ok, None) == -5
    bad = list(args)
    bad[9] = args[0] + 64                                     # dx inside dy
    assert g(*bad, *ok, None) == -6
    bad = list(args)
    bad[11] = D8[3] + 8                                       # db_attn inside dw_attn
    assert g(*bad, *ok, None) == -6


def test_block_workspace_size(L):
    # delta (10 floats per padded row) plus the largest of the K-split
    # partials of dW_attn and dW_proj and the column-sum partials
    n = L.attn_block_workspace_bytes(16, 1024, 12)
    assert n >= 4 * (10 * 16 * 12 * 1024 + 768 * 2304)
    assert n % 4 == 0
    assert L.attn_block_workspace_bytes(1, 1, 1) >= 4 * (10 * 64 + 64 * 192)
    assert L.attn_block_workspace_bytes(0, 5, 2) == 0
    assert L.attn_block_workspace_bytes(1, -1, 2) == -1


@no_gpu_only
def test_fp8_bwd_validation(L):
    F8, B8 = 0x70000000, 0x78000000
    fq, fb = L.attn_quantize_bwd_fp8, L.attn_bwd_fp8
    ok = (1, 64, 2, 64)
    assert fq(G, Q, O, LS, None, *ok, None) == -1
    assert fq(G, Q, O, LS, B8 + 8, *ok, None) == -5
    assert fq(G, Q, O, LS + 1, B8, *ok, None) == -5
    assert fq(G, Q, O, LS, Q + 64, *ok, None) == -6            # buffer inside qkv
    assert fq(G, Q, O, LS, B8, 1, 64, 2, 32, None) == -3
    assert fb(F8, B8, None, *ok, None) == -1
    assert fb(F8, B8, DQ + 8, *ok, None) == -5
    assert fb(F8, B8, B8 + 256, *ok, None) == -6               # dqkv inside the buffer
    assert fb(F8, B8, DQ, 1, 67108801, 1, 64, None) == -4
    assert fq(None, None, None, None, None, 0, 64, 2, 64, None) == 0
    assert fb(None, None, None, 1, 0, 2, 64, None) == 0


def test_fp8_bwd_buffer_size(L):
    # 320 code bytes per (head, padded position) plus 1152 side bytes per tile
    assert L.attn_fp8_bwd_buffer_bytes(1, 64, 1) == 320 * 64 + 1152
    assert L.attn_fp8_bwd_buffer_bytes(2, 65, 3) == 6 * (320 * 128 + 2 * 1152)
    assert L.attn_fp8_bwd_buffer_bytes(0, 5, 2) == 0
    assert L.attn_fp8_bwd_buffer_bytes(1, -1, 2) == -1


def test_fp8_buffer_size(L):
    # 192 code bytes per (head, padded position) plus 384 exponent bytes per
    # tile of 64 positions
    assert L.attn_fp8_buffer_bytes(1, 64, 1) == 192 * 64 + 384
    assert L.attn_fp8_buffer_bytes(1, 65, 2) == 2 * (192 * 128 + 2 * 384)
    assert L.attn_fp8_buffer_bytes(16, 1024, 12) == 16 * 12 * (192 * 1024 + 16 * 384)
    assert L.attn_fp8_buffer_bytes(0, 5, 2) == 0
    assert L.attn_fp8_buffer_bytes(1, -1, 2) == -1


def test_workspace_size(L):
    assert L.attn_bwd_workspace_floats(1, 64, 2) == 10 * 2 * 64
    assert L.attn_bwd_workspace_floats(1, 65, 2) == 10 * 2 * 128
    assert L.attn_bwd_workspace_floats(16, 1024, 12) == 10 * 16 * 12 * 1024
    assert L.attn_bwd_workspace_floats(3, 1, 5) == 10 * 3 * 5 * 64
    assert L.attn_bwd_workspace_floats(0, 10, 2) == 0
    assert L.attn_bwd_workspace_floats(-1, 10, 2) == -1


@no_gpu_only
def test_noalloc_validation(L):
    # Everything below is rejected before the library looks for its
    # workspace array on a device.
    assert L.attn_bwd_noalloc_max_floats() == 8 << 20
    assert L.attn_bwd_noalloc(None, None, None, None, None, 0, 64, 2, 64, None) == 0
    assert L.attn_bwd_noalloc(G, Q, O, LS, None, 1, 64, 2, 64, None) == -1
    assert L.attn_bwd_noalloc(G, Q, O, LS, DQ, 1, 64, 2, 32, None) == -3
    assert L.attn_bwd_noalloc(G, Q, O, LS, DQ, -1, 64, 2, 64, None) == -2
    # 10 * 64 * 12 * round_up(T, 64) floats: T = 1088 fits, T = 1089 does not.
    assert L.attn_bwd_workspace_floats(64, 1088, 12) <= L.attn_bwd_noalloc_max_floats()
    assert L.attn_bwd_workspace_floats(64, 1089, 12) > L.attn_bwd_noalloc_max_floats()
    assert L.attn_bwd_noalloc(G, Q, O, LS, DQ, 64, 1089, 12, 64, None) == -4
    assert "attn_bwd_noalloc_max_floats" in L.attn_last_error().decode()


def test_empty_problems_are_noops(L):
    for B, T, H in ((0, 64, 2), (1, 0, 2), (1, 64, 0)):
        assert L.attn_fwd(None, None, None, B, T, H, 64, None) == 0
        assert L.attn_fwd_f32(None, None, None, B, T, H, 64, None) == 0
        assert L.attn_bwd(None, None, None, None, None, None, B, T, H, 64, None) == 0
        assert L.attn_bwd_f32(None, None, None, None, None, None, B, T, H, 64, None) == 0
        assert L.attn_bwd_dkdv(None, None, None, None, B, T, H, 64, None) == 0
        assert L.attn_bwd_preprocess(None, None, None, None, B, T, H, 64, None) == 0
        assert L.attn_bwd_dq_preprocess(None, None, None, None, None, None, B, T, H, 64, None) == 0


@no_gpu_only
def test_launch_without_device_reports_hip_error(L):
    # Valid arguments on a machine with no GPU: the launch itself fails and
    # the call reports it instead of crashing.
    assert L.attn_fwd(Q, O, LS, 1, 64, 2, 64, None) == -7
    assert "attn_fwd" in L.attn_last_error().decode()
    assert L.attn_bwd(G, Q, O, LS, DQ, DL, 1, 64, 2, 64, None) == -7


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()


def test_binding_argument_checks_on_cpu_tensors():
    torch = pytest.importorskip("torch")
    qkv = torch.zeros(1, 4, 3 * 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        binding.attn_fwd(qkv, torch.zeros(1, 4, 64, dtype=torch.bfloat16),
                         torch.zeros(1, 1, 4), n_head=1)
    with pytest.raises(ValueError):
        binding.forward(torch.zeros(1, 4, 100, dtype=torch.bfloat16), n_head=1)
    with pytest.raises(ValueError):
        binding.forward(torch.zeros(1, 4, 192, dtype=torch.float16), n_head=1)


def test_peak_mfma_flops(L):
    # 4 waves x iters x 8 MFMAs x (32 x 32 x 16 x 2) FLOPs per workgroup
    assert L.attn_peak_mfma_flops(1, 1) == 4 * 8 * 32768
    assert L.attn_peak_mfma_flops(2048, 4096) == 2048 * 4 * 4096 * 8 * 32768
    for bad in ((0, 1), (1, 0), (-1, 5), (2**20 + 1, 1), (1, 2**20 + 1)):
        assert L.attn_peak_mfma_flops(*bad) == -1, bad


@no_gpu_only
def test_peak_probe_validation(L):
    assert L.attn_peak_mfma(None, DL, 4, 4, None) == -1
    assert L.attn_peak_mfma(O, None, 4, 4, None) == -1
    assert L.attn_peak_mfma(O, DL, 0, 4, None) == -2
    assert L.attn_peak_mfma(O, DL, 4, 2**20 + 1, None) == -2
    assert L.attn_peak_mfma(O + 2, DL, 4, 4, None) == -5
    assert L.attn_peak_mfma(O, DL + 4, 4, 4, None) == -5
    assert L.attn_peak_mfma(O, O + 1024, 4, 4, None) == -6   # ticks inside out
    assert L.attn_peak_copy(Q, O, 0, None) == 0                # nothing to copy
    assert L.attn_peak_copy(None, O, 64, None) == -1
    assert L.attn_peak_copy(Q, O, 24, None) == -2              # not a multiple of 16
    assert L.attn_peak_copy(Q, O, -16, None) == -2
    assert L.attn_peak_copy(Q + 8, O, 64, None) == -5
    assert L.attn_peak_copy(Q, Q + 32, 64, None) == -6         # dst overlaps src
    assert L.attn_peak_read_slots() == 8192
    assert L.attn_peak_read(Q, 0, None, None) == 0              # nothing to read
    assert L.attn_peak_read(None, 64, O, None) == -1
    assert L.attn_peak_read(Q, 64, None, None) == -1
    assert L.attn_peak_read(Q, 40, O, None) == -2
    assert L.attn_peak_read(Q + 4, 64, O, None) == -5
    assert L.attn_peak_read(Q, 64, O + 2, None) == -5
    assert L.attn_peak_read(Q, 1 << 20, Q + 64, None) == -6     # out inside src


def test_documented_status_codes_and_workspace_formula(L):
    """The numbering and the backward workspace size that the header and the
    design notes document (boundary reading b1)."""
    codes = {0: "ATTN_OK", -1: "ATTN_ERR_NULL_PTR", -2: "ATTN_ERR_BAD_SHAPE",
             -3: "ATTN_ERR_UNSUPPORTED", -4: "ATTN_ERR_TOO_LARGE", -5: "ATTN_ERR_MISALIGNED",
             -6: "ATTN_ERR_ALIAS", -7: "ATTN_ERR_HIP"}
    header = open(os.path.join(ROOT, "include", "causal_attn.h")).read()
    for code, name in codes.items():
        assert re.search(rf"\b{name}\s*=\s*{code}\b", header), name
        assert L.attn_status_string(code).decode() == name
    for B, T, H in [(1, 1, 1), (16, 1024, 12), (3, 700, 5), (2, 64, 2), (4, 2049, 25)]:
        assert L.attn_bwd_workspace_floats(B, T, H) == 10 * B * H * ((T + 63) // 64 * 64)
