"""Python binding of libcausal_attn.so (ctypes, argument marshalling only).

The functions named like the C ABI (``attn_fwd``, ``attn_bwd``, ...) take
torch tensors that already live on the GPU, check dtype / shape / device /
contiguity, pass raw pointers and the current HIP stream to the library and
raise :class:`AttnError` on a non-zero status. Every step of the computation
runs in the library's HIP kernels; there is no fallback. ``forward`` and
``backward`` additionally allocate their outputs with torch.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import threading
from typing import Optional, Tuple

from ._paths import LIB_PATH

ATTN_OK = 0
STATUS_NAMES = {
    0: "ATTN_OK",
    -1: "ATTN_ERR_NULL_PTR",
    -2: "ATTN_ERR_BAD_SHAPE",
    -3: "ATTN_ERR_UNSUPPORTED",
    -4: "ATTN_ERR_TOO_LARGE",
    -5: "ATTN_ERR_MISALIGNED",
    -6: "ATTN_ERR_ALIAS",
    -7: "ATTN_ERR_HIP",
}

# Every symbol include/causal_attn.h declares, with its ctypes signature.
_P = ctypes.c_void_p
_I = ctypes.c_int
SIGNATURES = {
    "attn_fwd": ([_P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_bwd": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_bwd_preprocess": ([_P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_bwd_dq_preprocess": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_bwd_dkdv": ([_P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_bwd_dq": ([_P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_bwd_workspace_floats": ([_I, _I, _I], ctypes.c_longlong),
    "attn_bwd_noalloc": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_bwd_noalloc_max_floats": ([], ctypes.c_longlong),
    "attn_unfused_workspace_bytes": ([_I, _I, _I], ctypes.c_longlong),
    "attn_fwd_unfused": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_decode_workspace_floats": ([_I, _I, _I], ctypes.c_longlong),
    "attn_decode": ([_P, ctypes.c_longlong, _P, _P, ctypes.c_longlong, ctypes.c_longlong,
                     _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_bwd_unfused": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_block_workspace_bytes": ([_I, _I, _I], ctypes.c_longlong),
    "attn_block_fwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_block_bwd": ([_P] * 15 + [_I, _I, _I, _I, _P], _I),
    "attn_fp8_buffer_bytes": ([_I, _I, _I], ctypes.c_longlong),
    "attn_fp8_bwd_buffer_bytes": ([_I, _I, _I], ctypes.c_longlong),
    "attn_quantize_bwd_fp8": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_bwd_fp8": ([_P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_quantize_fp8": ([_P, _P, _I, _I, _I, _I, _P], _I),
    "attn_fwd_fp8": ([_P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_fwd_f32": ([_P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_bwd_f32": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "attn_peak_mfma_flops": ([_I, _I], ctypes.c_longlong),
    "attn_peak_mfma": ([_P, _P, _I, _I, _P], _I),
    "attn_peak_copy": ([_P, _P, ctypes.c_longlong, _P], _I),
    "attn_peak_read_slots": ([], _I),
    "attn_peak_read": ([_P, ctypes.c_longlong, _P, _P], _I),
    "attn_status_string": ([_I], ctypes.c_char_p),
    "attn_last_error": ([], ctypes.c_char_p),
    "attn_version": ([], _I),
}

_lib = None
_lock = threading.Lock()


class AttnError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str = ""):
        self.status = status
        name = STATUS_NAMES.get(status, f"status {status}")
        super().__init__(f"{func}: {name}" + (f" ({detail})" if detail else ""))


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m causal_flash_attention_amd.build` (hipcc, gfx950)")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.argtypes = args
                fn.restype = res
            _lib = handle
    return _lib


def _check(status: int, func: str) -> None:
    if status != ATTN_OK:
        detail = lib().attn_last_error().decode(errors="replace")
        raise AttnError(status, func, detail)


def _torch():
    import torch
    return torch


def _stream_ptr(stream) -> Optional[int]:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t) -> int:
    return t.data_ptr() if t is not None else 0


def _require(t, name: str, dtype, shape) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dims(qkv, n_head: int, head_dim: int) -> Tuple[int, int, int]:
    if qkv.dim() != 3 or qkv.shape[2] != 3 * n_head * head_dim:
        raise ValueError("qkv must be (B, T, 3 * n_head * head_dim)")
    return int(qkv.shape[0]), int(qkv.shape[1]), n_head * head_dim


def _elem(qkv):
    torch = _torch()
    if qkv.dtype == torch.bfloat16:
        return torch.bfloat16, ""
    if qkv.dtype == torch.float32:
        return torch.float32, "_f32"
    raise ValueError("qkv must be bfloat16 or float32")


# ---------------------------------------------------------------------------
# Same-named wrappers of the C entry points.
# ---------------------------------------------------------------------------

def attn_fwd(qkv, out, lse, n_head: int, head_dim: int = 64, stream=None) -> None:
    torch = _torch()
    dt, sfx = _elem(qkv)
    B, T, C = _dims(qkv, n_head, head_dim)
    _require(qkv, "qkv", dt, (B, T, 3 * C))
    _require(out, "out", dt, (B, T, C))
    _require(lse, "lse", torch.float32, (B, n_head, T))
    fn = getattr(lib(), "attn_fwd" + sfx)
    _check(fn(_ptr(qkv), _ptr(out), _ptr(lse), B, T, n_head, head_dim, _stream_ptr(stream)),
           "attn_fwd" + sfx)


def workspace_floats(B: int, T: int, n_head: int) -> int:
    """Floats the backward workspace must hold: 10 * B * n_head * round_up(T, 64)."""
    n = int(lib().attn_bwd_workspace_floats(B, T, n_head))
    if n < 0:
        raise ValueError("B, T and n_head must be non-negative")
    return n


def _require_ws(delta, B, T, n_head):
    torch = _torch()
    if delta is None or not delta.is_cuda or delta.dtype != torch.float32:
        raise ValueError("delta must be a float32 GPU tensor")
    if not delta.is_contiguous() or delta.numel() < workspace_floats(B, T, n_head):
        raise ValueError("delta must be contiguous with at least "
                         f"{workspace_floats(B, T, n_head)} floats")


def attn_bwd(dout, qkv, out, lse, dqkv, delta, n_head: int, head_dim: int = 64,
             stream=None) -> None:
    _bwd_full("attn_bwd", dout, qkv, out, lse, dqkv, delta, n_head, head_dim, stream)


def attn_bwd_noalloc(dout, qkv, out, lse, dqkv, n_head: int, head_dim: int = 64,
                     stream=None) -> None:
    """attn_bwd with the library's own per-GPU workspace (no allocation)."""
    torch = _torch()
    if qkv is None or qkv.dtype != torch.bfloat16:
        raise ValueError("attn_bwd_noalloc takes bfloat16 tensors")
    B, T, C = _dims(qkv, n_head, head_dim)
    for t, name, shape in ((dout, "dout", (B, T, C)), (qkv, "qkv", (B, T, 3 * C)),
                           (out, "out", (B, T, C)), (dqkv, "dqkv", (B, T, 3 * C))):
        _require(t, name, torch.bfloat16, shape)
    _require(lse, "lse", torch.float32, (B, n_head, T))
    _check(lib().attn_bwd_noalloc(_ptr(dout), _ptr(qkv), _ptr(out), _ptr(lse), _ptr(dqkv),
                                  B, T, n_head, head_dim, _stream_ptr(stream)), "attn_bwd_noalloc")


def noalloc_max_floats() -> int:
    return int(lib().attn_bwd_noalloc_max_floats())


def attn_bwd_dq_preprocess(dout, qkv, out, lse, dqkv, delta, n_head: int, head_dim: int = 64,
                           stream=None) -> None:
    if qkv is not None and qkv.dtype != _torch().bfloat16:
        raise ValueError("attn_bwd_dq_preprocess takes bfloat16 tensors")
    _bwd_full("attn_bwd_dq_preprocess", dout, qkv, out, lse, dqkv, delta, n_head, head_dim,
              stream)


def _bwd_full(name, dout, qkv, out, lse, dqkv, delta, n_head, head_dim, stream) -> None:
    torch = _torch()
    dt, sfx = _elem(qkv)
    B, T, C = _dims(qkv, n_head, head_dim)
    _require(dout, "dout", dt, (B, T, C))
    _require(qkv, "qkv", dt, (B, T, 3 * C))
    _require(out, "out", dt, (B, T, C))
    _require(lse, "lse", torch.float32, (B, n_head, T))
    _require(dqkv, "dqkv", dt, (B, T, 3 * C))
    _require_ws(delta, B, T, n_head)
    fn = getattr(lib(), name + sfx)
    _check(fn(_ptr(dout), _ptr(qkv), _ptr(out), _ptr(lse), _ptr(dqkv), _ptr(delta),
              B, T, n_head, head_dim, _stream_ptr(stream)), name + sfx)


def attn_bwd_preprocess(dout, out, lse, delta, n_head: int, head_dim: int = 64,
                        stream=None) -> None:
    torch = _torch()
    B, T, C = int(out.shape[0]), int(out.shape[1]), n_head * head_dim
    _require(out, "out", torch.bfloat16, (B, T, C))
    _require(dout, "dout", torch.bfloat16, (B, T, C))
    _require(lse, "lse", torch.float32, (B, n_head, T))
    _require_ws(delta, B, T, n_head)
    _check(lib().attn_bwd_preprocess(_ptr(dout), _ptr(out), _ptr(lse), _ptr(delta), B, T, n_head,
                                     head_dim, _stream_ptr(stream)), "attn_bwd_preprocess")


def _bwd_stage(name, dout, qkv, delta, dqkv, n_head, head_dim, stream):
    torch = _torch()
    B, T, C = _dims(qkv, n_head, head_dim)
    _require(qkv, "qkv", torch.bfloat16, (B, T, 3 * C))
    _require(dout, "dout", torch.bfloat16, (B, T, C))
    _require(dqkv, "dqkv", torch.bfloat16, (B, T, 3 * C))
    _require_ws(delta, B, T, n_head)
    _check(getattr(lib(), name)(_ptr(dout), _ptr(qkv), _ptr(delta), _ptr(dqkv),
                                B, T, n_head, head_dim, _stream_ptr(stream)), name)


def attn_bwd_dkdv(dout, qkv, delta, dqkv, n_head: int, head_dim: int = 64, stream=None) -> None:
    _bwd_stage("attn_bwd_dkdv", dout, qkv, delta, dqkv, n_head, head_dim, stream)


def attn_bwd_dq(dout, qkv, delta, dqkv, n_head: int, head_dim: int = 64, stream=None) -> None:
    _bwd_stage("attn_bwd_dq", dout, qkv, delta, dqkv, n_head, head_dim, stream)


def unfused_row_stride(T: int) -> int:
    """Row length of the materialising path's T x T matrices: round_up(T, 8)."""
    return (T + 7) // 8 * 8


def unfused_workspace_bytes(B: int, T: int, n_head: int) -> int:
    """Bytes of the materialising path's workspace: 6 * B * n_head * T * round_up(T, 8)."""
    n = int(lib().attn_unfused_workspace_bytes(B, T, n_head))
    if n < 0:
        raise ValueError("B, T and n_head must be non-negative")
    return n


def _require_bytes(t, name: str, nbytes: int) -> None:
    if t is None or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} must hold at least {nbytes} bytes")


def attn_fwd_unfused(qkv, out, lse, probs, ws, n_head: int, head_dim: int = 64,
                     stream=None) -> None:
    torch = _torch()
    B, T, C = _dims(qkv, n_head, head_dim)
    _require(qkv, "qkv", torch.bfloat16, (B, T, 3 * C))
    _require(out, "out", torch.bfloat16, (B, T, C))
    _require(lse, "lse", torch.float32, (B, n_head, T))
    _require(probs, "probs", torch.bfloat16, (B, n_head, T, unfused_row_stride(T)))
    _require_bytes(ws, "ws", unfused_workspace_bytes(B, T, n_head))
    _check(lib().attn_fwd_unfused(_ptr(qkv), _ptr(out), _ptr(lse), _ptr(probs), _ptr(ws), B, T,
                                  n_head, head_dim, _stream_ptr(stream)), "attn_fwd_unfused")


def attn_bwd_unfused(dout, qkv, probs, dqkv, ws, n_head: int, head_dim: int = 64,
                     stream=None) -> None:
    torch = _torch()
    B, T, C = _dims(qkv, n_head, head_dim)
    _require(dout, "dout", torch.bfloat16, (B, T, C))
    _require(qkv, "qkv", torch.bfloat16, (B, T, 3 * C))
    _require(probs, "probs", torch.bfloat16, (B, n_head, T, unfused_row_stride(T)))
    _require(dqkv, "dqkv", torch.bfloat16, (B, T, 3 * C))
    _require_bytes(ws, "ws", unfused_workspace_bytes(B, T, n_head))
    _check(lib().attn_bwd_unfused(_ptr(dout), _ptr(qkv), _ptr(probs), _ptr(dqkv), _ptr(ws), B, T,
                                  n_head, head_dim, _stream_ptr(stream)), "attn_bwd_unfused")


def decode_workspace_floats(B: int, T: int, n_head: int) -> int:
    """Floats of the decode workspace for this shape."""
    n = int(lib().attn_decode_workspace_floats(B, T, n_head))
    if n < 0:
        raise ValueError("B, T and n_head must be non-negative")
    return n


def attn_decode(q, k_cache, v_cache, out, lse, ws, T: int, n_head: int, head_dim: int = 64,
                stream=None) -> None:
    """q: (B, C) bf16 view with unit stride along C; k_cache, v_cache:
    (B, T_max, C) bf16 views with unit stride along C (any row and batch
    strides, e.g. slices of a packed qkv); positions 0 .. T-1 are used."""
    torch = _torch()
    C = n_head * head_dim
    for t, name, dim in ((q, "q", 2), (k_cache, "k_cache", 3), (v_cache, "v_cache", 3)):
        if t is None or not t.is_cuda or t.dtype != torch.bfloat16 or t.dim() != dim:
            raise ValueError(f"{name} must be a {dim}-D bfloat16 GPU tensor")
        if t.shape[-1] != C or t.stride(-1) != 1:
            raise ValueError(f"{name} must have a last dimension of {C} with unit stride")
    B = int(q.shape[0])
    if k_cache.shape[0] != B or v_cache.shape[0] != B:
        raise ValueError("q, k_cache and v_cache must share the batch dimension")
    if k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must have the same strides")
    if not 0 <= T <= min(k_cache.shape[1], v_cache.shape[1]):
        raise ValueError("T exceeds the cache length")
    _require(out, "out", torch.bfloat16, (B, C))
    _require(lse, "lse", torch.float32, (B, n_head))
    n = decode_workspace_floats(B, T, n_head)
    if ws is None or not ws.is_cuda or ws.dtype != torch.float32 or not ws.is_contiguous() \
            or ws.numel() < n:
        raise ValueError(f"ws must be a contiguous float32 GPU tensor of at least {n} floats")
    _check(lib().attn_decode(_ptr(q), q.stride(0), _ptr(k_cache), _ptr(v_cache),
                             k_cache.stride(1), k_cache.stride(0), _ptr(out), _ptr(lse), _ptr(ws),
                             B, T, n_head, head_dim, _stream_ptr(stream)), "attn_decode")


def block_workspace_bytes(B: int, T: int, n_head: int) -> int:
    """Bytes of attn_block_bwd's workspace."""
    n = int(lib().attn_block_workspace_bytes(B, T, n_head))
    if n < 0:
        raise ValueError("B, T and n_head must be non-negative")
    return n


def attn_block_fwd(x, w_attn, b_attn, w_proj, b_proj, qkv, att, lse, y, n_head: int,
                   head_dim: int = 64, stream=None) -> None:
    torch = _torch()
    if x is None or x.dim() != 3:
        raise ValueError("x must be a (B, T, C) tensor")
    B, T, C = (int(v) for v in x.shape)
    if C != n_head * head_dim:
        raise ValueError("x's last dimension must be n_head * head_dim")
    bf = torch.bfloat16
    for t, name, shape in ((x, "x", (B, T, C)), (w_attn, "w_attn", (C, 3 * C)),
                           (b_attn, "b_attn", (3 * C,)), (w_proj, "w_proj", (C, C)),
                           (b_proj, "b_proj", (C,)), (qkv, "qkv", (B, T, 3 * C)),
                           (att, "att", (B, T, C)), (y, "y", (B, T, C))):
        _require(t, name, bf, shape)
    _require(lse, "lse", torch.float32, (B, n_head, T))
    _check(lib().attn_block_fwd(_ptr(x), _ptr(w_attn), _ptr(b_attn), _ptr(w_proj), _ptr(b_proj),
                                _ptr(qkv), _ptr(att), _ptr(lse), _ptr(y), B, T, n_head, head_dim,
                                _stream_ptr(stream)), "attn_block_fwd")


def attn_block_bwd(dy, x, w_attn, w_proj, qkv, att, lse, datt, dqkv, dx, dw_attn, db_attn,
                   dw_proj, db_proj, ws, n_head: int, head_dim: int = 64, stream=None) -> None:
    torch = _torch()
    if x is None or x.dim() != 3:
        raise ValueError("x must be a (B, T, C) tensor")
    B, T, C = (int(v) for v in x.shape)
    if C != n_head * head_dim:
        raise ValueError("x's last dimension must be n_head * head_dim")
    bf, f32 = torch.bfloat16, torch.float32
    for t, name, dt, shape in ((dy, "dy", bf, (B, T, C)), (x, "x", bf, (B, T, C)),
                               (w_attn, "w_attn", bf, (C, 3 * C)), (w_proj, "w_proj", bf, (C, C)),
                               (qkv, "qkv", bf, (B, T, 3 * C)), (att, "att", bf, (B, T, C)),
                               (lse, "lse", f32, (B, n_head, T)), (datt, "datt", bf, (B, T, C)),
                               (dqkv, "dqkv", bf, (B, T, 3 * C)), (dx, "dx", bf, (B, T, C)),
                               (dw_attn, "dw_attn", f32, (C, 3 * C)), (db_attn, "db_attn", f32, (3 * C,)),
                               (dw_proj, "dw_proj", f32, (C, C)), (db_proj, "db_proj", f32, (C,))):
        _require(t, name, dt, shape)
    _require_bytes(ws, "ws", block_workspace_bytes(B, T, n_head))
    _check(lib().attn_block_bwd(_ptr(dy), _ptr(x), _ptr(w_attn), _ptr(w_proj), _ptr(qkv),
                                _ptr(att), _ptr(lse), _ptr(datt), _ptr(dqkv), _ptr(dx),
                                _ptr(dw_attn), _ptr(db_attn), _ptr(dw_proj), _ptr(db_proj),
                                _ptr(ws), B, T, n_head, head_dim, _stream_ptr(stream)),
           "attn_block_bwd")


def fp8_buffer_bytes(B: int, T: int, n_head: int) -> int:
    """Bytes of the FP8 buffer of attn_quantize_fp8 / attn_fwd_fp8."""
    n = int(lib().attn_fp8_buffer_bytes(B, T, n_head))
    if n < 0:
        raise ValueError("B, T and n_head must be non-negative")
    return n


def attn_quantize_fp8(qkv, fp8, n_head: int, head_dim: int = 64, stream=None) -> None:
    """qkv: packed (B, T, 3C) bf16; fp8: contiguous GPU buffer of at least
    fp8_buffer_bytes(B, T, n_head) bytes (any dtype, e.g. uint8)."""
    torch = _torch()
    B, T, C = _dims(qkv, n_head, head_dim)
    _require(qkv, "qkv", torch.bfloat16, (B, T, 3 * C))
    _require_bytes(fp8, "fp8", fp8_buffer_bytes(B, T, n_head))
    _check(lib().attn_quantize_fp8(_ptr(qkv), _ptr(fp8), B, T, n_head, head_dim,
                                   _stream_ptr(stream)), "attn_quantize_fp8")


def attn_fwd_fp8(fp8, out, lse, n_head: int, head_dim: int = 64, stream=None) -> None:
    """fp8: the buffer written by attn_quantize_fp8 for these shapes; out
    (B, T, C) bf16 and lse (B, n_head, T) float32 give B and T."""
    torch = _torch()
    if out is None or out.dim() != 3:
        raise ValueError("out must be a (B, T, C) tensor")
    B, T, C = (int(x) for x in out.shape)
    if C != n_head * head_dim:
        raise ValueError("out's last dimension must be n_head * head_dim")
    _require(out, "out", torch.bfloat16, (B, T, C))
    _require(lse, "lse", torch.float32, (B, n_head, T))
    _require_bytes(fp8, "fp8", fp8_buffer_bytes(B, T, n_head))
    _check(lib().attn_fwd_fp8(_ptr(fp8), _ptr(out), _ptr(lse), B, T, n_head, head_dim,
                              _stream_ptr(stream)), "attn_fwd_fp8")


def attn_peak_mfma_flops(n_wg: int, iters: int) -> int:
    """bf16 MFMA FLOPs of one attn_peak_mfma call with these arguments."""
    n = int(lib().attn_peak_mfma_flops(n_wg, iters))
    if n < 0:
        raise ValueError("n_wg and iters must lie in [1, 2^20]")
    return n


def attn_peak_mfma(out, ticks, n_wg: int, iters: int, stream=None) -> None:
    """MFMA peak probe: out (n_wg * 256,) float32 and ticks (2 * n_wg,) int64
    GPU tensors (see causal_attn.h)."""
    torch = _torch()
    _require(out, "out", torch.float32, (256 * n_wg,))
    _require(ticks, "ticks", torch.int64, (2 * n_wg,))
    _check(lib().attn_peak_mfma(_ptr(out), _ptr(ticks), n_wg, iters, _stream_ptr(stream)),
           "attn_peak_mfma")


def attn_peak_copy(src, dst, stream=None) -> None:
    """HBM probe: copies the contiguous GPU tensor src into dst (same size in
    bytes, a multiple of 16)."""
    if src is None or dst is None:
        raise ValueError("src and dst are required")
    if not src.is_cuda or not dst.is_cuda:
        raise ValueError("src and dst must be GPU tensors")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n or not src.is_contiguous() or not dst.is_contiguous():
        raise ValueError("src and dst must be contiguous and of the same size in bytes")
    _check(lib().attn_peak_copy(_ptr(src), _ptr(dst), n, _stream_ptr(stream)), "attn_peak_copy")


def attn_peak_read(src, out, stream=None) -> None:
    """HBM read probe: reads the contiguous GPU tensor src; out is an int32
    GPU tensor of attn_peak_read_slots() elements."""
    torch = _torch()
    if src is None or not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    _require(out, "out", torch.int32, (int(lib().attn_peak_read_slots()),))
    n = src.numel() * src.element_size()
    _check(lib().attn_peak_read(_ptr(src), n, _ptr(out), _stream_ptr(stream)), "attn_peak_read")


def attn_status_string(status: int) -> str:
    return lib().attn_status_string(status).decode()


def attn_last_error() -> str:
    return lib().attn_last_error().decode(errors="replace")


def attn_version() -> int:
    return int(lib().attn_version())


# ---------------------------------------------------------------------------
# Allocating conveniences. With an explicit `stream`, the outputs and every
# scratch buffer are allocated while that stream is torch's current stream,
# so the caching allocator ties their memory to it: a scratch buffer dropped
# on return is handed out again only to work ordered after these kernels on
# the same stream. The outputs belong to `stream` in the same way; a caller
# that reads them on another stream orders the two streams first, as with
# any torch tensor.
# ---------------------------------------------------------------------------

def _on(stream):
    return _torch().cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def forward(qkv, n_head: int, head_dim: int = 64, stream=None):
    """Returns (out, lse) for a packed (B, T, 3C) bf16 or fp32 GPU tensor."""
    with _on(stream):
        torch = _torch()
        B, T, C = _dims(qkv, n_head, head_dim)
        out = torch.empty((B, T, C), dtype=qkv.dtype, device=qkv.device)
        lse = torch.empty((B, n_head, T), dtype=torch.float32, device=qkv.device)
        attn_fwd(qkv, out, lse, n_head, head_dim, stream)
        return out, lse


def fp8_bwd_buffer_bytes(B: int, T: int, n_head: int) -> int:
    """Bytes of the FP8 backward buffer of attn_quantize_bwd_fp8 / attn_bwd_fp8."""
    n = int(lib().attn_fp8_bwd_buffer_bytes(B, T, n_head))
    if n < 0:
        raise ValueError("B, T and n_head must be non-negative")
    return n


def attn_quantize_bwd_fp8(dout, qkv, out, lse, fp8_bwd, n_head: int, head_dim: int = 64,
                          stream=None) -> None:
    torch = _torch()
    B, T, C = _dims(qkv, n_head, head_dim)
    _require(dout, "dout", torch.bfloat16, (B, T, C))
    _require(qkv, "qkv", torch.bfloat16, (B, T, 3 * C))
    _require(out, "out", torch.bfloat16, (B, T, C))
    _require(lse, "lse", torch.float32, (B, n_head, T))
    _require_bytes(fp8_bwd, "fp8_bwd", fp8_bwd_buffer_bytes(B, T, n_head))
    _check(lib().attn_quantize_bwd_fp8(_ptr(dout), _ptr(qkv), _ptr(out), _ptr(lse), _ptr(fp8_bwd),
                                       B, T, n_head, head_dim, _stream_ptr(stream)),
           "attn_quantize_bwd_fp8")


def attn_bwd_fp8(fp8, fp8_bwd, dqkv, n_head: int, head_dim: int = 64, stream=None) -> None:
    """fp8 / fp8_bwd: the buffers of attn_quantize_fp8 and attn_quantize_bwd_fp8
    for these shapes; dqkv (B, T, 3C) bf16 gives B and T."""
    torch = _torch()
    B, T, C = _dims(dqkv, n_head, head_dim)
    _require(dqkv, "dqkv", torch.bfloat16, (B, T, 3 * C))
    _require_bytes(fp8, "fp8", fp8_buffer_bytes(B, T, n_head))
    _require_bytes(fp8_bwd, "fp8_bwd", fp8_bwd_buffer_bytes(B, T, n_head))
    _check(lib().attn_bwd_fp8(_ptr(fp8), _ptr(fp8_bwd), _ptr(dqkv), B, T, n_head, head_dim,
                              _stream_ptr(stream)), "attn_bwd_fp8")


def backward_fp8(dout, qkv, out, lse, n_head: int, head_dim: int = 64, stream=None):
    """dqkv of the FP8 backward for the FP8 forward that produced (out, lse)
    on qkv: quantize the forward and backward operands into new buffers, then
    attn_bwd_fp8."""
    with _on(stream):
        torch = _torch()
        B, T, C = _dims(qkv, n_head, head_dim)
        f8 = torch.empty(fp8_buffer_bytes(B, T, n_head), dtype=torch.uint8, device=qkv.device)
        b8 = torch.empty(fp8_bwd_buffer_bytes(B, T, n_head), dtype=torch.uint8, device=qkv.device)
        dqkv = torch.empty_like(qkv)
        attn_quantize_fp8(qkv, f8, n_head, head_dim, stream)
        attn_quantize_bwd_fp8(dout, qkv, out, lse, b8, n_head, head_dim, stream)
        attn_bwd_fp8(f8, b8, dqkv, n_head, head_dim, stream)
        return dqkv


def forward_fp8(qkv, n_head: int, head_dim: int = 64, stream=None):
    """Returns (out, lse) of the FP8 forward for a packed (B, T, 3C) bf16 GPU
    tensor: attn_quantize_fp8 into a new buffer, then attn_fwd_fp8."""
    with _on(stream):
        torch = _torch()
        B, T, C = _dims(qkv, n_head, head_dim)
        fp8 = torch.empty(fp8_buffer_bytes(B, T, n_head), dtype=torch.uint8, device=qkv.device)
        out = torch.empty((B, T, C), dtype=torch.bfloat16, device=qkv.device)
        lse = torch.empty((B, n_head, T), dtype=torch.float32, device=qkv.device)
        attn_quantize_fp8(qkv, fp8, n_head, head_dim, stream)
        attn_fwd_fp8(fp8, out, lse, n_head, head_dim, stream)
        return out, lse


def backward(dout, qkv, out, lse, n_head: int, head_dim: int = 64, stream=None):
    """Returns dqkv (B, T, 3C) for the forward that produced (out, lse)."""
    with _on(stream):
        torch = _torch()
        B, T, C = _dims(qkv, n_head, head_dim)
        dqkv = torch.empty_like(qkv)
        delta = torch.empty(workspace_floats(B, T, n_head), dtype=torch.float32, device=qkv.device)
        attn_bwd(dout, qkv, out, lse, dqkv, delta, n_head, head_dim, stream)
        return dqkv
