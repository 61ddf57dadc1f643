"""Seeded synthetic inputs for causal attention (host side, numpy only).

This module holds no attention arithmetic: it only draws i.i.d. normal numbers
and rounds them to the storage type. Tests feed the same arrays to the CPU
oracle and to the HIP library, and the bench uses it to fill device memory.

Definition of a draw ``normal(shape, std, seed, stream, dtype)``:

* The flat, row-major element range is cut into chunks of ``CHUNK`` elements.
* Chunk c is drawn from numpy's Philox4x64-10 counter-based generator
  (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
  3", SC'11) keyed by (seed, stream), with its 256-bit counter started at
  c * 2**192, through ``Generator.standard_normal`` in float64.
* Each value is multiplied by ``std`` in float64 and rounded to nearest-even
  float32; for bf16 that float32 is rounded to nearest-even bf16, kept as its
  16-bit pattern (the upper half of the float32 encoding).

The result depends only on (shape, std, seed, stream, dtype), never on the
number of threads used to fill it.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Sequence

import numpy as np

CHUNK = 1 << 20

# The streams used by every workload: the packed qkv tensor and the upstream
# gradient of the attention output.
STREAM_QKV = 0
STREAM_DOUT = 1


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to nearest-even bf16; returns uint16 bit patterns.

    NaN stays NaN (quiet); infinities and overflow to infinity follow IEEE
    round-to-nearest-even on the 16 dropped mantissa bits.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw_chunk(seed: int, stream: int, c: int, n: int, std: float) -> np.ndarray:
    bitgen = np.random.Philox(key=np.array([seed, stream], dtype=np.uint64),
                              counter=np.array([0, 0, 0, c], dtype=np.uint64))
    z = np.random.Generator(bitgen).standard_normal(n, dtype=np.float64)
    return (z * float(std)).astype(np.float32)


def normal(shape: Sequence[int], std: float, seed: int, stream: int,
           dtype: str = "bf16", threads: int | None = None) -> np.ndarray:
    """Draw an array of N(0, std^2) values, rounded to ``dtype``.

    dtype "f32" returns float32; "bf16" returns uint16 bf16 bit patterns.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16'")
    if seed < 0 or stream < 0:
        raise ValueError("seed and stream must be non-negative")
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape, dtype=np.int64)) if shape else 1
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    n_chunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        x = _draw_chunk(seed, stream, c, hi - lo, std)
        out[lo:hi] = x if dtype == "f32" else f32_to_bf16_bits(x)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if n_chunks <= 1 or threads <= 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


def attention_inputs(B: int, T: int, n_head: int, head_dim: int, dtype: str,
                     qkv_std: float = 1.0, dout_std: float = 1.0, seed: int = 0):
    """Packed qkv (B, T, 3C) from stream 0 and dout (B, T, C) from stream 1."""
    C = n_head * head_dim
    qkv = normal((B, T, 3 * C), qkv_std, seed, STREAM_QKV, dtype)
    dout = normal((B, T, C), dout_std, seed, STREAM_DOUT, dtype)
    return qkv, dout


def to_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of an array produced by :func:`normal`."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)
