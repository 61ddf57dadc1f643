"""Causal multi-head self-attention (FlashAttention style) for MI355X / gfx950.

The computation lives in the HIP library ``libcausal_attn.so`` (C ABI in
``include/causal_attn.h``); this package is its Python binding. Importing the
package does not load the library; the first call does, and fails loudly if
the library has not been built.
"""

from .binding import (  # noqa: F401
    AttnError,
    attn_block_bwd,
    attn_block_fwd,
    attn_bwd_fp8,
    attn_bwd,
    attn_bwd_dkdv,
    attn_bwd_dq,
    attn_bwd_dq_preprocess,
    attn_bwd_preprocess,
    attn_bwd_unfused,
    attn_decode,
    attn_fwd,
    attn_fwd_fp8,
    attn_fwd_unfused,
    attn_last_error,
    attn_quantize_bwd_fp8,
    attn_quantize_fp8,
    attn_status_string,
    attn_version,
    backward,
    backward_fp8,
    block_workspace_bytes,
    decode_workspace_floats,
    forward,
    forward_fp8,
    fp8_buffer_bytes,
    fp8_bwd_buffer_bytes,
    lib,
    unfused_row_stride,
    unfused_workspace_bytes,
    workspace_floats,
)
