"""Build the HIP library libcausal_attn.so in-tree with hipcc for gfx950.

Usage: python -m causal_flash_attention_amd.build [--verbose]
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

from causal_flash_attention_amd._paths import LIB_PATH, PKG_DIR

ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")

SOURCES = ["attn_api.hip", "attn_fwd_bf16.hip", "attn_bwd_bf16.hip", "attn_f32.hip",
           "attn_unfused_bf16.hip", "attn_decode_bf16.hip", "attn_fp8.hip",
           "attn_fp8_bwd.hip", "attn_block_bf16.hip", "peak_probe.hip"]

# -packed-fp32-ops: keep the compiler from forming packed fp32 add/mul/fma,
# which are avoided on this target; hipcc's host pass warns that it does not
# know the feature, which is harmless.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results stay in ordinary VGPRs instead of accumulation registers,
    # which the softmax and rescale would otherwise copy back and forth.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
    # the hand-scheduled programs clobber m0 on purpose (direct LDS loads)
    "-Wno-inline-asm",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


# Generators of hand-scheduled kernel programs: each writes an include next
# to itself (committed, so that the sources build as they stand).
GENERATORS = ["gen_attn_fwd_asm.py", "gen_attn_dkdv_asm.py", "gen_attn_dq_asm.py"]


def generate() -> None:
    for gen in GENERATORS:
        subprocess.run([sys.executable, os.path.join(CSRC, gen)], check=True, capture_output=True)


def build(verbose: bool = False) -> str:
    """Regenerate the kernel programs, then compile every HIP source into
    LIB_PATH; returns the path."""
    generate()
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if verbose and res.stderr:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
