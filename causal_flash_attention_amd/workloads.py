"""The synthetic attention workloads, by name and size.

Shapes are those of the GPT-2 family trained in "Let's reproduce GPT-2 (124M)"
(12 layers of width 768 for 124M, per the theprofessional.online summary) and
its larger siblings (the 350M model of "Réimplémenter à bas coût le modèle
GPT-2 avec llm.c", section "Modèle 350M"); head count and head width are those
of the released GPT-2 models. Values are i.i.d. normal draws from
:mod:`causal_flash_attention_amd.inputs` (seed 0, qkv on stream 0, dout on
stream 1) standing in for activations of a model trained on FineWeb-Edu, which
is not available here.
"""

from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    n_head: int
    head_dim: int
    dtype: str          # "f32" or "bf16": storage type of qkv, out, dout, dqkv
    qkv_std: float
    dout_std: float

    @property
    def C(self) -> int:
        return self.n_head * self.head_dim

    def counted_flops(self) -> dict:
        """Causal FLOPs by the usual convention: forward 2*B*H*T^2*d,
        backward 2.5 times the forward."""
        fwd = 2.0 * self.B * self.n_head * self.T * self.T * self.head_dim
        return {"fwd": fwd, "bwd": 2.5 * fwd, "total": 3.5 * fwd}


WORKLOADS = (
    Workload("tiny_f32_b1_h2_t64", 1, 64, 2, 64, "f32", 1.0, 1.0),
    Workload("gpt2_124m_b16_t1024", 16, 1024, 12, 64, "bf16", 1.0, 0.01),
    Workload("gpt2_124m_b64_t1024", 64, 1024, 12, 64, "bf16", 1.0, 0.01),
    Workload("gpt2_350m_b16_t1024", 16, 1024, 16, 64, "bf16", 1.0, 0.01),
    Workload("gpt2_1p5b_style_b4_t2048_h25", 4, 2048, 25, 64, "bf16", 1.0, 0.01),
)

BY_NAME = {w.name: w for w in WORKLOADS}

# The workload the headline throughput is quoted on: one GPT-2 124M attention
# layer at micro-batch 16 and context 1024.
HEADLINE = BY_NAME["gpt2_124m_b16_t1024"]
