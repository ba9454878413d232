"""The five synthetic workloads of the channel-pruned gated-MLP path.

Each FFN workload is one stack of independent gated-MLP layers (the layers do
not chain: every layer gets its own seeded prompt activations and decode
inputs).  The decoder-layer workload chains whole layers (attention and FFN)
over one residual stream, as a model's forward pass does.
Shapes follow the model families the POP notes evaluate (LLaMA-2-7B, Qwen2-7B,
a Mixtral-like MoE); the distributions are synthetic stand-ins for the QA and
generation benchmarks the notes measure on, since no dataset or trained weight
is used anywhere.

This module holds only sizes and distribution parameters, no arithmetic of the
method.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16": element type of weights and activations
    layers: int           # independent gated-MLP layers in the stack (experts for MoE)
    d: int                # model width D
    d_ff: int             # intermediate width D_FF
    r: float              # FFN pruning rate
    gamma: float          # partition width parameter (delta = gamma)
    prompt_batch: int     # B of the prompt
    prompt_len: int       # L of the prompt
    decode_steps: int
    decode_batch: int     # rows that share one mask per decode step
    weight_std: float = 0.02
    # prompt outliers: "scale" multiplies N(0,1) channels, "student_t" replaces them
    outlier_kind: str = "none"   # none | scale | student_t | drift_scale
    outlier_channels: int = 0
    outlier_factor: float = 20.0
    student_nu: float = 3.0
    outliers_in_decode: bool = False
    experts: int = 0             # >0: MoE layer with this many experts, top-2 routing
    top_k_route: int = 2
    notes: str = ""
    extra: dict = field(default_factory=dict)


TINY = Workload(
    name="tiny_f32", dtype="f32", layers=1, d=256, d_ff=688, r=0.3, gamma=0.1,
    prompt_batch=1, prompt_len=16, decode_steps=8, decode_batch=1,
    outlier_kind="scale", outlier_channels=4, outlier_factor=20.0,
    notes="single fp32 gated-MLP layer; prompt has 4 input channels scaled x20")

LLAMA2_7B = Workload(
    name="llama2_7b_ffn_b1", dtype="bf16", layers=32, d=4096, d_ff=11008, r=0.299,
    gamma=0.1, prompt_batch=1, prompt_len=512, decode_steps=256, decode_batch=1,
    outlier_kind="student_t", outlier_channels=41, student_nu=3.0,
    outliers_in_decode=True,
    notes="LLaMA-2-7B-shaped FFN stack; 1% of input channels heavy-tailed (t, nu=3)")

LLAMA2_7B_B16 = Workload(
    name="llama2_7b_ffn_b16", dtype="bf16", layers=32, d=4096, d_ff=11008, r=0.299,
    gamma=0.1, prompt_batch=16, prompt_len=2048, decode_steps=512, decode_batch=16,
    outlier_kind="student_t", outlier_channels=41, student_nu=3.0,
    outliers_in_decode=True,
    notes="batched decode, 16 rows share one mask (score = max over the batch)")

QWEN2_7B = Workload(
    name="qwen2_7b_ffn_b4", dtype="bf16", layers=28, d=3584, d_ff=18944, r=0.5,
    gamma=0.1, prompt_batch=4, prompt_len=1024, decode_steps=1024, decode_batch=4,
    outlier_kind="drift_scale", outlier_channels=36, outlier_factor=20.0,
    outliers_in_decode=True,
    notes="drifting outlier set: one member swapped per decode step (mask churn)")

MIXTRAL_MOE = Workload(
    name="mixtral_moe_ffn_t32", dtype="bf16", layers=8, d=4096, d_ff=14336, r=0.3,
    gamma=0.1, prompt_batch=8, prompt_len=1024, decode_steps=256, decode_batch=32,
    experts=8, top_k_route=2,
    notes="one MoE layer, 8 experts, top-2 routing of N(0,1) logits; one partition "
          "per expert over the prompt tokens routed to it")

LLAMA2_7B_LAYER = Workload(
    name="llama2_7b_layer_b1", dtype="bf16", layers=32, d=4096, d_ff=11008, r=0.299, gamma=0.1,
    prompt_batch=1, prompt_len=512, decode_steps=256, decode_batch=1,
    extra={"attention": {"n_heads": 32, "n_kv_heads": 32, "head_dim": 128, "eps": 1e-5, "rope_theta": 10000.0}},
    notes="32 chained LLaMA-2-7B-shaped decoder layers: dense attention over a key/value cache, the FFN pruned "
          "at the 29.9% that a 20% global budget gives it; RMSNorm gains 1, token inputs N(0,1)")

LLAMA2_7B_LAYER_B16 = Workload(
    name="llama2_7b_layer_b16", dtype="bf16", layers=32, d=4096, d_ff=11008, r=0.299, gamma=0.1,
    prompt_batch=16, prompt_len=512, decode_steps=256, decode_batch=16,
    extra={"attention": {"n_heads": 32, "n_kv_heads": 32, "head_dim": 128, "eps": 1e-5, "rope_theta": 10000.0}},
    notes="the decoder-layer stack decoding 16 sequences at once (one FFN mask per step for the batch)")

WORKLOADS = [TINY, LLAMA2_7B, LLAMA2_7B_B16, QWEN2_7B, MIXTRAL_MOE, LLAMA2_7B_LAYER, LLAMA2_7B_LAYER_B16]
BY_NAME = {w.name: w for w in WORKLOADS}
