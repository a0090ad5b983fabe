"""Seeded synthetic inputs for the block-diffusion denoise step.

This package holds random draws and the fp32 -> bf16 storage cast only: no
part of the attention or of the confidence commit is computed here.  It is the
one module that both sides of every parity test (and the bench) share: the
oracle consumes the arrays it returns after an exact upcast to float64, the
HIP path consumes the very same bits on the device.
"""
from .workloads import (  # noqa: F401
    ADALN_WORKLOADS,
    AdalnWorkload,
    LMHEAD_WORKLOADS,
    LMHeadWorkload,
    MAMBA_WORKLOADS,
    MambaWorkload,
    WORKLOADS,
    Workload,
    bf16_bits_to_f32,
    bf16_bits_to_f64,
    f32_to_bf16_bits,
    make_adaln_inputs,
    make_attention_inputs,
    make_commit_inputs,
    make_lmhead_inputs,
    make_mamba_inputs,
    make_eligible,
    loop_step_logits,
    loop_peak_values,
)
