"""Seeded synthetic inputs for routed sparse causal attention.

This package only draws random numbers and arranges them into the shapes the
workloads need.  It computes none of the method's steps (no block summaries,
addresses, posting lists, probes, reranking or attention), so both the CPU
oracle and the HIP path can take their inputs from it without sharing any of
the method's arithmetic.
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_round,
    make_core_inputs,
    make_grad_inputs,
    make_mixer_inputs,
    workload,
    zipf_code_bias,
)
