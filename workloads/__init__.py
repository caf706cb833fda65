"""Seeded synthetic workloads for the ResidualAttention hot path.

This package only draws random numbers and describes shapes and the order of
pool operations.  It holds none of the attention arithmetic: the oracle
(`oracle/`) and the HIP library both consume what it produces, each with its
own code.

Shapes follow the attention layers of the models the ForkKV note evaluates
(Llama3-8B, Qwen2.5-14B) and the Qwen3-8B long-context prefill of the Penelope
review; the agent / shared-prefix topology follows the ForkKV note's ReAct and
MapReduce workflows ("Q1 / Q2 / Q3").  The pages' datasets are not used: every
value is drawn from a seeded PCG64 stream.
"""
from .configs import CONFIGS, WorkloadConfig, config_by_name
from .synth import (draw_inputs, pool_ops, chunk_ops, bf16_bits_from_f32,
                    pool_value_shapes)

__all__ = ["CONFIGS", "WorkloadConfig", "config_by_name", "draw_inputs", "pool_ops",
           "chunk_ops", "bf16_bits_from_f32", "pool_value_shapes"]
