"""Seeded synthetic inputs for MLA latent-cache decode.

This module only draws numbers and lays them out (lengths, weights, queries,
latents, the page table). It holds none of the attention arithmetic, so both
the fp64 oracle and the HIP path can take their inputs from it without sharing
any of the computation under test.
"""
from .synth import (  # noqa: F401
    WORKLOADS,
    Workload,
    Inputs,
    make,
    seq_latents,
    seq_index_keys,
    random_selection,
    score_rows,
    round_bf16,
    bf16_bits,
)
