"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the bench.

Holds random draws and layouts only; no arithmetic of the verify step.
"""
from .inputs import (CONFIGS, Case, CaseSpec, as_f32, bf16_bits_to_f32, bf16_round_bits,
                     config, make_case)
from .trees import chain_tree, medusa_tree, sibling_rank

__all__ = ["CONFIGS", "Case", "CaseSpec", "as_f32", "bf16_bits_to_f32", "bf16_round_bits",
           "config", "make_case", "chain_tree", "medusa_tree", "sibling_rank"]
