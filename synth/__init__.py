"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the bench.

Holds random draws and layouts only; no arithmetic of the verify step.
"""
from .inputs import (WORKLOADS, Case, CaseSpec, as_f32, bf16_bits_to_f32, bf16_round_bits,
                     make_case, workload)
from .paged import PagedKV, page_case
from .trees import chain_tree, medusa_tree, sibling_rank

__all__ = ["WORKLOADS", "Case", "CaseSpec", "as_f32", "bf16_bits_to_f32", "bf16_round_bits",
           "workload", "make_case", "PagedKV", "page_case", "chain_tree", "medusa_tree", "sibling_rank"]
