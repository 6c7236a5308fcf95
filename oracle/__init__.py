"""CPU oracle for the speculative-decoding / Medusa verify step.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, float64 NumPy
definition of what the verify step computes.  Only the test-suite, the smoke
check and the bench's CPU-baseline leg may import it; the product path (the
HIP library and its Python binding) never does.  It shares no code with the
HIP path: it reads the same seeded inputs and nothing else.

Pages it follows (cited by title and section throughout):
  [P1] "大模型推理加速：推测解码与MTP核心原理与工程实践" (qwbw.cn)
  [P2] featured article on the founding speculative-decoding paper (hncyxsy.com),
       sections 2.1-2.3
  [P3] "Medusa推测解码：为LLM推理加速2-3倍的工程实践" (lpnh.cn)
  [P4] "推测解码技术详解：加速LLM推理的关键" (academy.cloudcc.io)
  [P5] "投机解码的五条路线:从小模型到 Prompt Lookup" (jennyma11.github.io)

Every function here is pinned by tests that do not re-derive it (worked
examples printed on the pages, closed forms, brute force on tiny inputs,
library routines, chi-square against the target distribution), except where a
docstring says "parity unpinned".
"""
from .tree import ancestors, check_parent, depths, tree_mask
from .attention import tree_attention_node, tree_attention_sequence
from .sampling import argmax_first, effective_distribution, inverse_cdf, inverse_cdf_rows, nucleus_margin
from .verify import (NEAR_TIE, TOPP_NEAR_TIE, accept_and_select, row_distributions, verify, verify_vocab,
                     widen)
from .lossless import lossless_walk
from .commit import commit_kv
from .paged import commit_kv_paged, gather_slots, kv_valid, pages_valid, slot_page_row, verify_paged
from .tree_build import build_tree, topk_ids, tree_template

__all__ = [
    "ancestors", "check_parent", "depths", "tree_mask",
    "tree_attention_node", "tree_attention_sequence",
    "argmax_first", "effective_distribution", "inverse_cdf", "inverse_cdf_rows", "nucleus_margin",
    "NEAR_TIE", "TOPP_NEAR_TIE", "accept_and_select", "row_distributions", "verify", "verify_vocab", "widen",
    "lossless_walk", "commit_kv",
    "commit_kv_paged", "gather_slots", "kv_valid", "pages_valid", "slot_page_row", "verify_paged",
    "build_tree", "topk_ids", "tree_template",
]
