"""Deterministic candidate trees for the verify step (input synthesis only).

The pages describe a Medusa candidate tree as per-head top-k candidates combined
into a shared-prefix tree ("推测解码技术详解：加速LLM推理的关键", section
"Tree Attention验证"; "Medusa推测解码：为LLM推理加速2-3倍的工程实践", section 3.2),
but give no pruning rule.  The rule used here is our own reading:

* a candidate at depth d is a rank tuple (r_1..r_d) with r_k < cap_k
  (r_k = which of head k's top-k guesses it takes);
* candidates are ranked by the key (prod(r_k + 1), d, ranks) ascending and
  the first T-1 are kept (a parent always sorts strictly before its children,
  so the kept set is closed under taking ancestors);
* kept nodes are ordered by (depth, ranks) after the root, so parent[i] < i
  and siblings are contiguous in rank order.

Nothing here computes any part of the verify step itself.
"""
from __future__ import annotations

import itertools
from typing import List, Sequence, Tuple


def medusa_tree(caps: Sequence[int], num_nodes: int) -> Tuple[List[int], List[Tuple[int, ...]]]:
    """Return (parent, ranks) for a pruned top-k tree of `num_nodes` nodes incl. the root."""
    if num_nodes < 1:
        raise ValueError("a tree has at least the root")
    cands = []
    for depth in range(1, len(caps) + 1):
        for ranks in itertools.product(*[range(c) for c in caps[:depth]]):
            prod = 1
            for r in ranks:
                prod *= r + 1
            cands.append((prod, depth, ranks))
    cands.sort()
    if num_nodes - 1 > len(cands):
        raise ValueError("caps too small for the requested node count")
    kept = sorted(cands[: num_nodes - 1], key=lambda c: (c[1], c[2]))
    index = {(): 0}
    parent = [-1]
    ranks_out: List[Tuple[int, ...]] = [()]
    for k, (_, _, ranks) in enumerate(kept, start=1):
        index[ranks] = k
        parent.append(index[ranks[:-1]])
        ranks_out.append(ranks)
    return parent, ranks_out


def chain_tree(gamma: int) -> List[int]:
    """A chain of gamma draft tokens after the root: parent[i] = i - 1."""
    return [-1] + list(range(gamma))


def sibling_rank(parent: Sequence[int]) -> List[int]:
    """Position of each node among its parent's children (root -> 0)."""
    seen = {}
    out = []
    for i, p in enumerate(parent):
        if i == 0:
            out.append(0)
            continue
        r = seen.get(p, 0)
        out.append(r)
        seen[p] = r + 1
    return out
