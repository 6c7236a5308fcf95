"""Candidate-tree construction for Medusa verification (oracle; test infrastructure only).

What the pages fix:
  * [P4] section "Tree Attention验证": two Medusa heads, the top-2 candidates of
    each; level 1 holds head 1's two tokens, and every level-1 node takes head
    2's two tokens as its children, so the tree is the Cartesian product of
    the per-head top-k lists: 7 nodes, 4 root paths (A-B-D, A-B-E, A-C-F,
    A-C-G), parents in level order [-1, 0, 0, 1, 1, 2, 2].
  * [P3] section 2.2 (step two: pick candidates from each head's distribution
    by top-k, top-p or greedy) and section 4.2 (5 heads, top-k = 10 per
    head): a full product of 10 candidates over 5 heads is 111110 nodes, far
    more than one verify pass holds, so the product must be pruned.

Readings taken here (the pages give neither a pruning rule nor a tie rule):
  * A candidate at depth d is a rank tuple (r_1..r_d), r_k < caps[k-1]: it
    takes entry r_k of the top-k list of the distribution for depth k.  The
    row for depth 1 is the target model's own next-token logits and the row
    for depth k >= 2 is Medusa head k-1's; this module takes the stacked rows
    as given.  Heads see only the root's hidden state, so every depth-d node
    with the same last rank carries the same token (in P4's example F = D and
    G = E as tokens; the figure's letters name nodes).
  * Pruning: keep the T-1 tuples with the smallest key (prod_k (r_k + 1), d,
    (r_1..r_d) lexicographically); a child's key always exceeds its parent's,
    so the kept set contains the ancestors of each kept node.  When T-1 equals
    the size of the full product, nothing is pruned and the tree is P4's
    Cartesian product.
  * Node order: the root, then the kept tuples by (d, ranks lexicographically),
    so parent[i] < i and siblings are adjacent in rank order.
  * Top-k order: larger logit first; equal logits by smaller token id; NaN
    ranks below every number, -inf included.
Parity of the pruning rule beyond the full product is unpinned by the pages
(it is pinned here by brute force and invariants only).
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def topk_ids(row: np.ndarray, k: int) -> np.ndarray:
    """Token ids of the k best entries of one logits row, best first."""
    row = np.asarray(row, dtype=np.float64)
    ids = np.arange(row.shape[0])
    nan = np.isnan(row)
    val = np.where(nan, 0.0, row)
    # np.lexsort: the last key is the primary one
    order = np.lexsort((ids, -val, nan))
    return order[:k]


def _all_rank_tuples(caps: Sequence[int]) -> List[Tuple[int, ...]]:
    """Every rank tuple of depth 1..len(caps), depth by depth, lexicographic within a depth."""
    out: List[Tuple[int, ...]] = []
    level: List[Tuple[int, ...]] = [()]
    for cap in caps:
        level = [t + (r,) for t in level for r in range(int(cap))]
        out.extend(level)
    return out


def _prune_key(t: Tuple[int, ...]):
    prod = 1
    for r in t:
        prod *= r + 1
    return (prod, len(t), t)


def tree_template(caps: Sequence[int], nodes: int) -> Tuple[np.ndarray, np.ndarray]:
    """(parent[T], rank[T]) of the pruned rank-tuple tree with `nodes` nodes incl. the root.

    rank[i] is the last entry of node i's tuple (which top-k entry of its
    depth's row it takes); rank[0] = 0 for the root.
    """
    if nodes < 1:
        raise ValueError("a tree holds at least the root")
    tuples = _all_rank_tuples(caps)
    if nodes - 1 > len(tuples):
        raise ValueError("the caps allow only %d candidates" % len(tuples))
    kept = sorted(tuples, key=_prune_key)[:nodes - 1]
    kept.sort(key=lambda t: (len(t), t))
    where = {(): 0}
    parent = np.full(nodes, -1, dtype=np.int64)
    rank = np.zeros(nodes, dtype=np.int64)
    for i, t in enumerate(kept, start=1):
        where[t] = i
        parent[i] = where[t[:-1]]
        rank[i] = t[-1]
    return parent, rank


def build_tree(cand_logits: np.ndarray, root_token: np.ndarray, parent: Sequence[int],
               rank: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Fill a template for every sequence.

    cand_logits [B, depth, V]: row d-1 is the distribution depth-d candidates come from.
    Returns (parent [B, T], tokens [B, T]): tokens[b, 0] = root_token[b]; for i >= 1,
    tokens[b, i] = entry rank[i] of the top-k list of row depth(i) - 1.
    """
    B = cand_logits.shape[0]
    T = len(parent)
    depth = [0] * T
    for i in range(1, T):
        depth[i] = depth[int(parent[i])] + 1
    tokens = np.zeros((B, T), dtype=np.int64)
    for b in range(B):
        tokens[b, 0] = int(root_token[b])
        for i in range(1, T):
            best = topk_ids(cand_logits[b, depth[i] - 1], int(rank[i]) + 1)
            tokens[b, i] = best[int(rank[i])]
    return np.tile(np.asarray(parent, dtype=np.int64), (B, 1)), tokens
