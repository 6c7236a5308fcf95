"""Candidate-tree structure from a parent[] array (oracle; test infrastructure only).

A Medusa candidate tree is flattened into one sequence of T nodes; node 0 is
the root (the current token, [P1] section 2.3: the root of the speculation
tree is the current step), and each node attends to exactly the nodes on its
own root path, itself included, never to siblings ([P4] section
"Tree Attention验证", the 7x7 mask; [P5] section 4, siblings may not peek at
each other; [P3] section 3.2, a node's context is the path back to the root).
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np


def check_parent(parent: Sequence[int]) -> bool:
    """True iff parent[] is a topologically ordered tree: parent[0] = -1, 0 <= parent[i] < i."""
    if len(parent) == 0 or int(parent[0]) != -1:
        return False
    return all(0 <= int(parent[i]) < i for i in range(1, len(parent)))


def depths(parent: Sequence[int]) -> List[int]:
    """depth(0) = 0, depth(i) = depth(parent[i]) + 1."""
    d = [0] * len(parent)
    for i in range(1, len(parent)):
        d[i] = d[int(parent[i])] + 1
    return d


def ancestors(parent: Sequence[int], i: int) -> List[int]:
    """anc*(i): node i and all its ancestors, listed root first."""
    path = []
    j = i
    while j != -1:
        path.append(j)
        j = int(parent[j])
    return path[::-1]


def tree_mask(parent: Sequence[int]) -> np.ndarray:
    """T x T visibility matrix: mask[i, j] = 1 iff node j is on node i's root path."""
    T = len(parent)
    m = np.zeros((T, T), dtype=np.uint8)
    for i in range(T):
        for j in ancestors(parent, i):
            m[i, j] = 1
    return m
