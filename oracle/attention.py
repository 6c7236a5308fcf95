"""Tree-masked attention over a shared KV prefix (oracle; test infrastructure only).

Definition ([P1] section 3.1 item 2: verification reuses the prefix KV cache and
only the new candidate positions get new KV; [P1] section 3.2: the tree is
flattened into one sequence with a mask that encodes its dependencies; [P4]
section "Tree Attention验证"; [P5] section 4):

  for sequence b, query head h, node i, with KV head kappa = floor(h * Hkv / Hq):
    S(b,i) = {0..L_b-1}  U  {L_b + j : j in anc*(i)}
    s_j    = scale * <Q[b,i,h,:], K[b,kappa,j,:]>      (scale = 1/sqrt(D))
    O[b,i,h,:] = sum_{j in S} softmax(s)_j * V[b,kappa,j,:]

The tree nodes' own K/V sit in the cache at slots L_b + i.  Everything is
evaluated in float64 from the stored values (bf16 inputs widen exactly).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .tree import ancestors


def visible_keys(kv_len: int, parent: Sequence[int], i: int) -> np.ndarray:
    """Explicit index list S(b,i): the whole prefix plus node i's root path in the tree slots."""
    tail = [kv_len + j for j in ancestors(parent, i)]
    return np.concatenate([np.arange(kv_len, dtype=np.int64), np.array(tail, dtype=np.int64)])


def tree_attention_node(q_i: np.ndarray, k: np.ndarray, v: np.ndarray, kv_len: int,
                        parent: Sequence[int], i: int, scale: Optional[float] = None,
                        heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """Attention output of node i for the given query heads.

    q_i: [Hq, D] (node i's queries); k, v: [Hkv, Lcap, D] (one sequence's cache).
    Returns [len(heads), D] float64.
    """
    hq, d = q_i.shape
    hkv = k.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if heads is None:
        heads = range(hq)
    keys = visible_keys(kv_len, parent, i)
    heads = list(heads)
    out = np.empty((len(heads), d), dtype=np.float64)
    gathered = {}  # kappa -> (K rows, V rows) of S(b,i), gathered once per KV head
    for n, h in enumerate(heads):
        kappa = (h * hkv) // hq
        if kappa not in gathered:
            gathered[kappa] = (np.asarray(k[kappa][keys], dtype=np.float64),
                               np.asarray(v[kappa][keys], dtype=np.float64))
        kk, vv = gathered[kappa]
        s = scale * (kk @ np.asarray(q_i[h], dtype=np.float64))
        w = np.exp(s - s.max())
        w /= w.sum()
        out[n] = w @ vv
    return out


def tree_attention_sequence(q: np.ndarray, k: np.ndarray, v: np.ndarray, kv_len: int,
                            parent: Sequence[int], scale: Optional[float] = None,
                            nodes: Optional[Sequence[int]] = None) -> np.ndarray:
    """Attention output for every (node, head) of one sequence: q [T,Hq,D] -> [T,Hq,D] float64.

    `nodes` restricts the computation to some nodes (the others stay NaN).
    """
    T, hq, d = q.shape
    out = np.full((T, hq, d), np.nan, dtype=np.float64)
    for i in (range(T) if nodes is None else nodes):
        out[i] = tree_attention_node(q[i], k, v, kv_len, parent, i, scale)
    return out
