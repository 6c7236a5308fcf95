"""Lossless multi-candidate tree sampling (oracle; test infrastructure only).

The independent per-node test of `verify.accept_and_select` is exact for
chains and for trees whose nodes have one drafted child, but not when a node
has several drafted children: two siblings can both pass, and the residual
ignores all but one of them.  This module implements the rule that keeps the
output distributed as the target's for any tree ("投机解码的五条路线", section
4, separates lossless verification from typical acceptance; the rejection
step and its residual are the featured article's section 2.1, applied once
per sibling):

  start at the root with r = p_root;
  at node v, try its children c_1, c_2, ... in increasing node id:
      accept c_j when u_{c_j} < r(x_{c_j}) / q_{c_j}(x_{c_j})
          -> emit x_{c_j}, move to c_j, r = p_{c_j}, start again;
      otherwise r <- norm([r - q_{c_j}]_+) and try the next child;
  when the children of v are exhausted (or v is a leaf) draw the final token
  from r with u_final (inverse CDF in token-id order).

For a chain this is exactly the independent rule (one child per node: the
first rejection ends the walk and the residual is norm([p_v - q_c]_+)).

Readings where the pages are silent:
  - siblings are tried in increasing node id (the rank order of the tree);
  - a child with q(x) = 0 is rejected (status bit 4 as in the independent
    rule, which flags any node with q(x) = 0);
  - if [r - q]_+ sums to 0, r is kept unchanged (the independent rule draws
    from p_v* in that case, the same thing for the first child);
  - node_accept / node_p / node_q describe the tests that were made: r(x) and
    q(x) at test time; children never tried get 0.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .sampling import inverse_cdf_rows


def lossless_walk(parent: np.ndarray, tokens: np.ndarray, u_accept: np.ndarray, u_final: np.ndarray,
                  p_rows: np.ndarray, q_rows: np.ndarray) -> Dict[str, np.ndarray]:
    """The walk above for a batch.  Shapes as in verify.accept_and_select (sampling mode)."""
    parent = np.asarray(parent, dtype=np.int64)
    tokens = np.asarray(tokens, dtype=np.int64)
    B, T = parent.shape
    V = p_rows.shape[-1]
    steps = np.arange(T)[None, :]
    bad_parent = (parent[:, 0] != -1) | ((parent[:, 1:] < 0) | (parent[:, 1:] >= steps[:, 1:])).any(axis=1)
    bad_token = ((tokens[:, 1:] < 0) | (tokens[:, 1:] >= V)).any(axis=1)
    status = (bad_parent * 1 + bad_token * 2).astype(np.int32)
    ok = status == 0
    par = np.where(ok[:, None], parent, 0)
    tok = np.where(ok[:, None], tokens, 0)
    bidx = np.arange(B)

    # status bit 4: some supplied draft gives its own token probability 0
    qself = q_rows[bidx[:, None], steps, tok]
    zero_any = (qself[:, 1:] <= 0.0).any(axis=1) if T > 1 else np.zeros(B, dtype=bool)
    status |= np.where(ok & zero_any, 4, 0).astype(np.int32)

    # children of every node in increasing id: child_at[b, v, k], -1 past the last
    child_at = np.full((B, T, T), -1, dtype=np.int64)
    nkids = np.zeros((B, T), dtype=np.int64)
    for i in range(1, T):
        pv = par[:, i]
        child_at[bidx, pv, nkids[bidx, pv]] = i
        nkids[bidx, pv] += 1

    v = np.zeros(B, dtype=np.int64)          # current node
    k = np.zeros(B, dtype=np.int64)          # next child of v to try
    depth = np.zeros(B, dtype=np.int64)
    r = p_rows[:, 0].astype(np.float64).copy()
    done = ~ok
    node_accept = np.zeros((B, T), dtype=np.uint8)
    node_accept[:, 0] = 1
    node_p = np.zeros((B, T))
    node_q = np.zeros((B, T))
    accept_margin = np.full((B, T), np.inf)
    tested = np.zeros((B, T), dtype=bool)
    path = np.full((B, T), -1, dtype=np.int64)
    path[:, 0] = 0
    out_tokens = np.full((B, T), -1, dtype=np.int64)
    final_tok = np.full(B, -1, dtype=np.int64)
    cdf_margin = np.full(B, np.inf)
    uf = np.asarray(u_final, dtype=np.float64)
    ua = np.asarray(u_accept, dtype=np.float64)

    for _ in range(2 * T + 1):             # each round accepts, rejects or ends a walk
        act = ~done
        if not act.any():
            break
        c = np.where(act, child_at[bidx, v, np.minimum(k, T - 1)], -1)
        c = np.where(act & (k < T), c, -1)
        fin = act & (c < 0)
        if fin.any():
            y, m = inverse_cdf_rows(r[fin], uf[fin])
            final_tok[fin] = y
            cdf_margin[fin] = m
            done |= fin
        test = act & (c >= 0)
        if not test.any():
            continue
        tb = bidx[test]
        cc = c[test]
        x = tok[tb, cc]
        rx = r[tb, x]
        qx = q_rows[tb, cc, x]
        node_p[tb, cc] = rx
        node_q[tb, cc] = qx
        tested[tb, cc] = True
        zq = qx <= 0.0
        ratio = np.where(zq, 0.0, rx / np.where(zq, 1.0, qx))
        acc = (~zq) & (ua[tb, cc] < ratio)
        accept_margin[tb, cc] = np.where(zq, np.inf, np.abs(ua[tb, cc] - ratio))
        # accepted: move down
        ab, ac = tb[acc], cc[acc]
        node_accept[ab, ac] = 1
        out_tokens[ab, depth[ab]] = tok[ab, ac]
        depth[ab] += 1
        path[ab, depth[ab]] = ac
        v[ab] = ac
        k[ab] = 0
        r[ab] = p_rows[ab, ac]
        # rejected: shrink the residual by this child's draft distribution
        rb, rc = tb[~acc], cc[~acc]
        resid = np.maximum(r[rb] - q_rows[rb, rc], 0.0)
        w = resid.sum(axis=-1)
        keep = w > 0.0
        r[rb[keep]] = resid[keep] / w[keep][:, None]
        k[rb] += 1

    out_tokens[bidx, depth] = final_tok
    path[~ok] = -1
    out_tokens[~ok] = -1
    final_node = np.where(ok, v, -1)
    accept_len = np.where(ok, depth, 0)
    from_residual = np.where(ok, nkids[bidx, v] > 0, False).astype(np.uint8)
    return dict(status=status, accept_len=accept_len.astype(np.int32), final_node=final_node.astype(np.int32),
                path=path.astype(np.int32), out_tokens=out_tokens.astype(np.int32), node_accept=node_accept,
                node_p=node_p, node_q=node_q, final_from_residual=from_residual,
                accept_margin=accept_margin, cdf_margin=cdf_margin, tested=tested, children=child_at,
                nkids=nkids)
