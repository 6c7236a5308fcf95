"""Acceptance, residual/bonus sampling and longest-path selection (oracle; test infrastructure only).

Rules, in the pages' order:

* Token-level test: accept draft x with probability min(1, p(x)/q(x)); with a
  supplied uniform u in [0,1) this is  u < p(x)/q(x)  ([P2] section 2.1; [P4]
  section "数学保证：无损输出质量" compares a uniform with the ratio; [P5]
  section on exact verification).  For tree node i, p is the target row of its
  parent (the row that predicts node i) and q is node i's own draft row.
* On rejection, sample from norm([p - q]_+) ([P2] section 2.1; [P4] same
  section; [P5]).  If every candidate on the path passed, draw a bonus token
  from the target's next-position distribution ([P2] section 2.2; [P5]).
* Chains are checked left to right and stop at the first rejection ([P2]
  section 2.2); in a tree only the prefix accepted consecutively from the root
  counts and the longest such path is kept ([P1] section 2.3; [P5] figure 3).
* Greedy mode accepts a candidate iff it equals the target's best token at
  that position ([P1] section 3.1 item 3; [P5]).

Readings where the pages are silent (also listed with the design notes):
  - v* = deepest node whose whole root path is accepted; ties -> smallest index.
  - the residual at v* uses q of v*'s smallest-index child; if [p - q]_+ sums
    to 0, sample from p.
  - q_i(x_i) = 0 for a supplied draft: reject and flag status bit 4.
  - in a tree with several drafted children per node each child is tested
    independently against its parent's p; this is lossless for chains and
    single-child trees only (parity unpinned for the multi-child sampling law).

Status bits: 1 invalid parent[], 2 token id out of range, 4 some q_i(x_i) = 0,
8 kv_len out of range.  Bits 1 or 2 void the sequence: accept_len 0,
final_node -1, path and out_tokens all -1.

Near-ties: a decision whose uniform lies within NEAR_TIE of its threshold
(accept test, inverse-CDF boundary), or a top-p cut whose cumulative mass lies
within TOPP_NEAR_TIE of top_p, is reported, and every output of that sequence
that depends on it is excluded from bit-exact comparison.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .attention import tree_attention_sequence
from .sampling import argmax_first, effective_distribution, inverse_cdf_rows, nucleus_margin
from .tree import check_parent

NEAR_TIE = 1e-5        # band for decisions taken against a supplied uniform
TOPP_NEAR_TIE = 1e-6   # band for the top-p cut (no uniform: fp32 mass error bound, ~2e-7, x5)


def widen(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Stored activations -> float64 (bf16 arrives as uint16 bit patterns)."""
    if dtype == "bf16":
        return (np.asarray(arr).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def row_distributions(logits: np.ndarray, temperature: float, top_p: float):
    """Effective distribution and top-p margin of every row of logits [R, V]."""
    p = np.empty(logits.shape, dtype=np.float64)
    margin = np.empty(logits.shape[0], dtype=np.float64)
    for r in range(logits.shape[0]):
        p[r] = effective_distribution(logits[r], temperature, top_p)
        margin[r] = nucleus_margin(logits[r], temperature, top_p)
    return p, margin


def accept_and_select(parent: np.ndarray, tokens: np.ndarray, u_accept: np.ndarray,
                      u_final: np.ndarray, mode: str, vocab: int,
                      p_rows: Optional[np.ndarray] = None, q_rows: Optional[np.ndarray] = None,
                      greedy_rows: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Steps 3 and 4 for a batch of sequences.

    parent, tokens, u_accept: [B,T]; u_final: [B].
    sampling: p_rows, q_rows [B,T,V] effective target / draft distributions
              (q row 0 unused).
    greedy_rows [B,T]: best target token of each row (needed in greedy mode,
              reported as row_token when given).
    """
    parent = np.asarray(parent, dtype=np.int64)
    tokens = np.asarray(tokens, dtype=np.int64)
    B, T = parent.shape
    # parent[] must be a topologically ordered tree (see check_parent), tokens in [0, V)
    steps = np.arange(T)[None, :]
    bad_parent = (parent[:, 0] != -1) | ((parent[:, 1:] < 0) | (parent[:, 1:] >= steps[:, 1:])).any(axis=1)
    bad_token = ((tokens[:, 1:] < 0) | (tokens[:, 1:] >= vocab)).any(axis=1)
    status = (bad_parent * 1 + bad_token * 2).astype(np.int32)
    ok = status == 0
    par = np.where(ok[:, None], parent, 0)
    par[:, 0] = 0
    tok = np.where(ok[:, None], tokens, 0)
    bidx = np.arange(B)

    node_p = np.zeros((B, T), dtype=np.float64)
    node_q = np.zeros((B, T), dtype=np.float64)
    accept_margin = np.full((B, T), np.inf)
    a = np.zeros((B, T), dtype=bool)
    a[:, 0] = True
    for i in range(1, T):
        if mode == "sampling":
            pi = p_rows[bidx, par[:, i], tok[:, i]]
            qi = q_rows[bidx, i, tok[:, i]]
            node_p[:, i] = pi
            node_q[:, i] = qi
            zero_q = qi <= 0.0
            ratio = np.where(zero_q, 0.0, pi / np.where(zero_q, 1.0, qi))
            a[:, i] = (~zero_q) & (u_accept[:, i].astype(np.float64) < ratio)
            accept_margin[:, i] = np.where(zero_q, np.inf, np.abs(u_accept[:, i] - ratio))
            status |= np.where(ok & zero_q, 4, 0).astype(np.int32)
        else:
            a[:, i] = tok[:, i] == greedy_rows[bidx, par[:, i]]

    # acc*(i) = a_i and acc*(parent(i)); depth(i) = depth(parent(i)) + 1
    acc = np.zeros((B, T), dtype=bool)
    acc[:, 0] = True
    depth = np.zeros((B, T), dtype=np.int64)
    for i in range(1, T):
        acc[:, i] = a[:, i] & acc[bidx, par[:, i]]
        depth[:, i] = depth[bidx, par[:, i]] + 1
    key = np.where(acc, depth, -1)
    vstar = np.argmax(key, axis=1)            # deepest; first index wins ties
    accept_len = depth[bidx, vstar]

    # first (smallest-index) child of every node, -1 for leaves
    first_child = np.full((B, T), -1, dtype=np.int64)
    for i in range(T - 1, 0, -1):
        first_child[bidx, par[:, i]] = i

    # the token drawn at v*:
    #   greedy -> best target token of row v*
    #   v* has children -> residual norm([p_v* - q_c]_+), c = first child (p_v* if that is all zero)
    #   v* is a leaf -> bonus token from p_v*
    cdf_margin = np.full(B, np.inf)
    fc = first_child[bidx, vstar]
    if mode == "greedy":
        final_tok = greedy_rows[bidx, vstar].astype(np.int64)
    else:
        pv = p_rows[bidx, vstar]
        qc = q_rows[bidx, np.maximum(fc, 0)]
        resid = np.maximum(pv - qc, 0.0)
        use_resid = (fc >= 0) & (resid.sum(axis=-1) > 0.0)
        w = np.where(use_resid[:, None], resid, pv)
        final_tok, cdf_margin = inverse_cdf_rows(w, np.asarray(u_final, dtype=np.float64))
    from_residual = ((fc >= 0) & (mode == "sampling")).astype(np.uint8)

    # root-to-v* path and the emitted tokens
    path = np.full((B, T), -1, dtype=np.int64)
    j = vstar.copy()
    for _ in range(T):
        live = j >= 0
        path[bidx[live], depth[bidx[live], j[live]]] = j[live]
        j = np.where(live & (j > 0), par[bidx, np.maximum(j, 0)], -1)
    out_tokens = np.full((B, T), -1, dtype=np.int64)
    for k in range(T - 1):
        take = k < accept_len
        out_tokens[take, k] = tok[take, path[take, k + 1]]
    out_tokens[bidx, accept_len] = final_tok
    path[~ok] = -1
    out_tokens[~ok] = -1

    final_node = np.where(ok, vstar, -1)
    accept_len = np.where(ok, accept_len, 0)
    final_from_residual = np.where(ok, from_residual, 0).astype(np.uint8)
    row_token = (np.asarray(greedy_rows, dtype=np.int64) if greedy_rows is not None
                 else np.full((B, T), -1, dtype=np.int64))
    return dict(status=status, accept_len=accept_len.astype(np.int32),
                final_node=final_node.astype(np.int32), path=path.astype(np.int32),
                out_tokens=out_tokens.astype(np.int32), node_accept=a.astype(np.uint8),
                node_p=node_p, node_q=node_q, row_token=row_token.astype(np.int32),
                final_from_residual=final_from_residual,
                accept_margin=accept_margin, cdf_margin=cdf_margin, first_child=first_child)


def verify_vocab(parent, tokens, target_logits, draft_logits, u_accept, u_final, *,
                 mode: str, temperature: float = 1.0, top_p: float = 1.0,
                 accept_band: float = NEAR_TIE, cdf_band: float = NEAR_TIE,
                 topp_band: float = TOPP_NEAR_TIE, rule: str = "independent") -> Dict[str, np.ndarray]:
    """Steps 2-4 for a batch: distributions, acceptance, final token and path.

    The *_band arguments set how close to its threshold a decision must be to
    be flagged as a near-tie (defaults: the bands stated above).  rule:
    "independent" (each node tested against its parent's p, longest accepted
    root path) or "lossless" (the sibling walk of oracle.lossless; sampling only).
    """
    target_logits = np.asarray(target_logits)
    B, T, V = target_logits.shape
    p_rows = q_rows = greedy_rows = None
    tmargin = np.full((B, T), np.inf)
    dmargin = np.full((B, T), np.inf)
    if mode == "sampling":
        p_rows = np.empty((B, T, V), dtype=np.float64)
        q_rows = np.zeros((B, T, V), dtype=np.float64)
        for b in range(B):
            p_rows[b], tmargin[b] = row_distributions(target_logits[b], temperature, top_p)
            if T > 1:
                q_rows[b, 1:], dmargin[b, 1:] = row_distributions(
                    np.asarray(draft_logits)[b, 1:], temperature, top_p)
    greedy_rows = argmax_first(target_logits)
    if rule == "lossless" and mode == "sampling":
        return _lossless_vocab(parent, tokens, u_accept, u_final, p_rows, q_rows, greedy_rows,
                               tmargin, dmargin, accept_band, cdf_band, topp_band)
    out = accept_and_select(parent, tokens, u_accept, u_final, mode, V, p_rows=p_rows,
                            q_rows=q_rows, greedy_rows=greedy_rows)

    # near-tie bookkeeping
    par = np.clip(np.asarray(parent, dtype=np.int64), 0, T - 1)
    bidx = np.arange(B)[:, None]
    node_near = ((out["accept_margin"] < accept_band) | (tmargin[bidx, par] < topp_band)
                 | (dmargin < topp_band))
    node_near[:, 0] = False
    # the final draw at v*: its CDF boundary and the top-p cuts of the rows it reads
    vstar = np.maximum(out["final_node"], 0)
    b1 = np.arange(B)
    fc = out["first_child"][b1, vstar]
    final_near = ((out["cdf_margin"] < cdf_band) | (tmargin[b1, vstar] < topp_band)
                  | ((fc >= 0) & (dmargin[b1, np.maximum(fc, 0)] < topp_band)))
    seq_near = node_near.any(axis=1) | final_near
    out.update(node_near=node_near, final_near=final_near, seq_near=seq_near,
               target_topp_margin=tmargin, draft_topp_margin=dmargin)
    if mode == "sampling":
        out["p_rows"], out["q_rows"] = p_rows, q_rows
    return out


def _lossless_vocab(parent, tokens, u_accept, u_final, p_rows, q_rows, greedy_rows, tmargin, dmargin,
                    accept_band, cdf_band, topp_band):
    """verify_vocab's result under the lossless sibling walk, with its near-tie flags."""
    from .lossless import lossless_walk

    out = lossless_walk(parent, tokens, u_accept, u_final, p_rows, q_rows)
    B, T = np.asarray(parent).shape
    out["row_token"] = np.asarray(greedy_rows, dtype=np.int32)
    tested = out["tested"]
    node_near = tested & (out["accept_margin"] < accept_band)
    node_near[:, 0] = False
    # every row the walk read: target rows of the path, draft rows of tested children
    rows_near = np.zeros(B, dtype=bool)
    for b in range(B):
        path = out["path"][b]
        on = path[path >= 0]
        if len(on):
            rows_near[b] |= bool((tmargin[b, on] < topp_band).any())
        rows_near[b] |= bool((dmargin[b][tested[b]] < topp_band).any())
    final_near = (out["cdf_margin"] < cdf_band) | rows_near
    out.update(node_near=node_near, final_near=final_near, seq_near=node_near.any(axis=1) | final_near,
               target_topp_margin=tmargin, draft_topp_margin=dmargin, p_rows=p_rows, q_rows=q_rows)
    return out


def verify(case, *, attention: bool = True, seqs=None, rule: str = "independent",
           **bands) -> Dict[str, np.ndarray]:
    """The whole verify step on a case (any object with the synthetic-case fields).

    seqs: restrict to some sequence indices (outputs are for those, in order).
    bands: accept_band / cdf_band / topp_band overrides for the near-tie flags.
    """
    spec = case.spec
    seqs = list(range(case.parent.shape[0])) if seqs is None else list(seqs)
    draft = None if case.draft_logits is None else case.draft_logits[seqs]
    out = verify_vocab(case.parent[seqs], case.tokens[seqs], case.target_logits[seqs], draft,
                       case.u_accept[seqs], case.u_final[seqs], mode=spec.mode,
                       temperature=spec.temperature, top_p=spec.top_p, rule=rule, **bands)
    if attention:
        T = case.parent.shape[1]
        lcap = case.k_cache.shape[2]
        attn = np.full((len(seqs),) + case.q.shape[1:], np.nan)
        kv_status = np.zeros(len(seqs), dtype=np.int32)
        for n, b in enumerate(seqs):
            L = int(case.kv_len[b])
            if L < 0 or L + T > lcap:
                kv_status[n] = 8
                continue
            if not check_parent(case.parent[b]):
                continue
            attn[n] = tree_attention_sequence(widen(case.q[b], spec.dtype),
                                              widen(case.k_cache[b], spec.dtype),
                                              widen(case.v_cache[b], spec.dtype),
                                              L, case.parent[b])
        out["attn_out"] = attn
        out["status"] = out["status"] | kv_status
    return out
