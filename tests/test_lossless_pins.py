"""Pins for the lossless sibling walk (oracle.lossless), each against something other than itself.

* On chains it must agree exactly with the independent rule, which the
  chain pins in test_oracle_pins.py already tie to the target law.
* For trees whose nodes have several drafted children, the law of the emitted
  tokens must be the target's: chi-square of the first token at a branching
  root and two levels down, and the joint law of two tokens of a table-driven
  language model.  The independent rule must fail the same test (power check).
* Forced cases: u = 0 follows the first children to a leaf; p = q accepts the
  first child at every node.
"""
import numpy as np
import pytest
import scipy.stats

import oracle
import synth
from oracle.lossless import lossless_walk


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([4321] + list(key))))


def _draw_rows(rng, q, n):
    """One draw per row of q [n, V] (or a shared row [V]) by inverse CDF."""
    q = np.broadcast_to(q, (n, q.shape[-1]))
    c = np.cumsum(q, axis=1)
    return np.minimum((rng.random(n)[:, None] * c[:, -1:] >= c).sum(axis=1), q.shape[-1] - 1)


@pytest.mark.parametrize("name,kw", [("tiny-chain-f32", dict(batch=400, seed=(5, 1))),
                                     ("chain-batch32-topp", dict(batch=64, vocab=2000, prefix_len=64,
                                                                 ragged=None, seed=(5, 2)))])
def test_lossless_walk_equals_independent_rule_on_chains(name, kw):
    case = synth.make_case(synth.workload(name, **kw), with_kv=False)
    a = oracle.verify(case, attention=False)
    b = oracle.verify(case, attention=False, rule="lossless")
    for k in ("status", "accept_len", "final_node", "path", "out_tokens", "final_from_residual"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    t = b["tested"]
    # the walk tests the path's nodes and the first rejected one
    np.testing.assert_array_equal(a["node_accept"][t], b["node_accept"][t])
    np.testing.assert_array_equal(a["node_p"][t], b["node_p"][t])
    np.testing.assert_array_equal(a["node_q"][t], b["node_q"][t])
    assert (b["node_accept"][~t][:, ] <= 1).all()


def _tree_trials(parent, p_rows, q_rows, n, rng, rule):
    """n trials of one tree with fixed rows: drafts of node i drawn from q_rows[i]."""
    parent = np.asarray(parent)
    T, V = p_rows.shape
    tokens = np.zeros((n, T), dtype=np.int64)
    for i in range(1, T):
        tokens[:, i] = _draw_rows(rng, q_rows[i], n)
    P = np.broadcast_to(p_rows, (n, T, V))
    Q = np.broadcast_to(q_rows, (n, T, V))
    par = np.tile(parent, (n, 1))
    u_acc = rng.random((n, T))
    u_fin = rng.random(n)
    if rule == "lossless":
        return lossless_walk(par, tokens, u_acc, u_fin, P, Q)
    return oracle.accept_and_select(par, tokens, u_acc, u_fin, "sampling", V, p_rows=P, q_rows=Q)


def _chi2(counts, p):
    support = p > 0
    assert counts[~support].sum() == 0
    exp = p[support] * counts.sum()
    return float(((counts[support] - exp) ** 2 / exp).sum()), int(support.sum()) - 1


def _first_token_chi2(parent, p_rows, q_rows, trials, seed, rule):
    rng = _rng(1, seed)
    V = p_rows.shape[1]
    counts = np.zeros(V, dtype=np.int64)
    done = 0
    while done < trials:
        n = min(200_000, trials - done)
        res = _tree_trials(parent, p_rows, q_rows, n, rng, rule)
        counts += np.bincount(res["out_tokens"][:, 0], minlength=V)
        done += n
    return _chi2(counts, p_rows[0])


def _rows(rng, T, V, scale=1.5, noise=1.0):
    zt = rng.standard_normal((T, V)) * scale
    zq = zt + rng.standard_normal((T, V)) * noise
    p = np.stack([oracle.effective_distribution(z, 1.0) for z in zt])
    q = np.stack([oracle.effective_distribution(z, 1.0) for z in zq])
    return p, q


@pytest.mark.slow
def test_chi_square_first_token_three_children_at_the_root():
    rng = _rng(2)
    V = 16
    parent = [-1, 0, 0, 0]
    p, q = _rows(rng, 4, V)
    q[2] = q[1]            # siblings drafted from one distribution (Medusa) ...
    q[3] = oracle.effective_distribution(rng.standard_normal(V), 1.0)   # ... or from another
    chi2, df = _first_token_chi2(parent, p, q, 1_000_000, 2, "lossless")
    assert df == 15 and chi2 < scipy.stats.chi2.ppf(0.999, df), chi2


@pytest.mark.slow
def test_chi_square_first_token_two_level_tree():
    rng = _rng(3)
    V = 16
    parent = [-1, 0, 0, 1, 1, 2, 2]
    p, q = _rows(rng, 7, V)
    chi2, df = _first_token_chi2(parent, p, q, 1_000_000, 3, "lossless")
    assert chi2 < scipy.stats.chi2.ppf(0.999, df), chi2


def test_independent_rule_is_biased_with_several_children():
    """Power check: the same chi-square rejects the independent per-node rule on a branching root."""
    rng = _rng(4)
    V = 16
    parent = [-1, 0, 0, 0]
    p, q = _rows(rng, 4, V, scale=2.0, noise=1.5)
    chi2, df = _first_token_chi2(parent, p, q, 200_000, 4, "independent")
    assert chi2 > scipy.stats.chi2.ppf(0.999, df), chi2
    chi2, df = _first_token_chi2(parent, p, q, 200_000, 5, "lossless")
    assert chi2 < scipy.stats.chi2.ppf(0.999, df), chi2


@pytest.mark.slow
def test_joint_law_of_two_tokens_branching_table_lm():
    """A table-driven target/draft pair decoded with a branching tree (2 children per node, depth 2).

    Every node's target row is p(. | tokens on its root path) and its draft is
    drawn from q(. | the same context).  The first two emitted tokens must
    follow p(y1) p(y2 | y1); when a round emits one token, a second round
    (fresh tree from the prefix y1) supplies y2.
    """
    rng = _rng(6)
    V = 4
    parent = np.array([-1, 0, 0, 1, 1, 2, 2])
    T = parent.size
    nctx = 1 + V + V ** 2 + V ** 3
    zt = rng.standard_normal((nctx, V)) * 1.2
    zq = zt + rng.standard_normal((nctx, V)) * 0.8
    Pt = np.stack([oracle.effective_distribution(z, 1.0) for z in zt])
    Qt = np.stack([oracle.effective_distribution(z, 1.0) for z in zq])

    def ctx_id(ctx):
        ln = ctx.shape[1]
        base = sum(V ** k for k in range(ln))
        code = np.zeros(ctx.shape[0], dtype=np.int64)
        for c in range(ln):
            code = code * V + ctx[:, c]
        return base + code

    def one_round(prefix, n):
        tokens = np.zeros((n, T), dtype=np.int64)
        ctxs = [prefix]                      # context after node i
        prows = np.zeros((n, T, V))
        qrows = np.zeros((n, T, V))
        prows[:, 0] = Pt[ctx_id(prefix)]
        for i in range(1, T):
            pctx = ctxs[parent[i]]
            q = Qt[ctx_id(pctx)]
            x = _draw_rows(rng, q, n)
            tokens[:, i] = x
            qrows[:, i] = q
            ctx = np.concatenate([pctx, x[:, None]], axis=1)
            ctxs.append(ctx)
            prows[:, i] = Pt[ctx_id(ctx)]
        return lossless_walk(np.tile(parent, (n, 1)), tokens, rng.random((n, T)), rng.random(n), prows, qrows)

    trials = 400_000
    r1 = one_round(np.zeros((trials, 0), dtype=np.int64), trials)
    y1 = r1["out_tokens"][:, 0]
    y2 = np.where(r1["accept_len"] >= 1, r1["out_tokens"][:, 1], -1)
    need = y2 < 0
    r2 = one_round(y1[need][:, None], int(need.sum()))
    y2[need] = r2["out_tokens"][:, 0]
    counts = np.bincount(y1 * V + y2, minlength=V * V)
    joint = np.array([Pt[0][a] * Pt[1 + a][b] for a in range(V) for b in range(V)])
    chi2, df = _chi2(counts, joint)
    assert chi2 < scipy.stats.chi2.ppf(0.999, df), chi2


def test_forced_walks():
    rng = _rng(7)
    V = 12
    parent = np.array([[-1, 0, 0, 1, 1, 3]])
    p, q = _rows(rng, 6, V)
    tokens = np.array([[0, 3, 5, 7, 2, 9]])
    P, Q = p[None], q[None]
    # u = 0: every child with q(x) > 0 and r(x) > 0 passes; the walk follows first children
    for i in range(1, 6):
        assert p[parent[0, i], tokens[0, i]] > 0 and q[i, tokens[0, i]] > 0
    res = lossless_walk(parent, tokens, np.zeros((1, 6)), np.array([0.37]), P, Q)
    assert list(res["path"][0]) == [0, 1, 3, 5, -1, -1]
    assert res["accept_len"][0] == 3 and res["final_from_residual"][0] == 0
    y = int(np.searchsorted(np.cumsum(p[5]), 0.37 * p[5].sum(), side="right"))
    assert list(res["out_tokens"][0]) == [3, 7, 9, y, -1, -1]
    # every draft row equals its parent's target row (q_i = p_parent(i)): the first child
    # passes at every node for any u < 1
    qp = p[np.maximum(parent[0], 0)]
    res = lossless_walk(parent, tokens, np.full((1, 6), 0.999), np.array([0.5]), P, qp[None])
    assert list(res["path"][0][:4]) == [0, 1, 3, 5]
    # a child with q(x) = 0 is rejected and flagged; its sibling is tried next against the residual
    q0 = q.copy()
    q0[1, tokens[0, 1]] = 0.0
    q0[1] /= q0[1].sum()
    res = lossless_walk(parent, tokens, np.zeros((1, 6)), np.array([0.5]), P, q0[None])
    assert res["status"][0] == 4 and res["node_accept"][0, 1] == 0 and res["tested"][0, 2]
    r = np.maximum(p[0] - q0[1], 0.0)
    r /= r.sum()
    assert res["node_p"][0, 2] == pytest.approx(r[tokens[0, 2]], rel=1e-12)
