"""Pins for the candidate-tree construction oracle (oracle.tree_build).

* P4's printed example ("Tree Attention验证"): two heads, top-2 each, give the
  7-node Cartesian-product tree whose mask is the printed 7x7 matrix, and the
  level-2 nodes take head 2's two best tokens under every level-1 node.
* Any full product: the root paths are exactly every rank tuple, once.
* The workload trees' level counts, [1, 6, 12, 17, 16, 12] (caps 10/4/2/1/1,
  64 nodes) and [1, 4, 8, 7, 6] (caps 10/4/2/1, 26 nodes), derived separately
  when the workloads were fixed.
* Top-k order against a plain repeated-maximum loop on tie-heavy rows with
  -inf and NaN, and against numpy's stable argsort on finite rows.
* Tokens of every node against a brute-force sort of its row.
The pruning rule itself is a reading (no rule on the pages): beyond the
full-product case it is pinned only by these invariants ("parity unpinned").
"""
import itertools
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _p4_mask():
    rows = []
    for line in open(os.path.join(GOLDEN, "p4_tree_mask_7x7.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append([int(x) for x in line.split()])
    return np.array(rows)


def test_p4_two_heads_top2_is_the_printed_tree():
    parent, rank = oracle.tree_template([2, 2], 7)
    assert list(parent) == [-1, 0, 0, 1, 1, 2, 2]
    assert list(rank) == [0, 0, 1, 0, 1, 0, 1]
    np.testing.assert_array_equal(oracle.tree_mask(parent), _p4_mask())
    # head 1 ranks tokens 7 > 3 > ..., head 2 ranks 5 > 9 > ...: A=1, B=7, C=3, D=F=5, E=G=9
    V = 12
    logits = np.zeros((1, 2, V))
    logits[0, 0, 7], logits[0, 0, 3] = 4.0, 2.0
    logits[0, 1, 5], logits[0, 1, 9] = 3.0, 1.0
    par, tok = oracle.build_tree(logits, np.array([1]), parent, rank)
    assert list(tok[0]) == [1, 7, 3, 5, 9, 5, 9]
    assert list(par[0]) == [-1, 0, 0, 1, 1, 2, 2]


@pytest.mark.parametrize("caps", [(3, 2), (2, 2, 2), (4,), (1, 3, 2), (2, 1, 1, 2)])
def test_full_product_has_every_rank_tuple_once(caps):
    n = 1 + sum(int(np.prod(caps[:d])) for d in range(1, len(caps) + 1))
    parent, rank = oracle.tree_template(caps, n)
    paths = set()
    for i in range(1, n):
        anc = oracle.ancestors(parent, i)
        paths.add(tuple(int(rank[j]) for j in anc[1:]))
    expect = set()
    for d in range(1, len(caps) + 1):
        expect |= set(itertools.product(*[range(c) for c in caps[:d]]))
    assert paths == expect and len(paths) == n - 1
    with pytest.raises(ValueError):
        oracle.tree_template(caps, n + 1)


@pytest.mark.parametrize("caps,nodes,levels", [
    ((10, 4, 2, 1, 1), 64, [1, 6, 12, 17, 16, 12]),
    ((10, 4, 2, 1), 26, [1, 4, 8, 7, 6]),
])
def test_workload_tree_level_counts(caps, nodes, levels):
    parent, rank = oracle.tree_template(caps, nodes)
    d = oracle.depths(parent)
    assert [d.count(k) for k in range(max(d) + 1)] == levels


@pytest.mark.parametrize("caps,nodes", [((10, 4, 2, 1, 1), 64), ((10, 4, 2, 1), 26), ((3, 3, 3), 20),
                                        ((5, 5), 9), ((2, 2), 4), ((6,), 1)])
def test_template_invariants(caps, nodes):
    parent, rank = oracle.tree_template(caps, nodes)
    assert oracle.check_parent(parent)
    d = oracle.depths(parent)
    assert all(d[i] <= d[i + 1] for i in range(nodes - 1))           # level order
    for i in range(1, nodes):
        assert 0 <= rank[i] < caps[d[i] - 1]
        sib = [j for j in range(1, nodes) if parent[j] == parent[i]]
        assert sib == list(range(sib[0], sib[0] + len(sib)))          # siblings adjacent
        assert [int(rank[j]) for j in sib] == sorted(int(rank[j]) for j in sib)
        # a kept node's smaller-ranked siblings are kept too
        assert [int(rank[j]) for j in sib] == list(range(len(sib)))


def _topk_loop(row, k):
    left = list(range(len(row)))
    out = []

    def better(a, b):   # does id a rank before id b?
        va, vb = row[a], row[b]
        if np.isnan(va) or np.isnan(vb):
            return (not np.isnan(va)) or (np.isnan(va) and np.isnan(vb) and a < b)
        return va > vb or (va == vb and a < b)

    for _ in range(k):
        best = left[0]
        for j in left[1:]:
            if better(j, best):
                best = j
        out.append(best)
        left.remove(best)
    return out


def test_topk_order_on_ties_infinities_and_nan():
    rng = np.random.default_rng(5)
    for _ in range(30):
        V = int(rng.integers(5, 60))
        row = np.round(rng.normal(size=V) * 2) / 2          # many ties
        for j in rng.choice(V, size=3, replace=False):
            row[j] = rng.choice([-np.inf, np.inf, np.nan])
        k = int(rng.integers(1, V + 1))
        assert list(oracle.topk_ids(row, k)) == _topk_loop(row, k)


def test_topk_matches_stable_argsort_on_finite_rows():
    rng = np.random.default_rng(6)
    row = np.round(rng.normal(size=5000) * 8) / 8
    np.testing.assert_array_equal(oracle.topk_ids(row, 40), np.argsort(-row, kind="stable")[:40])


def test_tokens_follow_each_nodes_row_and_rank():
    rng = np.random.default_rng(7)
    caps, nodes = (10, 4, 2, 1), 26
    parent, rank = oracle.tree_template(caps, nodes)
    B, V = 3, 300
    logits = np.round(rng.normal(size=(B, len(caps), V)) * 4) / 4
    root = rng.integers(0, V, size=B)
    par, tok = oracle.build_tree(logits, root, parent, rank)
    d = oracle.depths(parent)
    for b in range(B):
        assert tok[b, 0] == root[b]
        for i in range(1, nodes):
            order = sorted(range(V), key=lambda j: (-logits[b, d[i] - 1, j], j))
            assert tok[b, i] == order[rank[i]]
        assert (par[b] == parent).all()
