"""The Medusa workload trees against their stored parent[] arrays.

Three separate implementations of one pruning rule must give the stored
trees: the oracle's enumeration (oracle.tree_template), the input generator's
(synth.medusa_tree) and the library's best-first search
(spec_verify_tree_template, host only: no GPU needed).
"""
import json
import os

import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "medusa_trees.json")
TREES = json.load(open(GOLDEN, encoding="utf-8"))["trees"]


def _levels(parent):
    d = oracle.depths(parent)
    return [d.count(k) for k in range(max(d) + 1)]


@pytest.mark.parametrize("tree", TREES, ids=lambda t: "T%d" % t["nodes"])
def test_stored_tree_is_consistent(tree):
    assert oracle.check_parent(tree["parent"]) and len(tree["parent"]) == tree["nodes"]
    assert _levels(tree["parent"]) == tree["level_counts"]


@pytest.mark.parametrize("tree", TREES, ids=lambda t: "T%d" % t["nodes"])
def test_oracle_template_gives_the_stored_tree(tree):
    parent, _ = oracle.tree_template(tree["caps"], tree["nodes"])
    assert list(parent) == tree["parent"]


@pytest.mark.parametrize("tree", TREES, ids=lambda t: "T%d" % t["nodes"])
def test_input_generator_gives_the_stored_tree(tree):
    parent, _ = synth.medusa_tree(tuple(tree["caps"]), tree["nodes"])
    assert list(parent) == tree["parent"]
    # the workloads use these trees
    specs = [s for s in synth.WORKLOADS.values() if s.tree[0] == "medusa" and s.tree[2] == tree["nodes"]]
    assert specs and all(list(s.parent) == tree["parent"] for s in specs)


@pytest.mark.parametrize("tree", TREES, ids=lambda t: "T%d" % t["nodes"])
def test_library_template_gives_the_stored_tree(tree):
    import tree_attention_verification_verify_amd as sva

    parent, _ = sva.spec_verify_tree_template(tree["caps"], tree["nodes"])
    assert list(parent) == tree["parent"]
