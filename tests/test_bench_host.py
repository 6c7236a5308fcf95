"""Host-side checks of bench.py's bookkeeping (no GPU): the algorithmic work
formulas against hand-computed values, the acceptance statistics on a hand-made
tree, and that every kernel the bench can name is defined in its source."""
import os
import re

import numpy as np
import pytest

import bench
import synth

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "tree_attention_verification_verify_amd", "csrc")


def test_algorithmic_work_of_the_tiny_chain():
    # B=1, fp32, 4 heads x 64, L=128, chain of 5 nodes, V=1000, sampling:
    # K/V: 2 * 4 * 64 * 4 B * (128 + 5) = 272384; Q + O: 2 * 5 * 4 * 64 * 4 = 10240
    # node i sees 128 + i + 1 keys: 5 * 129 + (0+1+2+3+4) = 655 -> 4 * 4 * 64 * 655 flops
    # logits: 5 target + 4 draft rows of 1000 fp32
    case = synth.make_case(synth.workload("tiny-chain-f32"), with_kv=True)
    w = bench.algorithmic_work(case)
    assert w == dict(attention_bytes=282624, attention_flops=670720, vocab_bytes=36000)


def test_algorithmic_work_of_the_70b_shape():
    # 8 sequences, 8 KV heads x 128 bf16, L = 8192, T = 64 (the 64-node tree: 330 root-path
    # nodes in all, i.e. sum of (depth + 1) over the nodes), 64 query heads, V = 32000
    spec = synth.workload("70b-gqa-medusa")
    case = synth.make_case(spec, with_kv=False)
    case.k_cache = np.zeros((8, 8, spec.kv_capacity, 128), np.uint16)     # only the shape is read
    w = bench.algorithmic_work(case)
    depth_sum = sum(1 + d for d in __import__("oracle").depths(spec.parent))
    assert w["attention_bytes"] == 8 * (2 * 8 * 128 * 2 * (8192 + 64) + 2 * 64 * 64 * 128 * 2)
    assert w["attention_flops"] == 8 * 4 * 64 * 128 * (64 * 8192 + depth_sum)
    assert w["vocab_bytes"] == 8 * 4 * 32000 * 127
    assert abs(w["attention_bytes"] / 1e6 - 287.3) < 0.1 and abs(w["attention_flops"] / 1e9 - 137.5) < 0.1


def test_acceptance_statistics_on_a_hand_made_tree():
    # root -> {1, 2}, 1 -> {3}; node 1 and 3 pass, node 2 fails: path 0-1-3, length 2
    parent = np.array([[-1, 0, 0, 1], [-1, 0, 0, 1]])
    node_accept = np.array([[1, 1, 0, 1], [1, 0, 0, 1]])
    accept_len = np.array([2, 0])
    s = bench.acceptance_stats(parent, node_accept, accept_len)
    assert s["accept_len_histogram"] == {"0": 1, "2": 1}
    assert s["accepted_tokens_per_step"] == 4 and s["mean_accept_len"] == 1.0
    assert s["acceptance_rate"] == 0.5                      # mean length 1 over depth 2
    # depth 1: four children tried under an accepted root, one passed; depth 2: node 3 is
    # tried only where node 1 passed (sequence 0), and passed there
    assert s["nodes_tested_by_depth"] == {"1": 4, "2": 1}
    assert s["conditional_acceptance_by_depth"] == {"1": 0.25, "2": 1.0}


@pytest.mark.parametrize("kname", sorted(bench.KERNEL_SOURCES))
def test_every_named_kernel_is_defined_in_its_source(kname):
    src = open(os.path.join(CSRC, bench.KERNEL_SOURCES[kname])).read()
    assert re.search(r"__global__.*\bvoid\s+%s\s*\(" % kname, src), kname


def test_the_library_names_only_kernels_the_bench_knows():
    # spec_verify_describe returns these names (kernels.h helpers and the attention plan)
    names = set()
    for f in ("spec_verify.hip", "vocab_stats.hip", "lossless_walk.hip"):
        names |= set(re.findall(r'"((?:attn|row_stats)_\w+_kernel|attn_\w+)"', open(os.path.join(CSRC, f)).read()))
    assert names and names <= set(bench.KERNEL_SOURCES), names - set(bench.KERNEL_SOURCES)


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys

    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stdout
