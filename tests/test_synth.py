"""The seeded input generators: shapes, determinism, tree shapes, bf16 rounding."""
from collections import Counter

import numpy as np
import torch

import oracle
import synth


def _level_counts(parent):
    return [c for _, c in sorted(Counter(oracle.depths(parent)).items())]


def test_medusa_trees_shapes():
    p64, _ = synth.medusa_tree((10, 4, 2, 1, 1), 64)
    assert oracle.check_parent(p64) and len(p64) == 64
    assert _level_counts(p64) == [1, 6, 12, 17, 16, 12]
    p26, _ = synth.medusa_tree((10, 4, 2, 1), 26)
    assert oracle.check_parent(p26) and _level_counts(p26) == [1, 4, 8, 7, 6]


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100_000).astype(np.float32) * 10
    ours = synth.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_cases_are_deterministic_and_well_formed():
    spec = synth.workload("chain-batch32-topp", batch=3, prefix_len=64, ragged=(8, 64))
    a, b = synth.make_case(spec), synth.make_case(spec)
    for f in ("q", "k_cache", "v_cache", "kv_len", "tokens", "target_logits", "draft_logits",
              "u_accept", "u_final"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.k_cache.shape == (3, 32, 64 + 6, 128) and a.k_cache.dtype == np.uint16
    assert ((a.kv_len >= 8) & (a.kv_len <= 64)).all()
    assert (a.u_accept < 1).all() and (a.u_final < 1).all()
    assert ((a.tokens >= 0) & (a.tokens < spec.vocab)).all()


def test_drafted_tokens_lie_in_the_draft_nucleus():
    spec = synth.workload("chain-batch32-topp", batch=2, prefix_len=16, ragged=None, vocab=2000)
    c = synth.make_case(spec, with_kv=False)
    for b in range(2):
        for i in range(1, c.nodes):
            q = oracle.effective_distribution(c.draft_logits[b, i], spec.temperature, spec.top_p)
            assert q[c.tokens[b, i]] > 0


def test_greedy_children_are_distinct_ranked_candidates():
    spec = synth.workload("llama7b-medusa-greedy", prefix_len=16, vocab=500)
    c = synth.make_case(spec, with_kv=False)
    par = c.parent[0]
    for v in range(c.nodes):
        kids = [i for i in range(1, c.nodes) if par[i] == v]
        toks = [int(c.tokens[0, i]) for i in kids]
        assert len(set(toks)) == len(toks)
