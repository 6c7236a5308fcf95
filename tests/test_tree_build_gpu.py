"""GPU parity of the candidate-tree construction (spec_verify_build_tree) against oracle.build_tree.

Tokens and parents are integer outputs: they must match bit for bit, on rows
with many tied logits, infinities, NaN and signed zeros.
"""
import numpy as np
import pytest

import oracle
from gpu_harness import note

pytestmark = pytest.mark.gpu


def _config(B, T, V):
    return dict(max_batch=B, max_nodes=max(T, 1), num_q_heads=8, num_kv_heads=8, head_dim=128,
                kv_capacity=256, vocab=V, dtype="bf16", mode="greedy")


def _run(logits, root, parent_t, rank_t, label):
    import torch
    from tree_attention_verification_verify_amd import SpecVerify

    B, depth, V = logits.shape
    T = len(parent_t)
    note("%s: B=%d depth=%d V=%d T=%d" % (label, B, depth, V, T))
    dev = "cuda"
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(dev)
    rt = torch.from_numpy(np.ascontiguousarray(root, dtype=np.int32)).to(dev)
    par = torch.full((B, T), -9, dtype=torch.int32, device=dev)
    tok = torch.full((B, T), -9, dtype=torch.int32, device=dev)
    res = []
    # two builds on one handle: the second must repeat the first (the per-row
    # counters that join a long row's slices reset)
    with SpecVerify(**_config(B, T, V)) as sv:
        for _ in range(2):
            par.fill_(-9)
            tok.fill_(-9)
            sv.build_tree(lg, rt, list(parent_t), list(rank_t), par, tok)
            torch.cuda.synchronize()
            res.append((par.cpu().numpy(), tok.cpu().numpy()))
    np.testing.assert_array_equal(res[0][0], res[1][0])
    np.testing.assert_array_equal(res[0][1], res[1][1])
    return res[1]


def _check(logits, root, caps, nodes, label):
    parent_t, rank_t = oracle.tree_template(caps, nodes)
    par, tok = _run(logits, root, parent_t, rank_t, label)
    rpar, rtok = oracle.build_tree(logits.astype(np.float64), root, parent_t, rank_t)
    np.testing.assert_array_equal(par, rpar)
    np.testing.assert_array_equal(tok, rtok)
    return tok


@pytest.mark.parametrize("B,caps,nodes,V,step", [
    (8, (10, 4, 2, 1, 1), 64, 32000, 0.125),     # the 70B-shaped GQA tree workload's tree
    (1, (10, 4, 2, 1, 1), 64, 32000, 0.0),
    (16, (10, 4, 2, 1), 26, 128256, 0.25),       # the long-context large-vocab workload's tree
    (3, (2, 2), 7, 1000, 0.5),                   # the printed two-head top-2 tree
    (2, (40,), 33, 5000, 1.0),                   # 32 entries of one list
    (4, (3, 3, 3, 3), 64, 777, 0.0),
    (4, (10, 4, 2, 1, 1), 64, 50257, 0.125),     # odd vocabulary: 8 slices, a ragged last one, scalar rows
])
def test_tree_build_matches_oracle(B, caps, nodes, V, step):
    rng = np.random.default_rng(B * 1000 + V)
    logits = rng.normal(0.0, 3.0, size=(B, len(caps), V)).astype(np.float32)
    if step:
        logits = (np.round(logits / step) * step).astype(np.float32)   # many ties
    root = rng.integers(0, V, size=B)
    _check(logits, root, caps, nodes, "tree-%s-%d" % ("-".join(map(str, caps)), V))


def test_tree_build_special_values_and_tiny_vocab():
    rng = np.random.default_rng(11)
    B, V = 5, 20
    logits = np.round(rng.normal(size=(B, 3, V))).astype(np.float32)
    logits[0, 0, :6] = [np.nan, -np.inf, np.inf, -0.0, 0.0, np.nan]
    logits[1, 1, :] = -np.inf
    logits[2, 2, :] = np.nan
    logits[3, :, :] = 0.0
    logits[3, :, ::3] = -0.0
    root = np.arange(B)
    _check(logits, root, (4, 3, 2), 40, "tree-special")


def _wave_share(n, aligned, waves):
    """Ids (relative to a slice start) that the first `waves` waves of a
    1024-thread workgroup read: thread t takes float4 columns t, t + 1024, ...
    of a 16-byte aligned slice (then the < 4 tail ids one each), or ids t,
    t + 1024, ... of an unaligned one; wave w is threads 64w .. 64w + 63."""
    x = np.arange(n)
    if aligned:
        v4 = n // 4
        thread = np.where(x < 4 * v4, (x // 4) % 1024, (x - 4 * v4) % 1024)
    else:
        thread = x % 1024
    return thread // 64 < waves


def test_tree_build_crowded_row_takes_the_exact_path():
    # Rows split into 8 slices (50257 ids: spans of 6284, the last one 6269).
    # In the first and the last slice of each row, every id that the first 4
    # of the 16 waves read gets +100: over 1500 entries of the slice then pass
    # the first pass's bound (the smallest of the 16 wave maxima), three times
    # what the short list holds, so both slices take the exact fallback, on
    # the 16-byte aligned row 0 and on the unaligned rows alike.
    rng = np.random.default_rng(13)
    B, V, G, CAP = 2, 50257, 8, 512
    span = ((V + G - 1) // G + 3) & ~3
    logits = rng.normal(size=(B, 2, V)).astype(np.float32)
    for b in range(B):
        for d in range(2):
            aligned = ((b * 2 + d) * V) % 4 == 0          # float offset of the row start
            for sl in (0, G - 1):
                lo = sl * span
                n = min(V - lo, span)
                crowd = _wave_share(n, aligned, 4)
                assert crowd.sum() > 3 * CAP
                logits[b, d, lo:lo + n][crowd] += 100.0
    _check(logits, np.array([1, 2]), (16, 16), 60, "tree-crowded")


def test_tree_build_root_only_and_chain():
    rng = np.random.default_rng(12)
    logits = rng.normal(size=(2, 4, 300)).astype(np.float32)
    tok = _check(logits, np.array([7, 8]), (5,), 1, "tree-root-only")
    assert list(tok[:, 0]) == [7, 8]
    _check(logits, np.array([7, 8]), (1, 1, 1, 1), 5, "tree-chain")   # greedy chain: argmax of each row


def test_tree_build_rejects_bad_templates():
    import torch
    from tree_attention_verification_verify_amd import SpecVerify, SpecVerifyError

    B, V = 2, 100
    lg = torch.zeros((B, 2, V), dtype=torch.float32, device="cuda")
    rt = torch.zeros(B, dtype=torch.int32, device="cuda")
    par = torch.zeros((B, 40), dtype=torch.int32, device="cuda")
    tok = torch.zeros((B, 40), dtype=torch.int32, device="cuda")
    with SpecVerify(**_config(B, 40, V)) as sv:
        cases = [([-1, 0, 2], [0, 0, 0], -1),                  # not topological
                 ([0, 0], [0, 0], -1),                          # root with a parent
                 ([-1, 0, 1, 2], [0, 0, 0, 0], -1),             # deeper than the 2 rows given
                 ([-1, 0, 0], [0, 0, -1], -1),                  # negative rank
                 ([-1] + [0] * 33, [0] + list(range(33)), -2)]  # 33 entries of one list
        for p, r, code in cases:
            T = len(p)
            with pytest.raises(SpecVerifyError) as e:
                sv.build_tree(lg, rt, p, r, par[:, :T].contiguous(), tok[:, :T].contiguous())
            assert e.value.code == code, (p, r)
    torch.cuda.synchronize()


def test_built_tree_feeds_a_greedy_verify():
    # the construction's outputs are the verify step's parent/tokens inputs:
    # candidates of depth 1 come from the target's own row of the root, deeper
    # ones from a noisy copy of the target row of the first node one level up,
    # so greedy acceptance reaches past depth 1
    import dataclasses

    import torch
    import synth
    from gpu_harness import compare, device_inputs, handle_config, to_numpy
    from tree_attention_verification_verify_amd import SpecVerify, allocate_outputs

    spec = synth.workload("70b-gqa-medusa", batch=4, prefix_len=300, vocab=3000, mode="greedy", seed=(18, 1))
    case = synth.make_case(spec)
    caps, T = spec.tree[1], spec.tree[2]
    parent_t, rank_t = oracle.tree_template(caps, T)
    np.testing.assert_array_equal(case.parent[0], parent_t)
    depth = oracle.depths(parent_t)
    first = [depth.index(k) for k in range(max(depth) + 1)]
    rng = np.random.default_rng(181)
    rows = [case.target_logits[:, first[k]] + (rng.normal(0.0, 0.5, size=case.target_logits[:, 0].shape) if k else 0.0)
            for k in range(len(caps))]
    cand = np.stack(rows, axis=1).astype(np.float32)
    root = case.tokens[:, 0]
    par_o, tok_o = oracle.build_tree(cand.astype(np.float64), root, parent_t, rank_t)
    case2 = dataclasses.replace(case, parent=par_o.astype(np.int32), tokens=tok_o.astype(np.int32))

    note("tree-then-verify: B=%d T=%d V=%d" % (case.batch, T, spec.vocab))
    ins = device_inputs(case)
    with SpecVerify(**handle_config(spec)) as sv:
        lg = torch.from_numpy(cand).cuda()
        rt = torch.from_numpy(root.astype(np.int32)).cuda()
        sv.build_tree(lg, rt, list(parent_t), list(rank_t), ins["parent"], ins["tokens"])
        outs = allocate_outputs(case.batch, T, spec.hq, spec.head_dim, spec.dtype)
        sv.run(ins, outs)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ins["tokens"].cpu().numpy(), tok_o)
        np.testing.assert_array_equal(ins["parent"].cpu().numpy(), par_o)
        got = to_numpy(outs)
    ref = oracle.verify(case2)
    compare(case2, got, ref)
    assert int(ref["accept_len"].max()) >= 2, ref["accept_len"]
