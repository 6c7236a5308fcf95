"""GPU parity of the KV commit (spec_verify_commit) against oracle.commit_kv.

The caches must match bit for bit (data movement only), and the lengths exactly.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_harness import device_inputs, handle_config, note, run_gpu

pytestmark = pytest.mark.gpu


def _gpu_commit(case, path, accept_len, final_node, kv_len=None):
    import torch
    from tree_attention_verification_verify_amd import SpecVerify

    spec = case.spec
    ins = device_inputs(case)
    dev = ins["k_cache"].device
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    kl = t(case.kv_len if kv_len is None else kv_len)
    k0, v0, kl0 = ins["k_cache"].clone(), ins["v_cache"].clone(), kl.clone()
    as_np = lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.cpu().numpy()
    res = []
    # two calls on one handle from the same inputs: the second must repeat the
    # first (the per-sequence counters that order the length update reset)
    with SpecVerify(**handle_config(spec, kv_capacity=case.k_cache.shape[2])) as sv:
        for _ in range(2):
            ins["k_cache"].copy_(k0)
            ins["v_cache"].copy_(v0)
            kl.copy_(kl0)
            sv.commit(ins["k_cache"], ins["v_cache"], kl, t(path), t(accept_len), t(final_node))
            torch.cuda.synchronize()
            res.append((as_np(ins["k_cache"]), as_np(ins["v_cache"]), kl.cpu().numpy()))
    for a, b in zip(res[0], res[1]):
        np.testing.assert_array_equal(a, b)
    return res[1]


def _check(case, path, accept_len, final_node, label, kv_len=None):
    note("%s: commit B=%d T=%d" % (label, case.batch, case.nodes))
    k, v, kl = _gpu_commit(case, path, accept_len, final_node, kv_len)
    L = case.kv_len if kv_len is None else kv_len
    rk, rv, rl = oracle.commit_kv(case.k_cache, case.v_cache, L, path, accept_len, final_node, case.nodes)
    np.testing.assert_array_equal(kl, rl)
    np.testing.assert_array_equal(k, rk)
    np.testing.assert_array_equal(v, rv)
    return rl


def test_commit_with_oracle_paths_bf16():
    spec = synth.workload("70b-gqa-medusa", batch=4, prefix_len=100, vocab=1000, seed=(8, 1))
    case = synth.make_case(spec)
    ref = oracle.verify(case, attention=False)
    rl = _check(case, ref["path"], ref["accept_len"], ref["final_node"], "commit-bf16")
    assert (rl == case.kv_len + ref["accept_len"] + 1).all()


def test_commit_after_a_gpu_run_fp32_and_skipped_sequences():
    spec = synth.workload("tiny-chain-f32", batch=6, seed=(8, 2))
    case = synth.make_case(spec)
    got = run_gpu(case, "commit-run")[0]
    ref = oracle.verify(case, attention=False)
    assert not ref["seq_near"].any()
    np.testing.assert_array_equal(got["path"], ref["path"])
    path, acc, fin = got["path"].copy(), got["accept_len"].copy(), got["final_node"].copy()
    fin[1] = -1                       # void: skipped
    path[2, 1] = 0                    # not a root path: skipped (when accept_len >= 1)
    acc[2] = max(acc[2], 1)
    kv_len = case.kv_len.copy()
    kv_len[3] = spec.kv_capacity - spec.nodes + 1    # no room for the tree: skipped
    rl = _check(case, path, acc, fin, "commit-fp32", kv_len=kv_len)
    assert rl[1] == kv_len[1] and rl[2] == kv_len[2] and rl[3] == kv_len[3]


def test_commit_moves_rows_across_a_medusa_tree():
    # force deep accepted paths through non-first children, so rows really move
    spec = synth.workload("llama7b-medusa-greedy", batch=1, prefix_len=64, vocab=500, seed=(8, 3))
    case = synth.make_case(spec)
    T = case.nodes
    parent = case.parent[0]
    deepest = max(range(T), key=lambda i: (len(oracle.ancestors(parent, i)), i))
    p = oracle.ancestors(parent, deepest)
    path = np.full((1, T), -1, dtype=np.int32)
    path[0, :len(p)] = p
    assert any(p[k] != k for k in range(len(p)))
    _check(case, path, np.array([len(p) - 1]), np.array([deepest]), "commit-tree")


def test_commit_rejects_a_misaligned_cache():
    import torch
    from tree_attention_verification_verify_amd import SpecVerify, SpecVerifyError, spec_verify_commit

    spec = synth.workload("70b-gqa-medusa", batch=1, prefix_len=64, vocab=500, seed=(8, 4))
    case = synth.make_case(spec)
    ins = device_inputs(case)
    flat = ins["k_cache"].reshape(-1)
    bad = flat[1:1 + flat.numel() - 8]
    z = torch.zeros(1, dtype=torch.int32, device=flat.device)
    path = torch.zeros((1, case.nodes), dtype=torch.int32, device=flat.device)
    with SpecVerify(**handle_config(spec)) as sv:
        # the binding's shape check refuses the flat view first ...
        with pytest.raises(SpecVerifyError) as e:
            sv.commit(bad, ins["v_cache"], z.clone(), path, z, z)
        assert e.value.code == -1 and "shape" in str(e.value)
        # ... and without the config the library's own alignment check does
        note("misaligned cache: expect an argument error, no launch")
        with pytest.raises(SpecVerifyError) as e:
            spec_verify_commit(sv.handle, bad, ins["v_cache"], z.clone(), path, z, z)
        assert e.value.code == -1 and "aligned" in str(e.value)
