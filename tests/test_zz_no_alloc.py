"""spec_verify_run_noalloc (the entry point that allocates nothing) against
spec_verify_run on the same inputs, through the C ABI.

Decisions, tokens, paths and statuses must be bit-identical; attention output
within the stated tolerance (2e-2 bf16, 1e-4 fp32), since a shape whose split
partials do not fit the 16 MiB scratch is split fewer times.  Two calls in a
row, the second on a smaller input, then a third on a shape that needs fewer
splits; every call is also checked against the oracle's decisions.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_harness import ATTN_TOL, device_inputs, handle_config, note, run_gpu, to_numpy

pytestmark = pytest.mark.gpu

DECISIONS = ("accept_len", "final_node", "path", "out_tokens", "status", "node_p", "node_q", "node_accept",
             "final_from_residual", "row_token")


def _noalloc(case, label):
    import torch
    from tree_attention_verification_verify_amd import allocate_outputs, make_config, spec_verify_run_noalloc

    spec = case.spec
    cfg = make_config(**handle_config(spec, kv_capacity=case.k_cache.shape[2]))
    note("%s: no-alloc run B=%d T=%d L<=%d V=%d" % (label, case.batch, case.nodes, int(case.kv_len.max()),
                                                    spec.vocab))
    ins = device_inputs(case)
    outs = allocate_outputs(case.batch, case.nodes, spec.hq, spec.head_dim, spec.dtype)
    for v in outs.values():
        v.fill_(0x55 if v.dtype != torch.bfloat16 else 1.0)    # stale contents must all be overwritten
    spec_verify_run_noalloc(cfg, ins, outs)
    torch.cuda.synchronize()
    note("%s: done" % label)
    return to_numpy(outs)


def _same(case, label):
    got = _noalloc(case, label)
    ref = run_gpu(case, label + "-handle")[0]
    for k in DECISIONS:
        np.testing.assert_array_equal(got[k], ref[k], err_msg="%s %s" % (label, k))
    err = float(np.abs(got["attn_out"].astype(np.float64) - ref["attn_out"].astype(np.float64)).max())
    tol = ATTN_TOL[case.spec.dtype]
    print(label, "attn max |no-alloc - run| = %.3g" % err, flush=True)
    assert err <= tol
    ora = oracle.verify(case, attention=False)
    assert not ora["seq_near"].any()
    np.testing.assert_array_equal(got["out_tokens"], ora["out_tokens"])
    np.testing.assert_array_equal(got["accept_len"], ora["accept_len"])
    return got


def test_noalloc_matches_run_on_consecutive_calls():
    # first call: 4 sequences of the 70b-gqa-medusa shape, 64-node trees, 700-slot prefixes (2 splits)
    big = synth.make_case(synth.workload("70b-gqa-medusa", batch=4, prefix_len=700, seed=(31, 7)))
    _same(big, "noalloc-first")
    # second call right after, smaller in every dimension: 2 sequences, 26-node trees, 200 slots, top-p
    small = synth.make_case(synth.workload("70b-gqa-medusa", batch=2, prefix_len=200, tree=synth.inputs.MEDUSA_26,
                                           top_p=0.9, temperature=0.8, seed=(31, 2)))
    _same(small, "noalloc-second-smaller")


def test_noalloc_with_fewer_splits_than_the_handle():
    # one sequence of the 70b-gqa-medusa shape with a 4096-slot prefix: a handle
    # plans 8 splits (17 MB of partials), the scratch holds 7 splits' worth
    case = synth.make_case(synth.workload("70b-gqa-medusa", batch=1, prefix_len=4096, seed=(3, 4096)))
    got = _same(case, "noalloc-fewer-splits")
    ref = oracle.verify(case)
    err = float(np.abs(got["attn_out"].astype(np.float64) - ref["attn_out"]).max())
    print("noalloc-fewer-splits attn max |no-alloc - oracle| = %.3g" % err, flush=True)
    assert err <= ATTN_TOL["bf16"]


def test_noalloc_greedy_fp32_and_valu_shapes():
    _same(synth.make_case(synth.workload("tiny-chain-f32", batch=3, seed=(31, 3))), "noalloc-tiny-f32")
    _same(synth.make_case(synth.workload("llama7b-medusa-greedy", prefix_len=900, seed=(31, 4))),
          "noalloc-greedy-splits")
    _same(synth.make_case(synth.workload("chain-batch32-topp", batch=8, prefix_len=600, ragged=(100, 600),
                                         seed=(31, 5))), "noalloc-valu-topp")
