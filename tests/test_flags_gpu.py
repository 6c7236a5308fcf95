"""GPU tests of the run flags: the probability-row debug output, running one
half of the step alone, and the lossless walk's give-up path.

probs rows are compared with the oracle's effective distributions (relative
error <= 1e-4, exact zeros outside the nucleus); the skip flags must leave the
outputs of the part that runs bit-identical to a full run.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_harness import PROB_RTOL, device_inputs, handle_config, note, run_gpu, to_numpy

pytestmark = pytest.mark.gpu

DECISIONS = ("accept_len", "final_node", "path", "out_tokens", "status", "node_p", "node_q", "node_accept",
             "final_from_residual", "row_token")


def _run(case, label, **flags):
    import torch
    from tree_attention_verification_verify_amd import SpecVerify, allocate_outputs

    spec = case.spec
    note("%s: B=%d T=%d V=%d flags=%s" % (label, case.batch, case.nodes, spec.vocab, sorted(flags)))
    ins = device_inputs(case)
    cfg = handle_config(spec, kv_capacity=case.k_cache.shape[2])
    cfg.update(flags)
    outs = allocate_outputs(case.batch, case.nodes, spec.hq, spec.head_dim, spec.dtype,
                            vocab=spec.vocab if flags.get("write_probs") else None)
    if flags.get("skip_attention"):
        for k in ("q", "k_cache", "v_cache"):
            ins[k] = None
        outs["attn_out"] = None
    if flags.get("skip_vocab"):
        for k in ("tokens", "target_logits", "draft_logits", "u_accept", "u_final"):
            ins[k] = None
        outs = dict(attn_out=outs["attn_out"])
    with SpecVerify(**cfg) as sv:
        sv.run(ins, outs)
        torch.cuda.synchronize()
    note("%s: done" % label)
    return to_numpy({k: v for k, v in outs.items() if v is not None})


@pytest.mark.parametrize("name,kw", [
    ("70b-gqa-medusa", dict(batch=2, prefix_len=96, seed=(21, 1))),
    ("chain-batch32-topp", dict(batch=3, prefix_len=200, ragged=None, seed=(21, 2))),     # top-p 0.9, tau 0.8
    ("longctx-bigvocab", dict(batch=2, prefix_len=64, seed=(21, 3))),                      # V = 128256, tau 0.7
    ("longctx-bigvocab", dict(batch=2, prefix_len=64, top_p=0.8, seed=(21, 4))),           # streamed top-p cut
    ("tiny-chain-f32", dict(batch=2, seed=(21, 5))),                     # statistics in the attention launch
    ("llama7b-medusa-greedy", dict(mode="sampling", prefix_len=300, seed=(21, 6))),        # the same, MFMA
])
def test_write_probs_rows_match_the_oracle(name, kw):
    case = synth.make_case(synth.workload(name, **kw))
    got = _run(case, "probs-" + name, write_probs=True)
    ref = oracle.verify(case, attention=False)
    p = ref["p_rows"]
    g = got["probs"].astype(np.float64)
    big = p >= 1e-30
    rel = np.abs(g[big] - p[big]) / p[big]
    print(name, "probs max rel err %.3g over %d values" % (rel.max(), big.sum()), flush=True)
    assert rel.max() <= PROB_RTOL
    assert (g[~big] == 0).all()
    # outside the nucleus exactly zero, inside positive: the same kept set
    np.testing.assert_array_equal(g > 0, p > 0)
    # the acceptance test reads the same value: probs[b, parent(i), x_i] == node_p[b, i]
    B, T = case.batch, case.nodes
    for b in range(B):
        for i in range(1, T):
            assert got["probs"][b, case.parent[b, i], case.tokens[b, i]] == got["node_p"][b, i], (b, i)


@pytest.mark.parametrize("name,kw", [
    ("70b-gqa-medusa", dict(batch=2, prefix_len=500, seed=(22, 1))),                     # MFMA, prefix splits
    ("chain-batch32-topp", dict(batch=4, prefix_len=300, ragged=(100, 300), seed=(22, 2))),  # tiled VALU
    ("tiny-chain-f32", dict(batch=3, seed=(22, 3))),                                       # fp32 VALU
])
def test_skip_flags_leave_the_other_half_bit_identical(name, kw):
    case = synth.make_case(synth.workload(name, **kw))
    full = run_gpu(case, "full-" + name)[0]
    vocab_only = _run(case, "skip-attention-" + name, skip_attention=True)
    attn_only = _run(case, "skip-vocab-" + name, skip_vocab=True)
    for k in DECISIONS:
        np.testing.assert_array_equal(vocab_only[k], full[k], err_msg=k)
    np.testing.assert_array_equal(attn_only["attn_out"], full["attn_out"])
    # and the full run is the oracle's
    ref = oracle.verify(case)
    assert not ref["seq_near"].any()
    np.testing.assert_array_equal(full["out_tokens"], ref["out_tokens"])


@pytest.mark.parametrize("name,kw", [
    ("tiny-chain-f32", dict(batch=2, seed=(24, 1))),                              # tiled VALU attention
    ("llama7b-medusa-greedy", dict(prefix_len=900, seed=(24, 2))),                # MFMA, prefix splits
    ("llama7b-medusa-greedy", dict(mode="sampling", prefix_len=300, seed=(24, 3))),
    ("70b-gqa-medusa", dict(mode="greedy", prefix_len=256, seed=(24, 5))),        # two rows per workgroup after
    ("70b-gqa-medusa", dict(mode="greedy", prefix_len=1000, seed=(24, 4))),       # the attention grid
])
def test_row_statistics_inside_the_attention_launch(name, kw):
    """The attention launch carries the row statistics (beside a small
    attention grid, or after one that fills the GPU); a timing handle keeps
    them apart.  Both give the same outputs bit for bit."""
    import json
    import torch
    from tree_attention_verification_verify_amd import SpecVerify

    case = synth.make_case(synth.workload(name, **kw))
    cfg = handle_config(case.spec, kv_capacity=case.k_cache.shape[2])
    with torch.cuda.device(0):
        with SpecVerify(**cfg) as sv:
            plan = sv.describe(case.batch, case.nodes)
        with SpecVerify(**dict(cfg, timing=True)) as sv:
            tplan = sv.describe(case.batch, case.nodes)
    plan = plan if isinstance(plan, dict) else json.loads(plan)
    tplan = tplan if isinstance(tplan, dict) else json.loads(tplan)
    assert plan["vocab_in_attention_launch"] == 1 and tplan["vocab_in_attention_launch"] == 0, (plan, tplan)
    fused = run_gpu(case, "fused-" + name)[0]
    apart = _run(case, "apart-" + name, timing=True)
    for k in DECISIONS + ("attn_out",):
        np.testing.assert_array_equal(fused[k], apart[k], err_msg=k)
    ref = oracle.verify(case, attention=False)
    assert not ref["seq_near"].any()
    np.testing.assert_array_equal(fused["out_tokens"], ref["out_tokens"])


def test_lossless_walk_gives_up_without_hanging():
    """Waits of the walk across workgroups that give up at once (a test-only
    flag): every kernel ends, a sequence whose workgroups were not all there
    is flagged with status bit 16, any other sequence has the normal outputs."""
    spec = synth.workload("70b-gqa-medusa", batch=4, prefix_len=64, seed=(23, 1))   # 8 workgroups per sequence
    case = synth.make_case(spec)
    normal = run_gpu(case, "walk-normal", lossless_tree=True)[0]
    ref = oracle.verify(case, rule="lossless", attention=False)
    assert not ref["seq_near"].any()
    np.testing.assert_array_equal(normal["out_tokens"], ref["out_tokens"])
    assert not (normal["status"] & 16).any()
    flagged = 0
    for r in range(3):
        got = _run(case, "walk-no-wait-%d" % r, lossless_tree=True, walk_no_wait=True)
        for b in range(case.batch):
            if got["status"][b] & 16:
                flagged += 1
                continue
            for k in ("accept_len", "final_node", "path", "out_tokens", "status"):
                np.testing.assert_array_equal(got[k][b], normal[k][b], err_msg="%s b=%d" % (k, b))
    print("sequences flagged with bit 16: %d of %d" % (flagged, 3 * case.batch), flush=True)
    assert flagged > 0
    # the GPU and a fresh handle are fine afterwards
    again = run_gpu(case, "walk-normal-again", lossless_tree=True)[0]
    for k in DECISIONS:
        np.testing.assert_array_equal(again[k], normal[k], err_msg=k)
