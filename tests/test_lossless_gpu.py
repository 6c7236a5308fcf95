"""GPU parity of the lossless sibling walk (SPEC_VERIFY_FLAG_LOSSLESS_TREE) against oracle.lossless.

Every case runs the whole step through the C ABI with the flag set; the
oracle takes the same walk in float64.  Decisions, paths and tokens must match
bit for bit except near-ties (then the whole sequence is excluded: which nodes
are tested depends on earlier decisions).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_harness import compare, note, run_gpu, sampled_attention

pytestmark = pytest.mark.gpu

STRICT = dict(accept_band=2e-6, cdf_band=2e-6)


def check(case, label, attn_rows=None):
    got = run_gpu(case, label, lossless_tree=True)[0]
    ref = oracle.verify(case, attention=attn_rows is None, rule="lossless", **STRICT)
    stats = compare(case, got, ref, attn=True, attn_rows=attn_rows, rule="lossless")
    tested = int(ref["tested"].sum())
    rejected = int((ref["tested"] & (ref["node_accept"] == 0)).sum())
    print(label, stats, "tested", tested, "rejected", rejected, flush=True)
    assert stats["seq_near"] < max(2, case.batch // 4)
    return got, ref, stats


def test_lossless_chain_equals_independent_rule_on_gpu():
    case = synth.make_case(synth.workload("tiny-chain-f32", batch=16, seed=(7, 1)))
    a = run_gpu(case, "chain-independent")[0]
    b, ref, _ = check(case, "chain-lossless")
    for k in ("status", "accept_len", "final_node", "path", "out_tokens", "final_from_residual"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_lossless_gqa_medusa_tree_short_prefix():
    spec = synth.workload("70b-gqa-medusa", batch=4, prefix_len=256, vocab=4000, seed=(7, 2))
    check(synth.make_case(spec), "lossless-gqa-tree")


def test_lossless_many_seeds_and_rejections():
    # broad draft noise: many rejected siblings, several residual passes per node
    for s in range(3):
        spec = synth.workload("70b-gqa-medusa", batch=8, prefix_len=64, vocab=2000, draft_sigma=2.5,
                              seed=(7, 3, s))
        _, ref, _ = check(synth.make_case(spec), "lossless-seed%d" % s)
        assert (ref["tested"] & (ref["node_accept"] == 0)).sum(axis=1).max() >= 3


def test_lossless_streamed_vocab():
    # vocab above one on-chip chunk (32768): residual rows and the draw stream through the workspace
    spec = synth.workload("longctx-bigvocab", batch=2, prefix_len=128, vocab=40000, seed=(7, 4))
    check(synth.make_case(spec), "lossless-big-vocab")
    # and with a top-p cut taken over the streamed rows
    spec = synth.workload("longctx-bigvocab", batch=2, prefix_len=128, vocab=40000, top_p=0.9, seed=(7, 41))
    check(synth.make_case(spec), "lossless-big-vocab-topp")


@pytest.mark.parametrize("batch,vocab", [(72, 32000), (16, 140000)])
def test_lossless_grids_too_large_for_the_workgroup_walk(batch, vocab):
    # batch * ceil(V / 4096) above two workgroups per CU: one workgroup per
    # sequence instead (r in registers up to 32768 ids, in HBM rows above)
    spec = synth.CaseSpec("walk-fallback", batch, "bf16", 8, 2, 64, 64, vocab, "sampling", ("medusa", (3, 2), 9),
                          temperature=1.0, draft_sigma=2.0, seed=(7, 9, vocab))
    _, ref, _ = check(synth.make_case(spec), "lossless-fallback-V%d" % vocab)
    assert (ref["tested"] & (ref["node_accept"] == 0)).sum() > batch


def test_lossless_largest_vocabulary():
    # 4194304 ids: 1024 workgroups of 4096 would not fit the GPU twice over,
    # so the streamed one-workgroup kernel runs (128 chunks per pass); logits
    # peaked on 40 ids keep the top-p cut far from the near-tie band
    rng = np.random.default_rng(7)
    spec = synth.CaseSpec("max-vocab", 1, "bf16", 8, 2, 64, 64, 4194304, "sampling", ("medusa", (2, 2), 5),
                          temperature=1.0, top_p=0.9, seed=(7, 4194304))
    case = synth.make_case(spec)
    hot = rng.choice(spec.vocab, size=40, replace=False)
    case.target_logits[:] = -30.0
    case.draft_logits[:] = -30.0
    z = rng.normal(0.0, 2.0, size=(1, case.nodes, hot.size)).astype(np.float32)
    case.target_logits[:, :, hot] = z
    case.draft_logits[:, :, hot] = z + rng.normal(0.0, 1.5, size=z.shape).astype(np.float32)
    case.tokens[:, 1:] = rng.choice(hot, size=(1, case.nodes - 1))
    _, ref, _ = check(case, "lossless-max-vocab")
    assert not ref["seq_near"].any() and int(ref["tested"].sum()) >= 2


def test_lossless_tree_with_temperature_and_top_p():
    spec = synth.workload("70b-gqa-medusa", batch=4, prefix_len=128, vocab=3000, temperature=0.8, top_p=0.9,
                          seed=(7, 5))
    check(synth.make_case(spec), "lossless-topp")


def test_lossless_forced_uniforms():
    spec = synth.workload("70b-gqa-medusa", batch=4, prefix_len=64, vocab=1500, seed=(7, 6))
    case = synth.make_case(spec)
    case.u_accept[:2] = 0.0                    # every child with r(x) > 0 passes: first children to a leaf
    case.u_accept[2:] = np.float32(0.999999)   # nearly every test fails: all siblings of the root rejected
    got, ref, _ = check(case, "lossless-forced")
    assert (ref["accept_len"][:2] > 0).all()


def test_lossless_full_size_70b_sampled_attention():
    spec = synth.workload("70b-gqa-medusa")
    note("building the full-size 70b-gqa-medusa case")
    case = synth.make_case(spec)
    picks = [(0, 0, 0), (3, 17, 40), (7, 63, 63)]
    check(case, "lossless-70b-full", attn_rows=sampled_attention(case, picks))
