"""GPU parity of the paged-KV entry points against the oracle's paged reading.

spec_verify_run_paged reads the caches through a block table (fragmented
pools whose unused pages and last-page tails hold NaN, so a read of any slot
outside a node's visible set shows up); every output is compared with
oracle.verify_paged under the same rules as the dense path, and at full size
the paged run must equal the dense run of the same slots bit for bit.
spec_verify_commit_paged must equal oracle.commit_kv_paged bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_harness import compare, device_inputs, handle_config, note, sampled_attention, to_numpy

pytestmark = pytest.mark.gpu

STRICT = dict(accept_band=2e-6, cdf_band=2e-6)


def _act(arr, dtype, dev):
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev)


def _paged_device(paged, dtype, dev="cuda"):
    import torch

    return dict(k_pool=_act(paged.k_pool, dtype, dev), v_pool=_act(paged.v_pool, dtype, dev),
                block_table=torch.from_numpy(np.ascontiguousarray(paged.block_table, dtype=np.int32)).to(dev))


def run_paged(case, paged, label, dense_too=False, lossless_tree=False):
    """Paged run (and optionally the dense run of the same case) on the GPU."""
    import torch
    from tree_attention_verification_verify_amd import SpecVerify, allocate_outputs, paged_kv

    spec = case.spec
    note("%s: upload B=%d T=%d bs=%d pages=%d" % (label, case.batch, case.nodes, paged.block_size,
                                                  paged.num_blocks))
    ins = device_inputs(case)
    pd = _paged_device(paged, spec.dtype)
    pk = paged_kv(pd["k_pool"], pd["v_pool"], pd["block_table"])
    res = {}
    cap = max(case.k_cache.shape[2], paged.capacity)
    with SpecVerify(**handle_config(spec, kv_capacity=cap, lossless_tree=lossless_tree)) as sv:
        outs = allocate_outputs(case.batch, case.nodes, spec.hq, spec.head_dim, spec.dtype)
        paged_ins = {k: v for k, v in ins.items() if k not in ("k_cache", "v_cache")}
        note("%s: paged run" % label)
        sv.run_paged(paged_ins, pk, outs)
        torch.cuda.synchronize()
        res["paged"] = to_numpy(outs)
        if dense_too:
            outs = allocate_outputs(case.batch, case.nodes, spec.hq, spec.head_dim, spec.dtype)
            note("%s: dense run" % label)
            sv.run(ins, outs)
            torch.cuda.synchronize()
            res["dense"] = to_numpy(outs)
    note("%s: done" % label)
    return res


def check_paged(case, paged, label, attn_rows=None, dense_too=False):
    got = run_paged(case, paged, label, dense_too=dense_too)
    ref = oracle.verify_paged(case, paged, **STRICT) if attn_rows is None else \
        oracle.verify(case, attention=False, **STRICT)
    stats = compare(case, got["paged"], ref, attn=True, attn_rows=attn_rows)
    print(label, stats, flush=True)
    return got, ref


@pytest.mark.parametrize("name,bs,kw", [
    ("tiny-chain-f32", 16, dict(batch=3, ragged=(40, 128), seed=(16, 1))),
    ("chain-batch32-topp", 32, dict(batch=4, prefix_len=500, ragged=(60, 500), seed=(16, 2))),
    ("70b-gqa-medusa", 16, dict(batch=2, prefix_len=333, seed=(16, 3))),
    ("70b-gqa-medusa", 64, dict(batch=3, prefix_len=700, ragged=(100, 700), mode="greedy", seed=(16, 4))),
    ("llama7b-medusa-greedy", 128, dict(prefix_len=450, seed=(16, 5))),
    ("longctx-bigvocab", 16, dict(batch=2, prefix_len=400, seed=(16, 6))),
])
def test_paged_matches_oracle(name, bs, kw):
    case = synth.make_case(synth.workload(name, **kw))
    case, paged = synth.page_case(case, bs, seed=kw["seed"])
    got, ref = check_paged(case, paged, "paged-%s-bs%d" % (name, bs))
    assert (got["paged"]["status"] & 8 == 0).all()
    assert np.isfinite(got["paged"]["attn_out"]).all()


def test_paged_tiled_valu_with_prefix_splits():
    # one sequence, long prefix, few rows: the tiled VALU kernel over several splits, through the table
    spec = synth.CaseSpec("valu-split", 2, "bf16", 4, 4, 128, 2500, 500, "sampling", ("chain", 5),
                          ragged=(1500, 2500), seed=(16, 11))
    case, paged = synth.page_case(synth.make_case(spec), 16, seed=(16, 11))
    got, ref = check_paged(case, paged, "paged-valu-split")
    assert np.isfinite(got["paged"]["attn_out"]).all()


def test_paged_shared_prefix_pages():
    spec = synth.workload("70b-gqa-medusa", batch=3, prefix_len=300, ragged=(200, 300), seed=(16, 7))
    case, paged = synth.page_case(synth.make_case(spec), 32, share_prefix_pages=4, seed=(16, 7))
    assert (paged.block_table[1:, :4] == paged.block_table[0, :4]).all()
    check_paged(case, paged, "paged-shared-prefix")


def test_paged_bad_entries_flag_status_and_zero_attention():
    spec = synth.workload("70b-gqa-medusa", batch=4, prefix_len=200, vocab=2000, ragged=(100, 200), seed=(16, 8))
    case, paged = synth.page_case(synth.make_case(spec), 16, seed=(16, 8))
    table = paged.block_table.copy()
    L = case.kv_len
    used3 = -(-(int(L[3]) + case.nodes) // 16)
    assert used3 < table.shape[1]
    table[1, 3] = paged.num_blocks                  # a prefix page past the pool
    table[2, (L[2] + case.nodes - 1) // 16] = -1     # the page of the last tree slot
    table[3, used3:] = -7                            # past the slots in use: never read, fine
    import dataclasses
    paged = dataclasses.replace(paged, block_table=table)
    got, ref = check_paged(case, paged, "paged-bad-entries")
    st = got["paged"]["status"]
    assert list(st & 8) == [0, 8, 8, 0]
    for b in (1, 2):
        assert (got["paged"]["attn_out"][b] == 0).all()
    assert np.isfinite(got["paged"]["attn_out"][[0, 3]]).all()


def test_paged_full_size_gqa_medusa_equals_dense():
    # the 70B-shaped GQA tree workload at full size, pages of 16 slots: the
    # paged run must give the dense run's outputs bit for bit, and sampled
    # attention rows match the oracle
    spec = synth.workload("70b-gqa-medusa")
    case = synth.make_case(spec)
    rows = sampled_attention(case, [(0, 0, 0), (3, 63, 17), (7, 40, 63), (5, 9, 30)])
    case, paged = synth.page_case(case, 16, seed=(16, 9))
    got, ref = check_paged(case, paged, "paged-gqa-medusa-full", attn_rows=rows, dense_too=True)
    for k, v in got["dense"].items():
        np.testing.assert_array_equal(got["paged"][k], v, err_msg=k)


@pytest.mark.parametrize("name,kw", [
    ("70b-gqa-medusa", dict(batch=2, prefix_len=333, seed=(16, 11))),                        # MFMA kernel
    ("chain-batch32-topp", dict(batch=2, prefix_len=301, ragged=(150, 301), seed=(16, 12))),  # tiled VALU kernel
])
def test_paged_pool_beyond_4gib_equals_small_pool(name, kw):
    # a pool spanning more than 4 GiB takes the per-page buffer resources for
    # every block (a pool under 4 GiB reads whole blocks through one resource
    # with the page in the scalar offset): the same pages moved to the top of
    # a 4 GiB + pool must give the small pool's outputs bit for bit
    import torch
    from tree_attention_verification_verify_amd import SpecVerify, allocate_outputs, paged_kv

    spec = synth.workload(name, **kw)
    case, paged = synth.page_case(synth.make_case(spec), 16, seed=kw["seed"])
    small = _paged_device(paged, spec.dtype)
    nb, hkv, bs, d = paged.k_pool.shape
    page_bytes = hkv * bs * d * 2
    top = (1 << 32) // page_bytes + 1            # pages below the moved ones
    note("paged-4gib: pool of %d pages (%.2f GiB per operand)" % (top + nb, (top + nb) * page_bytes / 2 ** 30))
    big_k = torch.empty((top + nb, hkv, bs, d), dtype=torch.bfloat16, device="cuda")
    big_v = torch.empty_like(big_k)
    big_k[top:] = small["k_pool"]
    big_v[top:] = small["v_pool"]
    table = small["block_table"].clone()
    table[table >= 0] += top
    ins = {k: v for k, v in device_inputs(case).items() if k not in ("k_cache", "v_cache")}
    got = {}
    with SpecVerify(**handle_config(spec, kv_capacity=max(case.k_cache.shape[2], paged.capacity))) as sv:
        for name, pk in (("small", paged_kv(small["k_pool"], small["v_pool"], small["block_table"])),
                         ("big", paged_kv(big_k, big_v, table))):
            outs = allocate_outputs(case.batch, case.nodes, spec.hq, spec.head_dim, spec.dtype)
            note("paged-4gib: %s pool run" % name)
            sv.run_paged(ins, pk, outs)
            torch.cuda.synchronize()
            got[name] = to_numpy(outs)
    assert (got["big"]["status"] == 0).all()
    for k, v in got["small"].items():
        np.testing.assert_array_equal(got["big"][k], v, err_msg=k)
    del big_k, big_v
    torch.cuda.empty_cache()


def test_paged_with_the_lossless_tree_rule():
    spec = synth.workload("70b-gqa-medusa", batch=3, prefix_len=260, vocab=4000, ragged=(120, 260), seed=(16, 10))
    case, paged = synth.page_case(synth.make_case(spec), 32, seed=(16, 10))
    got = run_paged(case, paged, "paged-lossless", lossless_tree=True)
    ref = oracle.verify_paged(case, paged, rule="lossless", **STRICT)
    stats = compare(case, got["paged"], ref, attn=True, rule="lossless")
    print("paged-lossless", stats, flush=True)


# ------------------------------------------------------------------ commit through the table

def _gpu_commit_paged(case, paged, path, accept_len, final_node):
    import torch
    from tree_attention_verification_verify_amd import SpecVerify, paged_kv

    spec = case.spec
    pd = _paged_device(paged, spec.dtype)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")
    kl = t(case.kv_len)
    with SpecVerify(**handle_config(spec, kv_capacity=max(paged.capacity, case.k_cache.shape[2]))) as sv:
        sv.commit_paged(paged_kv(pd["k_pool"], pd["v_pool"], pd["block_table"]), kl, t(path), t(accept_len),
                        t(final_node))
        torch.cuda.synchronize()
    as_np = lambda x: (x.view(torch.int16).cpu().numpy().view(np.uint16) if x.dtype == torch.bfloat16
                       else x.cpu().numpy())
    return as_np(pd["k_pool"]), as_np(pd["v_pool"]), kl.cpu().numpy()


@pytest.mark.parametrize("name,bs,kw", [
    ("70b-gqa-medusa", 16, dict(batch=4, prefix_len=100, vocab=1000, seed=(17, 1))),
    ("tiny-chain-f32", 32, dict(batch=5, ragged=(30, 128), seed=(17, 2))),
])
def test_paged_commit_matches_oracle(name, bs, kw):
    case = synth.make_case(synth.workload(name, **kw))
    case, paged = synth.page_case(case, bs, seed=kw["seed"])
    ref = oracle.verify(case, attention=False)
    path, acc, fin = ref["path"].copy(), ref["accept_len"].copy(), ref["final_node"].copy()
    # a deep path through later siblings, so rows move across pages
    T = case.nodes
    deepest = max(range(T), key=lambda i: (len(oracle.ancestors(case.parent[0], i)), i))
    p = oracle.ancestors(case.parent[0], deepest)
    path[0] = -1
    path[0, :len(p)] = p
    acc[0], fin[0] = len(p) - 1, deepest
    table = paged.block_table.copy()
    table[1, 0] = -1                                  # leaves the pool: sequence 1 skipped
    import dataclasses
    paged = dataclasses.replace(paged, block_table=table)
    note("paged-commit-%s: B=%d bs=%d" % (name, case.batch, bs))
    k, v, kl = _gpu_commit_paged(case, paged, path, acc, fin)
    rk, rv, rl = oracle.commit_kv_paged(paged.k_pool, paged.v_pool, paged.block_table, case.kv_len, path, acc,
                                        fin, T, bs, paged.capacity)
    np.testing.assert_array_equal(kl, rl)
    assert rl[1] == case.kv_len[1] and rl[0] == case.kv_len[0] + len(p)
    np.testing.assert_array_equal(k, rk)
    np.testing.assert_array_equal(v, rv)


def test_paged_arguments_are_checked():
    import torch
    from tree_attention_verification_verify_amd import SpecVerify, SpecVerifyError, allocate_outputs, paged_kv

    spec = synth.workload("70b-gqa-medusa", batch=1, prefix_len=64, vocab=500, seed=(17, 3))
    case, paged = synth.page_case(synth.make_case(spec), 16, seed=(17, 3))
    ins = device_inputs(case)
    pd = _paged_device(paged, spec.dtype)
    outs = allocate_outputs(1, case.nodes, spec.hq, spec.head_dim, spec.dtype)
    with SpecVerify(**handle_config(spec, kv_capacity=paged.capacity)) as sv:
        good = paged_kv(pd["k_pool"], pd["v_pool"], pd["block_table"])
        for field, value in [("block_size", 24), ("block_size", 8), ("num_blocks", 0), ("table_width", 0),
                             ("table_width", paged.block_table.shape[1] + 1)]:
            bad = paged_kv(pd["k_pool"], pd["v_pool"], pd["block_table"])
            setattr(bad, field, value)
            with pytest.raises(SpecVerifyError) as e:
                sv.run_paged(ins, bad, outs)
            assert e.value.code == -1, field
        bad = paged_kv(pd["k_pool"], pd["v_pool"], pd["block_table"])
        bad.k_pool = good.k_pool + 2
        with pytest.raises(SpecVerifyError):
            sv.run_paged(ins, bad, outs)
        torch.cuda.synchronize()
