"""Pins for the paged KV reading (oracle.paged), each against something other than itself.

* A hand-written table and a pool whose entries encode (page, head, row): the
  slots gathered through the table are checked against values worked out by
  hand.
* Attention and commit through a fragmented table equal the dense oracle's
  (pinned in test_oracle_pins.py / test_commit_pins.py) on the same slots;
  unused pages and the tail rows of the last page hold NaN, so a read of any
  slot outside a node's visible set would show.
* Entries of the slots in use outside the pool flag status 8; entries past
  the slots in use are never read.
* Sequences sharing prefix pages give the dense result of the shared prefix.
"""
import numpy as np
import pytest

import oracle
import synth


def _pool_codes(nb, hkv, bs, d):
    pool = np.zeros((nb, hkv, bs, d), dtype=np.float32)
    for p in range(nb):
        for h in range(hkv):
            for r in range(bs):
                pool[p, h, r, :] = 1000 * p + 100 * h + r
    return pool


def test_gathered_slots_follow_the_table_by_hand():
    pool = _pool_codes(6, 2, 4, 3)
    table = np.array([5, 0, 3, -1])
    got = oracle.gather_slots(pool, table, 10, 4)
    # slot: (page, row) -> 0:(5,0) 3:(5,3) 4:(0,0) 7:(0,3) 8:(3,0) 9:(3,1)
    expect = {0: 5000, 3: 5003, 4: 0, 7: 3, 8: 3000, 9: 3001}
    for s, code in expect.items():
        assert (got[0, s] == code).all() and (got[1, s] == code + 100).all(), s
    assert oracle.pages_valid(table, 12, 4, 6)       # slots 0..11 use entries 0..2
    assert not oracle.pages_valid(table, 13, 4, 6)   # slot 12 would need entry 3 (-1)
    assert not oracle.pages_valid(np.array([5, 6, 3]), 9, 4, 6)   # page 6 is past the pool
    assert oracle.slot_page_row(table, 6, 4) == (0, 2)


@pytest.mark.parametrize("name,bs,kw", [
    ("tiny-chain-f32", 16, dict(batch=3, ragged=(40, 128), seed=(6, 1))),
    ("70b-gqa-medusa", 16, dict(batch=2, prefix_len=150, vocab=500, seed=(6, 2))),
    ("70b-gqa-medusa", 64, dict(batch=2, prefix_len=150, vocab=500, ragged=(70, 150), seed=(6, 3))),
])
def test_paged_attention_equals_dense(name, bs, kw):
    case = synth.make_case(synth.workload(name, **kw))
    case, paged = synth.page_case(case, bs, seed=kw["seed"])
    assert paged.capacity % bs == 0 and paged.capacity >= case.k_cache.shape[2]
    dense = oracle.verify(case)
    pg = oracle.verify_paged(case, paged)
    assert np.isfinite(pg["attn_out"]).all()
    np.testing.assert_array_equal(pg["attn_out"], dense["attn_out"])
    for k in ("status", "accept_len", "path", "out_tokens"):
        np.testing.assert_array_equal(pg[k], dense[k])


def test_shared_prefix_pages():
    case = synth.make_case(synth.workload("tiny-chain-f32", batch=3, ragged=(40, 100), seed=(6, 4)))
    case, paged = synth.page_case(case, 16, share_prefix_pages=2, seed=(6, 4))
    assert (paged.block_table[1:, :2] == paged.block_table[0, :2]).all()
    assert len(set(paged.block_table[:, 2:].ravel()) - {-1}) == int((paged.block_table[:, 2:] >= 0).sum())
    np.testing.assert_array_equal(case.k_cache[2, :, :32], case.k_cache[0, :, :32])
    pg = oracle.verify_paged(case, paged)
    np.testing.assert_array_equal(pg["attn_out"], oracle.verify(case)["attn_out"])


def test_invalid_entries_flag_the_sequence_and_unused_entries_are_not_read():
    case = synth.make_case(synth.workload("tiny-chain-f32", batch=4, ragged=(40, 100), seed=(6, 5)))
    case, paged = synth.page_case(case, 16, seed=(6, 5))
    T = case.nodes
    tab = paged.block_table.copy()
    used = [-(-(int(case.kv_len[b]) + T) // 16) for b in range(4)]
    tab[1, used[1] - 1] = paged.num_blocks      # last used page: past the pool
    tab[2, 0] = -3                              # first page: negative
    tab[3, used[3]:] = 10 ** 6                  # past the slots in use: never read
    bad = synth.PagedKV(paged.k_pool, paged.v_pool, tab, paged.block_size, paged.capacity)
    pg = oracle.verify_paged(case, bad)
    dense = oracle.verify(case)
    assert list(pg["status"] & 8) == [0, 8, 8, 0]
    assert np.isnan(pg["attn_out"][1]).all() and np.isnan(pg["attn_out"][2]).all()
    np.testing.assert_array_equal(pg["attn_out"][[0, 3]], dense["attn_out"][[0, 3]])
    # the vocabulary part does not read the caches
    np.testing.assert_array_equal(pg["accept_len"], dense["accept_len"])


def test_paged_commit_equals_dense_commit_and_touches_only_the_written_slots():
    case = synth.make_case(synth.workload("70b-gqa-medusa", batch=3, prefix_len=90, vocab=400,
                                          ragged=(50, 90), seed=(6, 6)))
    case, paged = synth.page_case(case, 16, share_prefix_pages=1, seed=(6, 6))
    ref = oracle.verify(case, attention=False)
    T = case.nodes
    path, acc, fin = ref["path"].copy(), ref["accept_len"].copy(), ref["final_node"].copy()
    # force a long path in sequence 2 (the tree's first-child chain)
    chain = [0]
    for i in range(1, T):
        if case.parent[2, i] == chain[-1]:
            chain.append(i)
    path[2] = -1
    path[2, :len(chain)] = chain
    acc[2], fin[2] = len(chain) - 1, chain[-1]
    dk, dv, dl = oracle.commit_kv(case.k_cache, case.v_cache, case.kv_len, path, acc, fin, T)
    pk, pv, pl = oracle.commit_kv_paged(paged.k_pool, paged.v_pool, paged.block_table, case.kv_len, path, acc,
                                        fin, T, paged.block_size, paged.capacity)
    np.testing.assert_array_equal(pl, dl)
    for b in range(3):
        n = int(case.kv_len[b]) + T
        np.testing.assert_array_equal(oracle.gather_slots(pk, paged.block_table[b], n, 16), dk[b, :, :n])
        np.testing.assert_array_equal(oracle.gather_slots(pv, paged.block_table[b], n, 16), dv[b, :, :n])
    # rows other than slots L_b..L_b+accept_len of each sequence are bit-identical (NaN included)
    touched = np.zeros(pk.shape[:1] + pk.shape[2:3], dtype=bool)
    for b in range(3):
        for s in range(int(case.kv_len[b]), int(dl[b])):
            p, r = oracle.slot_page_row(paged.block_table[b], s, 16)
            touched[p, r] = True
    same = lambda a, b: (a.view(np.uint16) == b.view(np.uint16)).all(axis=(1, 3))
    assert same(pk, paged.k_pool)[~touched].all() and same(pv, paged.v_pool)[~touched].all()
    # an invalid used entry skips the sequence
    tab = paged.block_table.copy()
    tab[0, 0] = -1
    _, _, bl = oracle.commit_kv_paged(paged.k_pool, paged.v_pool, tab, case.kv_len, path, acc, fin, T, 16,
                                      paged.capacity)
    assert bl[0] == case.kv_len[0] and (bl[1:] == dl[1:]).all()
