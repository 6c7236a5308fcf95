"""Pins for the KV commit (oracle.commit_kv), each against something other than itself.

* A hand-worked case where a destination slot is also an earlier source.
* After the commit, ordinary causal attention over the committed prefix gives,
  for every node on the accepted path, the tree attention that node had
  before (the point of keeping the path): checked against torch's float64
  scaled_dot_product_attention.
* Chains only move the length; invalid sequences stay untouched.
"""
import numpy as np
import torch

import oracle


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([777] + list(key))))


def test_commit_moves_the_path_even_when_a_destination_is_an_earlier_source():
    Hkv, Lcap, D, L = 2, 16, 4, 3
    parent = [-1, 0, 0, 2, 2, 4]
    path = np.array([[0, 2, 4, 5, -1, -1]])
    k = np.zeros((1, Hkv, Lcap, D), dtype=np.float32)
    for h in range(Hkv):
        for s in range(Lcap):
            k[0, h, s, :] = 100 * h + s
    v = -k
    nk, nv, nl = oracle.commit_kv(k, v, np.array([L]), path, np.array([3]), np.array([5]), len(parent))
    assert nl[0] == L + 3 + 1
    for h in range(Hkv):
        # slot 4 <- node 2 (slot 5), slot 5 <- node 4 (slot 7), slot 6 <- node 5 (slot 8)
        assert list(nk[0, h, :, 0]) == [100 * h + s for s in [0, 1, 2, 3, 5, 7, 8, 7, 8, 9, 10, 11, 12, 13, 14, 15]]
    np.testing.assert_array_equal(nv, -nk)
    assert (k[0, :, :, 0] == np.arange(Lcap)[None, :] + 100 * np.arange(Hkv)[:, None]).all()   # inputs intact


def _sdpa_last(q, k, v, scale):
    """Causal attention of the last position: q [Hq, D] against keys/values [Hkv, n, D] (GQA groups)."""
    Hq, Hkv = q.shape[0], k.shape[0]
    kk = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=0))[None]
    vv = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=0))[None]
    qq = torch.from_numpy(q)[None, :, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
    return out[0, :, 0, :].numpy()


def test_committed_cache_reproduces_tree_attention_of_the_path():
    rng = _rng(1)
    for trial in range(6):
        T, Hq, Hkv, D, L = 9, 4, 2, 8, 5 + trial
        parent = [-1] + [int(rng.integers(0, i)) for i in range(1, T)]
        Lcap = L + T + 3
        q = rng.standard_normal((T, Hq, D))
        k = rng.standard_normal((1, Hkv, Lcap, D))
        v = rng.standard_normal((1, Hkv, Lcap, D))
        end = int(rng.integers(1, T))
        p = [end]
        while p[-1] != 0:
            p.append(parent[p[-1]])
        p = p[::-1]
        A = len(p) - 1
        path = np.full((1, T), -1)
        path[0, :A + 1] = p
        nk, nv, nl = oracle.commit_kv(k, v, np.array([L]), path, np.array([A]), np.array([end]), T)
        assert nl[0] == L + A + 1
        scale = 1.0 / np.sqrt(D)
        for depth, node in enumerate(p):
            tree = oracle.tree_attention_node(q[node], k[0], v[0], L, np.array(parent), node, scale=scale)
            causal = _sdpa_last(q[node], nk[0][:, :L + depth + 1], nv[0][:, :L + depth + 1], scale)
            np.testing.assert_allclose(causal, tree, atol=1e-12)


def test_chains_only_move_the_length_and_invalid_sequences_stay():
    rng = _rng(2)
    B, Hkv, Lcap, D, T = 4, 2, 20, 4, 5
    k = rng.standard_normal((B, Hkv, Lcap, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, Lcap, D)).astype(np.float32)
    kv_len = np.array([6, 6, 16, 6])
    path = np.tile(np.array([0, 1, 2, -1, -1]), (B, 1))
    path[3] = [0, 3, 1, -1, -1]          # not a valid root path: k <= path[k] fails at k = 2
    accept_len = np.array([2, 2, 2, 2])
    final_node = np.array([2, -1, 2, 2])  # sequence 1 void; sequence 2's kv_len leaves no room (16 + 5 > 20)
    nk, nv, nl = oracle.commit_kv(k, v, kv_len, path, accept_len, final_node, T)
    assert list(nl) == [9, 6, 16, 6]
    np.testing.assert_array_equal(nk, k)
    np.testing.assert_array_equal(nv, v)
