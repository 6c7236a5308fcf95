"""Pins for the CPU oracle: each test checks it against something other than itself.

Worked examples the pages print (tests/golden), closed forms, brute force on
tiny inputs, library routines, and chi-square tests against the target law.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1234] + list(key))))


# ---------------------------------------------------------------- tree structure

def _load_mask_fixture():
    rows, parent = [], None
    with open(os.path.join(GOLDEN, "p4_tree_mask_7x7.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line.startswith("# parent:"):
                parent = [int(x) for x in line.split(":", 1)[1].split()]
            elif line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return parent, np.array(rows, dtype=np.uint8)


def test_tree_mask_matches_printed_7x7_example():
    parent, mask = _load_mask_fixture()
    assert oracle.check_parent(parent)
    np.testing.assert_array_equal(oracle.tree_mask(parent), mask)


def test_chain_mask_is_lower_triangular():
    parent = [-1, 0, 1, 2, 3, 4]
    np.testing.assert_array_equal(oracle.tree_mask(parent), np.tril(np.ones((6, 6), np.uint8)))
    assert oracle.depths(parent) == list(range(6))


@pytest.mark.parametrize("parent,ok", [
    ([-1, 0, 0, 1], True), ([0, 0, 1], False), ([-1, 1, 0], False), ([-1, 0, 3, 1], False),
    ([-1, -1, 0], False), ([-1], True)])
def test_check_parent(parent, ok):
    assert oracle.check_parent(parent) is ok


# ---------------------------------------------------------------- attention

def _random_tree(rng, T):
    return [-1] + [int(rng.integers(0, i)) for i in range(1, T)]


def _sdpa_causal(q, k, v, scale):
    """torch's attention (float64, CPU) with an explicit bottom-right causal mask.

    q [H, Tq, D], k/v [H, N, D]; query t sits at key position N - Tq + t.
    """
    Tq, N = q.shape[1], k.shape[1]
    mask = torch.ones(Tq, N, dtype=torch.bool).tril(diagonal=N - Tq)
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask,
        scale=scale).numpy()


@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (8, 1)])
def test_chain_tree_equals_causal_attention(hq, hkv):
    rng = _rng(1, hq, hkv)
    L, T, D = 9, 5, 8
    q = rng.standard_normal((T, hq, D))
    k = rng.standard_normal((hkv, L + T + 3, D))
    v = rng.standard_normal((hkv, L + T + 3, D))
    parent = list(range(-1, T - 1))
    got = oracle.tree_attention_sequence(q, k, v, L, parent)
    g = hq // hkv
    kk = np.repeat(k[:, :L + T], g, axis=0)       # contiguous head groups
    vv = np.repeat(v[:, :L + T], g, axis=0)
    ref = _sdpa_causal(np.ascontiguousarray(q.transpose(1, 0, 2)), kk, vv, 1 / math.sqrt(D))
    np.testing.assert_allclose(got, ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_tree_attention_equals_per_path_causal_attention(seed):
    """Brute force: node i's output = causal attention over prefix + its root path."""
    rng = _rng(2, seed)
    L, T, D, hq, hkv = 6, 8, 4, 4, 2
    parent = _random_tree(rng, T)
    q = rng.standard_normal((T, hq, D))
    k = rng.standard_normal((hkv, L + T, D))
    v = rng.standard_normal((hkv, L + T, D))
    got = oracle.tree_attention_sequence(q, k, v, L, parent)
    g = hq // hkv
    for i in range(T):
        path = oracle.ancestors(parent, i)
        assert path[-1] == i and path[0] == 0
        cols = list(range(L)) + [L + j for j in path]
        kk = np.repeat(k[:, cols], g, axis=0)
        vv = np.repeat(v[:, cols], g, axis=0)
        qq = np.ascontiguousarray(q[path].transpose(1, 0, 2))
        ref = _sdpa_causal(qq, kk, vv, 1 / math.sqrt(D))[:, -1]
        np.testing.assert_allclose(got[i], ref, rtol=0, atol=1e-12)


def test_tree_attention_ignores_siblings_and_empty_prefix():
    rng = _rng(3)
    D = 4
    parent = [-1, 0, 0]
    q = rng.standard_normal((3, 1, D))
    k = rng.standard_normal((1, 3, D))
    v = rng.standard_normal((1, 3, D))
    out = oracle.tree_attention_sequence(q, k, v, 0, parent)
    np.testing.assert_allclose(out[0, 0], v[0, 0], atol=1e-15)   # root sees only itself
    s = k[0, [0, 2]] @ q[2, 0] / 2.0
    w = np.exp(s - s.max()); w /= w.sum()
    np.testing.assert_allclose(out[2, 0], w @ v[0, [0, 2]], atol=1e-15)


# ---------------------------------------------------------------- distributions

@pytest.mark.parametrize("tau", [1.0, 0.7, 0.8, 1.3])
def test_softmax_matches_scipy(tau):
    z = _rng(4).standard_normal(1000) * 3
    np.testing.assert_allclose(oracle.effective_distribution(z, tau), scipy.special.softmax(z / tau),
                               rtol=1e-13, atol=0)


@pytest.mark.parametrize("top_p,expected", [
    (0.7, [0, 0.5 / 0.8, 0, 0.3 / 0.8]),
    (0.85, [0, 0.5 / 0.95, 0.15 / 0.95, 0.3 / 0.95]),
    (0.4, [0, 1, 0, 0]),
    (0.99, [0.05, 0.5, 0.15, 0.3]),
])
def test_top_p_hand_cases(top_p, expected):
    z = np.log(np.array([0.05, 0.5, 0.15, 0.3]))
    np.testing.assert_allclose(oracle.effective_distribution(z, 1.0, top_p), expected, atol=1e-12)


def test_top_p_ties_keep_smallest_indices():
    z = np.zeros(4)
    np.testing.assert_allclose(oracle.effective_distribution(z, 1.0, 0.6), [1 / 3, 1 / 3, 1 / 3, 0], atol=1e-15)
    np.testing.assert_allclose(oracle.effective_distribution(z, 1.0, 0.2), [1, 0, 0, 0], atol=1e-15)


def test_temperature_closed_form():
    # z = tau * log([1,2,4]) -> p = [1,2,4]/7 exactly in the limit
    tau = 0.7
    z = tau * np.log(np.array([1.0, 2.0, 4.0]))
    np.testing.assert_allclose(oracle.effective_distribution(z, tau), np.array([1, 2, 4]) / 7, rtol=1e-14)


def test_argmax_first_on_ties():
    rng = _rng(5)
    for _ in range(200):
        z = rng.integers(0, 4, size=17).astype(np.float32)
        best = 0
        for k in range(1, z.size):
            if z[k] > z[best]:
                best = k
        assert int(oracle.argmax_first(z)) == best


def test_inverse_cdf_matches_searchsorted():
    rng = _rng(6)
    for _ in range(300):
        w = rng.random(12) * (rng.random(12) < 0.7)
        if w.sum() == 0:
            continue
        u = float(rng.random())
        y, _ = oracle.inverse_cdf(w, u)
        c = np.cumsum(w)
        assert y == int(np.searchsorted(c, u * c[-1], side="right"))
        yb, _ = oracle.inverse_cdf_rows(w[None], np.array([u]))
        assert int(yb[0]) == y


# ---------------------------------------------------------------- acceptance / selection

def _chain_inputs(p_rows, q_rows, drafts, u_acc, u_fin):
    """Batch of chains sharing fixed rows: p_rows [T,V], q_rows [T,V], drafts [B,T-1]."""
    B = drafts.shape[0]
    T = p_rows.shape[0]
    parent = np.tile(np.arange(-1, T - 1), (B, 1))
    tokens = np.zeros((B, T), dtype=np.int64)
    tokens[:, 1:] = drafts
    P = np.broadcast_to(p_rows, (B,) + p_rows.shape)
    Q = np.broadcast_to(q_rows, (B,) + q_rows.shape)
    return oracle.accept_and_select(parent, tokens, u_acc, u_fin, "sampling", p_rows.shape[1],
                                    p_rows=P, q_rows=Q)


def _draw(rng, probs, n):
    c = np.cumsum(probs)
    return np.minimum(np.searchsorted(c, rng.random(n) * c[-1], side="right"), probs.size - 1)


def test_exact_output_law_equals_target_one_draft():
    """Integrate the oracle's decisions over a grid of each uniform: the output law is p.

    The accept test depends on u_accept only and the correction on u_final only,
    so law(y) = sum_x q(x) [P(accept | x) 1{y = x} + P(reject | x) law(correction)].
    """
    rng = _rng(7)
    V, N = 6, 100_000
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V))
    P, Q = np.stack([p, p]), np.stack([q, q])
    grid = (np.arange(N) + 0.5) / N
    x_low = int(np.argmin(p / q))          # ratio < 1: rejected for u near 1
    assert p[x_low] < q[x_low]
    corr = _chain_inputs(P, Q, np.full((N, 1), x_low), np.full((N, 2), 0.9999999), grid)
    assert (corr["accept_len"] == 0).all()
    corr_law = np.bincount(corr["out_tokens"][:, 0], minlength=V) / N
    law = np.zeros(V)
    for x in range(V):
        r = _chain_inputs(P, Q, np.full((N, 1), x), np.stack([np.zeros(N), grid], axis=1),
                          np.full(N, 0.5))
        acc = float((r["accept_len"] == 1).mean())
        law += q[x] * acc * np.eye(V)[x] + q[x] * (1 - acc) * corr_law
    np.testing.assert_allclose(law, p, atol=1e-4)


def _chi2_first_token(p_rows, q_rows, trials, seed):
    rng = _rng(8, seed)
    T, V = p_rows.shape
    counts = np.zeros(V, dtype=np.int64)
    chunk = 200_000
    done = 0
    while done < trials:
        n = min(chunk, trials - done)
        drafts = np.stack([_draw(rng, q_rows[i], n) for i in range(1, T)], axis=1)
        u_acc = rng.random((n, T)).astype(np.float32)
        u_fin = rng.random(n).astype(np.float32)
        res = _chain_inputs(p_rows, q_rows, drafts, u_acc, u_fin)
        counts += np.bincount(res["out_tokens"][:, 0], minlength=V)
        done += n
    target = p_rows[0]
    support = target > 0
    assert counts[~support].sum() == 0
    exp = target[support] * trials
    chi2 = float(((counts[support] - exp) ** 2 / exp).sum())
    df = int(support.sum()) - 1
    return chi2, df


@pytest.mark.slow
@pytest.mark.parametrize("gamma", [1, 4])
def test_chi_square_first_token_matches_target(gamma):
    rng = _rng(9, gamma)
    V = 16
    zt = rng.standard_normal((gamma + 1, V)) * 1.5
    zq = zt + rng.standard_normal((gamma + 1, V))
    p_rows = np.stack([oracle.effective_distribution(z, 1.0) for z in zt])
    q_rows = np.stack([oracle.effective_distribution(z, 1.0) for z in zq])
    chi2, df = _chi2_first_token(p_rows, q_rows, 1_000_000, gamma)
    assert df == 15
    assert chi2 < scipy.stats.chi2.ppf(0.999, df), chi2   # 37.70


@pytest.mark.slow
def test_chi_square_with_temperature_and_top_p():
    rng = _rng(10)
    V, gamma, tau, top_p = 16, 3, 0.8, 0.9
    zt = rng.standard_normal((gamma + 1, V)) * 1.5
    zq = zt + rng.standard_normal((gamma + 1, V))
    p_rows = np.stack([oracle.effective_distribution(z, tau, top_p) for z in zt])
    q_rows = np.stack([oracle.effective_distribution(z, tau, top_p) for z in zq])
    chi2, df = _chi2_first_token(p_rows, q_rows, 1_000_000, 99)
    assert chi2 < scipy.stats.chi2.ppf(0.999, df), (chi2, df)


def test_chi_square_detects_a_wrong_rule():
    """Power check: accepting with p/q but resampling from p (not [p-q]_+) is biased."""
    rng = _rng(11)
    V, n = 16, 200_000
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V))
    x = _draw(rng, q, n)
    u = rng.random(n)
    y = _draw(rng, p, n)
    out = np.where(u < p[x] / q[x], x, y)
    counts = np.bincount(out, minlength=V)
    chi2 = float(((counts - p * n) ** 2 / (p * n)).sum())
    assert chi2 > scipy.stats.chi2.ppf(0.999, V - 1)


@pytest.mark.slow
def test_expected_lengths_constant_acceptance():
    fx = json.load(open(os.path.join(GOLDEN, "worked_examples.json"), encoding="utf-8"))["p5_expected_lengths"]
    alpha, gamma = fx["alpha"], fx["gamma"]
    e_out = sum(alpha ** k for k in range(gamma + 1))
    e_acc = sum(alpha ** k for k in range(1, gamma + 1))
    assert abs(e_out - fx["expected_output_tokens_printed"]) < 0.005
    assert abs(e_acc - fx["expected_accepted_drafts_printed"]) < 0.005
    # every position: p = [0.6, 0.4], q = [0.4, 0.6] -> sum(min(p, q)) = 0.8
    p = np.array([0.6, 0.4]); q = np.array([0.4, 0.6])
    p_rows = np.stack([oracle.effective_distribution(np.log(p), 1.0)] * (gamma + 1))
    q_rows = np.stack([oracle.effective_distribution(np.log(q), 1.0)] * (gamma + 1))
    rng = _rng(12)
    trials, chunk = 1_000_000, 250_000
    tot_len = 0
    for _ in range(trials // chunk):
        drafts = np.stack([_draw(rng, q, chunk) for _ in range(gamma)], axis=1)
        res = _chain_inputs(p_rows, q_rows, drafts, rng.random((chunk, gamma + 1)), rng.random(chunk))
        tot_len += int(res["accept_len"].sum())
    mean_acc = tot_len / trials
    assert abs(mean_acc - e_acc) < 0.008, mean_acc          # 5 sigma
    assert abs(mean_acc + 1 - e_out) < 0.008


def test_forced_decisions():
    V, gamma = 8, 4
    rng = _rng(13)
    p = rng.dirichlet(np.ones(V)); q = rng.dirichlet(np.ones(V))
    P = np.stack([p] * (gamma + 1)); Q = np.stack([q] * (gamma + 1))
    drafts = np.array([[1, 2, 3, 4]])
    # u = 0 with p(x) > 0: everything accepted, bonus from the leaf's row
    r = _chain_inputs(P, Q, drafts, np.zeros((1, gamma + 1)), np.array([0.5]))
    assert r["accept_len"][0] == gamma and r["final_from_residual"][0] == 0
    assert list(r["out_tokens"][0, :gamma]) == [1, 2, 3, 4]
    assert r["out_tokens"][0, gamma] == oracle.inverse_cdf(p, 0.5)[0]
    # p == q: ratio 1, accepted for any u < 1
    r = _chain_inputs(P, P, drafts, np.full((1, gamma + 1), 0.9999999), np.array([0.1]))
    assert r["accept_len"][0] == gamma
    # disjoint supports: rejected at depth 1 and the correction comes from p
    p2 = np.array([0.5, 0.5, 0, 0, 0, 0, 0, 0]); q2 = np.array([0, 0, 0.25, 0.25, 0.25, 0.25, 0, 0])
    r = _chain_inputs(np.stack([p2] * 5), np.stack([q2] * 5), drafts, np.zeros((1, 5)), np.array([0.7]))
    assert r["accept_len"][0] == 0 and r["out_tokens"][0, 0] == 1 and r["final_from_residual"][0] == 1
    # u just below 1 with p(x) < q(x): rejected
    x = int(np.argmax(q - p))
    r = _chain_inputs(P, Q, np.array([[x, x, x, x]]), np.full((1, 5), 0.99999994), np.array([0.3]))
    assert r["accept_len"][0] == 0
    # q(x) = 0 for a supplied draft: rejected and flagged
    r = _chain_inputs(np.stack([p2] * 5), np.stack([q2] * 5), np.array([[0, 0, 0, 0]]),
                      np.zeros((1, 5)), np.array([0.3]))
    assert r["accept_len"][0] == 0 and r["status"][0] & 4


def _greedy_chain(tokens, best):
    """Greedy chain with per-row best tokens `best` (row i predicts node i+1)."""
    T = len(tokens)
    parent = np.arange(-1, T - 1)[None]
    return oracle.accept_and_select(parent, np.array([tokens]), np.zeros((1, T)), np.zeros(1),
                                    "greedy", 100, greedy_rows=np.array([best]))


def test_worked_example_draft_verify_walkthrough():
    fx = json.load(open(os.path.join(GOLDEN, "worked_examples.json"), encoding="utf-8"))["p4_draft_verify"]
    names = ["root"] + fx["drafts"] + [fx["target_token_at_reject"], "other"]
    ids = {n: k for k, n in enumerate(names)}
    tokens = [ids["root"]] + [ids[d] for d in fx["drafts"]]
    # the target's best token agrees with d1..d3, prefers c4 over d4
    best = [ids["d1"], ids["d2"], ids["d3"], ids["c4"], ids["other"], ids["other"]]
    r = _greedy_chain(tokens, best)
    out = [names[t] for t in r["out_tokens"][0] if t >= 0]
    assert out == fx["output"]
    assert r["accept_len"][0] + 1 == fx["tokens_per_target_call"]
    verdict = ["accept" if a else "reject" for a in r["node_accept"][0, 1:]]
    assert verdict[:4] == fx["verdicts"][:4]


def test_worked_example_medusa_greedy():
    fx = json.load(open(os.path.join(GOLDEN, "worked_examples.json"), encoding="utf-8"))["p3_medusa_greedy"]
    vocab = ["<ctx>"] + fx["candidates"] + ["不错"]
    ids = {w: k for k, w in enumerate(vocab)}
    tokens = [0] + [ids[w] for w in fx["candidates"]]
    best = [ids[w] for w in fx["target_best"]] + [0, 0, 0]
    r = _greedy_chain(tokens, best)
    n = int(r["accept_len"][0])
    assert [vocab[t] for t in r["out_tokens"][0, :n]] == fx["accepted"]
    emitted = {vocab[t] for t in r["out_tokens"][0] if t >= 0}
    assert not emitted & set(fx["discarded"])
    assert vocab[r["out_tokens"][0, n]] == fx["target_best"][n]   # the target's own token at the mismatch


@pytest.mark.parametrize("seed", range(20))
def test_tree_selection_equals_brute_force_over_paths(seed):
    rng = _rng(14, seed)
    T = int(rng.integers(2, 9))
    parent = _random_tree(rng, T)
    V = 5
    B = 64
    greedy = rng.integers(0, V, size=(B, T))
    tokens = rng.integers(0, V, size=(B, T))
    res = oracle.accept_and_select(np.tile(parent, (B, 1)), tokens, np.zeros((B, T)), np.zeros(B),
                                   "greedy", V, greedy_rows=greedy)
    depth = oracle.depths(parent)
    leaves = [i for i in range(T) if i not in parent[1:]]
    for b in range(B):
        best = (0, 0)       # (accepted length, -deepest node index)
        for leaf in leaves:
            path = oracle.ancestors(parent, leaf)
            n = 0
            for j in path[1:]:
                if tokens[b, j] != greedy[b, parent[j]]:
                    break
                n += 1
            cand = (n, -path[n])
            if cand > best:
                best = cand
        assert res["accept_len"][b] == best[0]
        assert res["final_node"][b] == -best[1]
        v = -best[1]
        assert list(res["path"][b, :depth[v] + 1]) == oracle.ancestors(parent, v)
        assert res["out_tokens"][b, best[0]] == greedy[b, v]


@pytest.mark.slow
def test_joint_law_of_two_tokens_table_lm():
    """Decode two tokens with a table-driven target/draft pair over up to two rounds.

    The joint law of the first two emitted tokens must be p(y1) p(y2 | y1).
    """
    rng = _rng(15)
    V, gamma = 4, 2
    nctx = 1 + V + V ** 2 + V ** 3
    zt = rng.standard_normal((nctx, V)) * 1.2
    zq = zt + rng.standard_normal((nctx, V)) * 0.8
    Pt = np.stack([oracle.effective_distribution(z, 1.0) for z in zt])
    Qt = np.stack([oracle.effective_distribution(z, 1.0) for z in zq])

    def ctx_id(ctx):          # ctx: [n, len] -> id of the context
        ln = ctx.shape[1]
        base = sum(V ** k for k in range(ln))
        code = np.zeros(ctx.shape[0], dtype=np.int64)
        for c in range(ln):
            code = code * V + ctx[:, c]
        return base + code

    def one_round(prefix, n):
        T = gamma + 1
        drafts = np.zeros((n, gamma), dtype=np.int64)
        ctx = prefix
        qrows = np.zeros((n, T, V)); prows = np.zeros((n, T, V))
        for i in range(gamma):
            q = Qt[ctx_id(ctx)]
            c = np.cumsum(q, axis=1)
            x = np.minimum((rng.random(n)[:, None] * c[:, -1:] >= c).sum(axis=1), V - 1)
            drafts[:, i] = x
            qrows[:, i + 1] = q
            ctx = np.concatenate([ctx, x[:, None]], axis=1)
        for i in range(T):
            prows[:, i] = Pt[ctx_id(np.concatenate([prefix, drafts[:, :i]], axis=1))]
        tokens = np.concatenate([np.zeros((n, 1), dtype=np.int64), drafts], axis=1)
        parent = np.tile(np.arange(-1, T - 1), (n, 1))
        return oracle.accept_and_select(parent, tokens, rng.random((n, T)), rng.random(n),
                                        "sampling", V, p_rows=prows, q_rows=qrows)

    trials = 400_000
    r1 = one_round(np.zeros((trials, 0), dtype=np.int64), trials)
    y1 = r1["out_tokens"][:, 0]
    y2 = np.where(r1["accept_len"] >= 1, r1["out_tokens"][:, 1], -1)
    need = y2 < 0
    r2 = one_round(y1[need][:, None], int(need.sum()))
    y2[need] = r2["out_tokens"][:, 0]
    counts = np.bincount(y1 * V + y2, minlength=V * V)
    p1 = Pt[0]
    joint = np.array([p1[a] * Pt[1 + a][b] for a in range(V) for b in range(V)])
    exp = joint * trials
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert chi2 < scipy.stats.chi2.ppf(0.999, V * V - 1), chi2


def test_accept_test_is_strict_at_equality():
    """The page's sampler accepts when the uniform is below the ratio (strict compare)."""
    p = np.array([0.25, 0.75]); q = np.array([0.5, 0.5])     # ratio p(0)/q(0) = 0.5 exactly
    r = _chain_inputs(np.stack([p, p]), np.stack([q, q]), np.array([[0], [0]]),
                      np.array([[0.0, 0.5], [0.0, 0.4999999]]), np.array([0.0, 0.0]))
    assert list(r["accept_len"]) == [0, 1]


def test_inverse_cdf_boundaries():
    # u * W equal to a prefix sum moves to the next token; zero-weight tokens are never drawn
    assert oracle.inverse_cdf(np.array([0.25, 0.25, 0.5]), 0.25)[0] == 1
    assert oracle.inverse_cdf(np.array([0.25, 0.25, 0.5]), 0.5)[0] == 2
    assert oracle.inverse_cdf(np.array([0.0, 0.5, 0.5]), 0.0)[0] == 1
    assert oracle.inverse_cdf(np.array([0.5, 0.5, 0.0]), 0.9999999)[0] == 1
    y, _ = oracle.inverse_cdf_rows(np.array([[0.25, 0.25, 0.5], [0.0, 0.5, 0.5]]), np.array([0.25, 0.0]))
    assert list(y) == [1, 1]


def test_residual_uses_the_smallest_index_child():
    """Root with two drafted children, both rejected: the correction is drawn from
    [p_0 - q_c]_+ of the smallest-index child c (the reading taken where the pages
    name only one draft per position).  p_0 = [1/2, 1/4, 1/8, 1/8];
    q_1 uniform -> [p_0 - q_1]_+ = [1/4, 0, 0, 0]: token 0 for any uniform;
    q_2 = [1/8, 1/8, 1/2, 1/4] -> [3/8, 1/8, 0, 0]: token 1 for u_final = 0.9."""
    p0 = np.array([0.5, 0.25, 0.125, 0.125])
    q1 = np.full(4, 0.25)
    q2 = np.array([0.125, 0.125, 0.5, 0.25])
    P = np.stack([p0, p0, p0])[None]
    Q = np.stack([q1, q1, q2])[None]
    # node 1 = token 2 (ratio 0.125/0.25), node 2 = token 3 (ratio 0.125/0.25): both rejected at u = 0.9
    r = oracle.accept_and_select(np.array([[-1, 0, 0]]), np.array([[0, 2, 3]]), np.array([[0.0, 0.9, 0.9]]),
                                 np.array([0.9]), "sampling", 4, p_rows=P, q_rows=Q)
    assert r["accept_len"][0] == 0 and r["final_node"][0] == 0 and r["final_from_residual"][0] == 1
    assert r["out_tokens"][0, 0] == 0
    # with the children swapped the other draft row is the smallest-index child's
    r = oracle.accept_and_select(np.array([[-1, 0, 0]]), np.array([[0, 3, 2]]), np.array([[0.0, 0.9, 0.9]]),
                                 np.array([0.9]), "sampling", 4, p_rows=P, q_rows=np.stack([q1, q2, q1])[None])
    assert r["out_tokens"][0, 0] == 1
