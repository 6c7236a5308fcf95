"""Pins for the oracle's near-tie bookkeeping.

These margins decide which decisions leave the bit-exact GPU comparison
(a decision whose uniform lies within 1e-5 of its threshold is reported
separately; the acceptance test compares a uniform with p(x)/q(x):
"推测解码技术详解：加速LLM推理的关键", section "数学保证：无损输出质量").  Every
expected margin below is worked out by hand from distributions whose
cumulative masses are known exactly: logits z = tau * log(p) give
softmax(z / tau) = p, and the masses are short binary or decimal fractions.
"""
import numpy as np
import pytest

import oracle

INF = float("inf")


def _logits(p, tau=1.0):
    return tau * np.log(np.asarray(p, dtype=np.float64))


# ---------------------------------------------------------------- top-p cut

# p in token order [0.1, 0.4, 0.2, 0.3]: by (probability desc, id asc) the
# order is ids 1, 3, 2, 0 with cumulative masses 0.4, 0.7, 0.9, 1.0.
P_SCRAMBLED = [0.1, 0.4, 0.2, 0.3]


@pytest.mark.parametrize("top_p,margin", [
    (0.05, 0.05),   # cut at the first token: mass before it is 0 -> |0 - 0.05|
    (0.30, 0.10),   # first token: |0.4 - 0.3| beats |0 - 0.3|
    (0.43, 0.03),   # second token (0.7 >= 0.43): the side before it is closer, |0.4 - 0.43|
    (0.69, 0.01),   # second token: the side including it is closer, |0.7 - 0.69|
    (0.85, 0.05),   # third token: |0.9 - 0.85| beats |0.7 - 0.85|
    (0.93, 0.03),   # fourth token: |0.9 - 0.93| beats |1.0 - 0.93|
    (0.99, 0.01),   # fourth token: |1.0 - 0.99|
])
@pytest.mark.parametrize("tau", [1.0, 0.7, 1.6])
def test_nucleus_margin_hand_cases(top_p, margin, tau):
    got = oracle.nucleus_margin(_logits(P_SCRAMBLED, tau), tau, top_p)
    assert abs(got - margin) < 1e-12, (top_p, tau, got, margin)


def test_nucleus_margin_on_the_boundary_and_off():
    # top_p equal to a cumulative mass: the cut sits exactly on it
    assert oracle.nucleus_margin(_logits([0.25, 0.25, 0.25, 0.25]), 1.0, 0.5) < 1e-15
    assert oracle.nucleus_margin(_logits([0.5, 0.25, 0.125, 0.125]), 1.0, 0.75) < 1e-15
    # top-p off
    assert oracle.nucleus_margin(_logits(P_SCRAMBLED), 1.0, 1.0) == INF


def test_nucleus_margin_ties_are_ordered_by_token_id():
    # four equal masses: the masses before/including the crossing token are
    # multiples of 1/4 whichever tied token crosses
    assert abs(oracle.nucleus_margin(np.zeros(4), 1.0, 0.3) - 0.05) < 1e-12    # |0.25 - 0.3|
    assert abs(oracle.nucleus_margin(np.zeros(4), 1.0, 0.6) - 0.10) < 1e-12    # |0.5 - 0.6|


# ---------------------------------------------------------------- inverse CDF

# w = [2, 0, 3, 5]: W = 10, C / W = [0.2, 0.2, 0.5, 1.0]
W_ROW = [2.0, 0.0, 3.0, 5.0]


@pytest.mark.parametrize("u,y,margin", [
    (0.03, 0, 0.03),    # token 0, the lower bound 0 is closer
    (0.13, 0, 0.07),    # token 0, its upper bound 0.2 is closer
    (0.21, 2, 0.01),    # token 2 (token 1 has no weight): lower bound C_1 / W = 0.2
    (0.48, 2, 0.02),    # token 2, upper bound 0.5
    (0.57, 3, 0.07),    # token 3, lower bound 0.5
    (0.93, 3, 0.07),    # token 3, upper bound 1.0
])
@pytest.mark.parametrize("scale", [1.0, 7.3, 1e-3])
def test_inverse_cdf_margin_hand_cases(u, y, margin, scale):
    w = np.array(W_ROW) * scale                     # unnormalised weights: margins are relative to W
    got_y, got_m = oracle.inverse_cdf(w, u)
    assert got_y == y
    assert abs(got_m - margin) < 1e-12, (u, got_m, margin)


def test_inverse_cdf_rows_margins_match_hand_cases():
    cases = [(0.03, 0, 0.03), (0.13, 0, 0.07), (0.21, 2, 0.01), (0.48, 2, 0.02), (0.57, 3, 0.07), (0.93, 3, 0.07)]
    scales = np.array([1.0, 2.0, 0.5, 3.0, 1e-3, 10.0])
    w = np.array(W_ROW)[None, :] * scales[:, None]
    u = np.array([c[0] for c in cases])
    y, m = oracle.inverse_cdf_rows(w, u)
    assert list(y) == [c[1] for c in cases]
    np.testing.assert_allclose(m, [c[2] for c in cases], rtol=0, atol=1e-12)
    # a leading batch axis is kept
    y2, m2 = oracle.inverse_cdf_rows(w.reshape(2, 3, 4), u.reshape(2, 3))
    assert y2.shape == (2, 3) and list(y2.ravel()) == list(y)
    np.testing.assert_allclose(m2.ravel(), m, rtol=0, atol=0)


def test_inverse_cdf_fallback_draw_has_zero_margin():
    # u * W not below any prefix sum (u = 1): the last token with weight is
    # drawn and the draw sits on its upper bound
    for fn in (lambda w, u: oracle.inverse_cdf(w, u),
               lambda w, u: tuple(a[0] for a in oracle.inverse_cdf_rows(w[None], np.array([u])))):
        y, m = fn(np.array([1.0, 2.0, 0.0]), 1.0)
        assert int(y) == 1 and float(m) == 0.0


# ---------------------------------------------------------------- which decisions a margin taints

# Four-token rows with exact binary masses.  Row 0 = p_0, row 1 = p_1, ...
P0 = [0.5, 0.25, 0.125, 0.125]
P1 = [0.125, 0.25, 0.375, 0.25]
P2 = [0.25, 0.25, 0.25, 0.25]
Q_UNIFORM = [0.25, 0.25, 0.25, 0.25]
Q_SKEW = [0.5, 0.125, 0.125, 0.25]


def _vocab(parent, tokens, tgt, dft, u_acc, u_fin, top_p=1.0):
    B = len(u_fin)
    T = len(parent)
    tl = np.stack([_logits(r) for r in tgt])
    dl = np.stack([_logits(Q_UNIFORM)] + [_logits(r) for r in dft])
    return oracle.verify_vocab(np.tile(parent, (B, 1)), np.tile(tokens, (B, 1)), np.tile(tl, (B, 1, 1)),
                               np.tile(dl, (B, 1, 1)), np.asarray(u_acc, dtype=np.float64),
                               np.asarray(u_fin, dtype=np.float64), mode="sampling", temperature=1.0,
                               top_p=top_p)


def test_accept_margin_flags_only_the_decision_near_its_ratio():
    # chain root -> 1 -> 2; node 1 = token 2 tested against p_0(2)/q_1(2) = 0.125/0.25 = 0.5,
    # node 2 = token 0 tested against p_1(0)/q_2(0) = 0.125/0.5 = 0.25
    parent, tokens = [-1, 0, 1], [0, 2, 0]
    u = [[0.0, 0.5 - 5e-6, 0.9],      # node 1 within 1e-5 of 0.5
         [0.0, 0.5 - 2e-5, 0.9],      # 2e-5 away: not a near-tie
         [0.0, 0.1, 0.25 + 7e-6],     # node 2 within 1e-5 of 0.25
         [0.0, 0.1, 0.25 - 3e-5],     # clear of both thresholds
         [0.0, 0.5 + 9e-6, 0.25]]     # node 1 just above (rejected, still near); node 2 exactly on 0.25
    out = _vocab(parent, tokens, [P0, P1, P2], [Q_UNIFORM, Q_SKEW], u, [0.6] * 5)
    np.testing.assert_allclose(out["node_p"][0, 1:], [0.125, 0.125], rtol=1e-14)
    np.testing.assert_allclose(out["node_q"][0, 1:], [0.25, 0.5], rtol=1e-14)
    np.testing.assert_allclose(out["accept_margin"][:, 1], [5e-6, 2e-5, 0.4, 0.4, 9e-6], rtol=1e-6)
    np.testing.assert_allclose(out["accept_margin"][:, 2], [0.65, 0.65, 7e-6, 3e-5, 0.0], rtol=1e-6, atol=1e-15)
    expect = np.array([[0, 1, 0], [0, 0, 0], [0, 0, 1], [0, 0, 0], [0, 1, 1]], dtype=bool)
    np.testing.assert_array_equal(out["node_near"], expect)
    np.testing.assert_array_equal(out["seq_near"], expect.any(axis=1))
    # a ratio >= 1 is never near for u in [0, 1)
    out = _vocab(parent, [0, 0, 0], [P0, P1, P2], [Q_UNIFORM, Q_SKEW], [[0.0, 0.99999, 0.0]], [0.6])
    assert out["accept_margin"][0, 1] > 0.9 and not out["node_near"][0, 1]


def test_top_p_margin_of_a_row_flags_the_nodes_that_row_verifies():
    # top_p = 0.75 + 3e-7: a P0 row (sorted masses 0.5, 0.75, 0.875, 1) has its
    # cut 3e-7 above the mass 0.75; a P1 row (0.375, 0.625, 0.875, 1) is far.
    top_p = 0.75 + 3e-7
    # tree root -> {1, 2}, 1 -> {3}
    parent, tokens = [-1, 0, 0, 1], [0, 1, 2, 1]
    u = [[0.0, 0.1, 0.1, 0.1]]
    out = _vocab(parent, tokens, [P1, P0, P1, P1], [P1, P1, P1], u, [0.6], top_p=top_p)
    assert abs(out["target_topp_margin"][0, 1] - 3e-7) < 1e-12
    assert out["target_topp_margin"][0, 0] > 0.1
    # target row 1 verifies node 3 (its child) only; nodes 1 and 2 are verified by row 0
    np.testing.assert_array_equal(out["node_near"][0], [False, False, False, True])
    # the same cut on a draft row flags the node drafted from it
    out = _vocab(parent, tokens, [P1, P1, P1, P1], [P1, P0, P1], u, [0.6], top_p=top_p)
    assert abs(out["draft_topp_margin"][0, 2] - 3e-7) < 1e-12
    np.testing.assert_array_equal(out["node_near"][0], [False, False, True, False])


def test_final_draw_margins():
    # chain root -> 1 with token 2: p_0(2)/q_1(2) = 0.125/0.25 = 0.5.
    parent, tokens = [-1, 0], [0, 2]
    # (a) rejected (u = 0.9): residual [p_0 - q_1]_+ = [0.25, 0, 0, 0] -> token 0 for any
    #     u_final; its CDF bounds are 0 and 1, so u_final = 3e-6 is near, 0.5 is not
    out = _vocab(parent, tokens, [P0, P1], [Q_UNIFORM], [[0.0, 0.9], [0.0, 0.9]], [3e-6, 0.5])
    assert list(out["final_node"]) == [0, 0] and list(out["out_tokens"][:, 0]) == [0, 0]
    np.testing.assert_allclose(out["cdf_margin"], [3e-6, 0.5], rtol=1e-9)
    np.testing.assert_array_equal(out["final_near"], [True, False])
    # (b) accepted (u = 0.1): bonus from p_1, C = [0.125, 0.375, 0.75, 1.0];
    #     u_final = 0.375 + 4e-6 -> token 2, 4e-6 above its lower bound
    out = _vocab(parent, tokens, [P0, P1], [Q_UNIFORM], [[0.0, 0.1], [0.0, 0.1]], [0.375 + 4e-6, 0.6])
    assert list(out["final_node"]) == [1, 1] and list(out["out_tokens"][:, 1]) == [2, 2]
    np.testing.assert_allclose(out["cdf_margin"], [4e-6, 0.15], rtol=1e-6)
    np.testing.assert_array_equal(out["final_near"], [True, False])
    np.testing.assert_array_equal(out["seq_near"], [True, False])


def test_final_draw_inherits_the_top_p_margins_of_the_rows_it_reads():
    top_p = 0.75 + 3e-7        # near the cut of a P0 row, far from the cut of a P1 row (see above)
    parent = [-1, 0]
    # node 1 rejected (u near 1): the draw reads target row 0 and node 1's draft row
    out = _vocab(parent, [0, 2], [P0, P1], [P1], [[0.0, 0.9999]], [0.6], top_p=top_p)
    assert out["final_node"][0] == 0 and out["final_near"][0]
    # token 0 lies outside row 0's nucleus (p = 0): rejected, and node 1's draft row is near
    out = _vocab(parent, [0, 0], [P1, P1], [P0], [[0.0, 0.0]], [0.6], top_p=top_p)
    assert out["final_node"][0] == 0 and out["final_near"][0]
    # node 1 accepted (ratio 3 at token 2): a bonus from target row 1, the near
    # draft row of node 1 is not read by the draw
    out = _vocab(parent, [0, 2], [P1, P1], [P0], [[0.0, 0.0]], [0.6], top_p=top_p)
    assert out["final_node"][0] == 1 and not out["final_near"][0] and out["node_near"][0, 1]
    out = _vocab(parent, [0, 2], [P1, P0], [P1], [[0.0, 0.0]], [0.6], top_p=top_p)
    assert out["final_node"][0] == 1 and out["final_near"][0] and not out["node_near"][0, 1]


def test_lossless_rule_flags_match_the_independent_rule_on_chains():
    parent, tokens = [-1, 0, 1], [0, 2, 0]
    u = [[0.0, 0.5 - 5e-6, 0.9], [0.0, 0.1, 0.25 + 7e-6], [0.0, 0.1, 0.3]]
    kw = dict(mode="sampling", temperature=1.0, top_p=1.0)
    tl = np.tile(np.stack([_logits(r) for r in (P0, P1, P2)]), (3, 1, 1))
    dl = np.tile(np.stack([_logits(r) for r in (Q_UNIFORM, Q_UNIFORM, Q_SKEW)]), (3, 1, 1))
    args = (np.tile(parent, (3, 1)), np.tile(tokens, (3, 1)), tl, dl, np.array(u), np.array([0.6, 0.6, 3e-6]))
    a = oracle.verify_vocab(*args, **kw)
    b = oracle.verify_vocab(*args, rule="lossless", **kw)
    np.testing.assert_array_equal(a["node_near"], [[0, 1, 0], [0, 0, 1], [0, 0, 0]])
    np.testing.assert_array_equal(b["node_near"], [[0, 1, 0], [0, 0, 1], [0, 0, 0]])
    np.testing.assert_array_equal(a["seq_near"], b["seq_near"])
