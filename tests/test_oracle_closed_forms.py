"""Hand-worked cases pinning each building block of the oracle: temperature softmax, the
accept rule, the inverse-CDF convention, argmax and top-F tie-breaks, row errors, KV advance and
the outcome hit rule. Every expected value below is worked out by hand in its comment."""
import math

import numpy as np
import pytest

import oracle

LN3 = math.log(3.0)
U_MAX = float(np.float32(1) - np.float32(2 ** -24))   # largest float32 uniform below 1


# ---------------------------------------------------------------------------------- softmax
@pytest.mark.parametrize("T,expected", [
    (1.0, [0.25, 0.75]),      # exp(0) : exp(ln 3) = 1 : 3
    (0.5, [0.10, 0.90]),      # logits / T = (0, 2 ln 3) -> 1 : 9
    (2.0, [1 / (1 + 3 ** 0.5), 3 ** 0.5 / (1 + 3 ** 0.5)]),   # (0, ln 3 / 2) -> 1 : sqrt 3
])
def test_softmax_temperature_hand_values(T, expected):
    np.testing.assert_allclose(oracle.softmax(np.array([0.0, LN3]), T), expected, rtol=0,
                               atol=1e-15)


def test_softmax_masked_tokens():
    # -inf logits are masked tokens of probability 0; the rest share equally
    np.testing.assert_array_equal(oracle.softmax(np.array([-np.inf, 2.0, 2.0]), 0.7),
                                  [0.0, 0.5, 0.5])


def test_softmax_shift_invariance_large_logits():
    # adding 1000 to every logit changes nothing (no overflow): p = (1/4, 3/4)
    np.testing.assert_allclose(oracle.softmax(np.array([1000.0, 1000.0 + LN3]), 1.0),
                               [0.25, 0.75], atol=1e-15)


# ------------------------------------------------------------------------------ accept rule
def two_token_request(t0, d0, x, u0, u1, T=1.0, kv=10):
    t_rows = np.array([t0, [0.0, 0.0]])
    d_rows = np.array([d0])
    return oracle.verify_sample_request(t_rows, d_rows, [x], np.array([u0, u1]), kv, T)


@pytest.mark.parametrize("u0,kept", [(0.33, True), (0.34, False)])
def test_accept_ratio_hand_case(u0, kept):
    """p = (1/4, 3/4), q = (3/4, 1/4), x = 0: ratio 1/3, kept iff u < 1/3. On rejection the
    residual max(0, p - q) = (0, 1/2) can only give token 1, whatever u_1 is."""
    r = two_token_request([0.0, LN3], [LN3, 0.0], 0, u0, 0.999)
    assert abs(r["p_x"][0] - 0.25) < 1e-15 and abs(r["q_x"][0] - 0.75) < 1e-15
    if kept:
        assert r["tau"] == 2 and r["tokens"][0] == 0
    else:
        assert r["tau"] == 1 and list(r["tokens"]) == [1, -1]
        assert abs(r["resid_mass"] - 0.5) < 1e-15
        assert r["kv_out"] == 11


@pytest.mark.parametrize("u0,kept", [(0.11, True), (0.12, False)])
def test_accept_ratio_depends_on_temperature(u0, kept):
    """Same logits at T = 0.5: p = (1/10, 9/10), q = (9/10, 1/10), ratio 1/9 = 0.111..."""
    r = two_token_request([0.0, LN3], [LN3, 0.0], 0, u0, 0.5, T=0.5)
    assert (r["tau"] == 2) == kept


@pytest.mark.parametrize("u0", [0.0, 0.5, U_MAX])
def test_target_at_least_as_likely_is_always_kept(u0):
    """p(x) = 3/4 >= q(x) = 1/4: kept for every u in [0,1), including the largest float32."""
    r = two_token_request([0.0, LN3], [LN3, 0.0], 1, u0, 0.5)
    assert r["tau"] == 2 and r["tokens"][0] == 1


def test_equal_rows_keep_every_draft_and_sample_the_extra_row():
    """Draft rows equal to target rows: ratio 1 everywhere, so all K drafts are kept for any u;
    the last token comes from the extra target row p_K = (1/4, 1/4, 1/2): u_K = 0.3 lands in the
    second quarter (running sums 0.25, 0.5, 1) -> token 1; u_K = 0.6 -> token 2."""
    rng = np.random.default_rng(3)
    K = 3
    rows = rng.normal(size=(K, 3))
    t_rows = np.vstack([rows, np.log([0.25, 0.25, 0.5])])
    x = [0, 2, 1]
    for uK, y in [(0.3, 1), (0.6, 2), (0.0, 0)]:
        r = oracle.verify_sample_request(t_rows, rows.copy(), x, np.array([U_MAX] * K + [uK]),
                                         5, 1.0)
        assert list(r["tokens"]) == x + [y] and r["tau"] == K + 1 and r["kv_out"] == 5 + K + 1


# ------------------------------------------------------------------------------ inverse CDF
@pytest.mark.parametrize("w,u,y", [
    ([0.25, 0.0, 0.25, 0.5], 0.0, 0),     # running sums .25 .25 .5 1; first above 0 -> 0
    ([0.25, 0.0, 0.25, 0.5], 0.25, 2),    # first strictly above .25 is index 2; the zero-weight
                                          # token 1 is never drawn
    ([0.25, 0.0, 0.25, 0.5], 0.5, 3),     # .5 is not above .5 -> 3
    ([0.25, 0.0, 0.25, 0.5], U_MAX, 3),
    ([1.0, 0.0, 3.0], 0.25, 2),           # unnormalised: Z = 4, threshold 1, sums 1 1 4 -> 2
    ([0.5, 0.5, 0.0, 0.0], 0.99, 1),      # trailing zero weights are never drawn
    ([0.5, 0.5, 0.0, 0.0], 1.0, 1),       # u = 1 (outside [0,1)) reaches the fallback: the last
                                          # token of positive weight
])
def test_inverse_cdf_hand_cases(w, u, y):
    assert oracle.inverse_cdf(np.array(w), u)[0] == y


# ------------------------------------------------------------------------------ greedy / top-F
def test_greedy_ties_go_to_lowest_id():
    """Row 0 has its maximum 2.0 at ids 1 and 3 -> 1 (draft 1 kept); row 1 has 5.0 at ids 0 and 2
    -> 0, draft 2 differs, so 0 is placed and tau = 2."""
    t_rows = np.array([[0.0, 2.0, 1.0, 2.0], [5.0, 1.0, 5.0, 0.0], [0.0, 0.0, 0.0, 0.0]])
    r = oracle.verify_greedy_request(t_rows, [1, 2], 0)
    assert list(r["tokens"]) == [1, 0, -1] and r["tau"] == 2


def test_greedy_all_masked_row_picks_id_zero():
    t_rows = np.array([[-np.inf, -np.inf, -np.inf], [1.0, 2.0, 3.0]])
    r = oracle.verify_greedy_request(t_rows, [0], 0)
    assert list(r["tokens"]) == [0, 2] and r["tau"] == 2


@pytest.mark.parametrize("row,F,keys", [
    ([1.0, 3.0, 3.0, 2.0], 3, [1, 2, 3]),          # equal logits: lower id first
    ([-np.inf, 0.5, -np.inf, 0.5], 3, [1, 3, 0]),  # masked tokens come last, lowest id first
    ([2.0, 2.0, 2.0, 2.0], 2, [0, 1]),
])
def test_top_f_order(row, F, keys):
    k, p = oracle.predict_request(np.array([row]), F, 0.0)
    assert list(k[0]) == keys
    assert list(p[0]) == [1.0] + [0.0] * (F - 1)


def test_top_f_probabilities():
    """logits (0, ln 3) at T = 1: keys (1, 0) with q = (3/4, 1/4)."""
    k, p = oracle.predict_request(np.array([[0.0, LN3]]), 2, 1.0)
    assert list(k[0]) == [1, 0]
    np.testing.assert_allclose(p[0], [0.75, 0.25], atol=1e-15)


# ------------------------------------------------------------------------------ row errors
@pytest.mark.parametrize("bad", [-1, 4, 1 << 30])
def test_out_of_range_draft_token_is_a_row_error(bad):
    t_rows = np.zeros((3, 4))
    d_rows = np.zeros((2, 4))
    r = oracle.verify_sample_request(t_rows, d_rows, [1, bad], np.array([0.1, 0.2, 0.3]), 9, 1.0)
    assert r["row_error"] and r["tau"] == -1 and r["kv_out"] == 9
    assert list(r["tokens"]) == [-1, -1, -1] and np.all(np.isnan(r["p_x"]))
    g = oracle.verify_greedy_request(t_rows, [1, bad], 9)
    assert g["row_error"] and g["tau"] == -1 and list(g["tokens"]) == [-1, -1, -1]


def test_masked_draft_token_is_a_row_error_when_sampling_only():
    t_rows = np.zeros((2, 3))
    d_rows = np.array([[0.0, -np.inf, 0.0]])
    r = oracle.verify_sample_request(t_rows, d_rows, [1], np.array([0.1, 0.2]), 0, 1.0)
    assert r["row_error"] and r["tau"] == -1
    g = oracle.verify_greedy_request(t_rows, [1], 0)       # greedy never reads draft logits
    assert not g["row_error"] and g["tau"] == 1 and g["y"] == 0


def test_masked_target_token_is_always_rejected():
    """p(x) = 0 (target logit -inf) gives ratio 0: rejected even at u = 0."""
    t_rows = np.array([[-np.inf, 0.0], [0.0, 0.0]])
    d_rows = np.array([[0.0, 0.0]])
    r = oracle.verify_sample_request(t_rows, d_rows, [0], np.array([0.0, 0.0]), 0, 1.0)
    assert r["tau"] == 1 and r["y"] == 1


# ------------------------------------------------------------------------------ hit rule
def test_hit_rule_page_examples():
    """D3D page, sections ヒット / ミス: five kept and the sixth rejected (m = 5); the token the
    target placed is one of the two prepared candidates -> hit; not one of them -> miss; a
    rejection at the twelfth draft or later (m >= 11) when eleven slots are prepared -> miss."""
    K = 15
    keys = np.zeros((K, 2), np.int64)
    keys[5] = [42, 17]
    assert oracle.outcome_hit(keys, 5, 17, K, positions=11)
    assert not oracle.outcome_hit(keys, 5, 99, K, positions=11)
    keys[11] = [7, 8]
    assert not oracle.outcome_hit(keys, 11, 7, K, positions=11)
    assert oracle.outcome_hit(keys, 11, 7, K)              # no position limit
    assert not oracle.outcome_hit(keys, K, 0, K)           # every draft kept: no key
    assert not oracle.outcome_hit(keys, -1, 0, K)          # row error
