"""Pins of the per-slot fan-out oracle (prepared outcomes in the manner of D3D): the page's
prepared-token table, its hit and miss examples, the "2nd and 3rd candidates" rule worked by
hand, the invariant that makes excluding the draft token free (a rejected draft token is never
the placed token), and a brute-force cross-check against the naive statement of the rules."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.naive import naive_outcome_slot, naive_predict_fanout

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "fanout_budget_d3d.json")


@pytest.fixture(scope="module")
def page():
    with open(GOLDEN, encoding="utf-8") as fh:
        return json.load(fh)


def test_budget_matches_the_page_table(page):
    for s in page["settings"]:
        fanout = [s["candidates"]] * s["positions"]
        assert oracle.fanout_budget(fanout, page["block_tokens"]) == s["prepared_tokens"], s


def test_page_hit_and_miss_examples(page):
    """K = 15 drafts, 11 prepared positions with 2 candidates each. The draft rows are built so
    that slot k's candidates (top choices other than the draft token) are known by hand."""
    K, P, F = page["drafts_per_block"], 11, 2
    V = 40
    d = np.zeros((K, V))
    x = np.zeros(K, np.int64)
    for k in range(K):
        x[k] = k                     # the draft token: the row's top logit
        d[k, k] = 10.0
        d[k, 20 + k] = 9.0           # 2nd choice
        d[k, 21 + k] = 8.0           # 3rd choice
    keys, _ = oracle.predict_fanout_request(d, x, [F] * P, 1.0)
    assert keys.shape == (P * F,)
    assert list(keys[10:12]) == [25, 26]          # slot 5 (the 6th draft): 2nd and 3rd choices
    for ex in page["hit_miss_examples"]:
        m = ex["kept"]
        if m == K:
            y = 7
        elif ex["placed_among_candidates"]:
            y = 20 + m + 1                            # the 3rd choice of slot m
        else:
            y = 39
        slot = oracle.outcome_slot(keys, [F] * P, K, m, y)
        assert (slot >= 0) == (ex["expected"] == "hit"), ex
        if m == 5 and ex["placed_among_candidates"]:
            assert slot == 5 * F + 1
        if m == K:
            assert slot == P * F                      # the all-accept continuation is last
            assert oracle.outcome_slot(keys, [F] * P, K, m, y, all_accept=False) == -1


def test_second_and_third_candidates_by_hand():
    # logits 5 9 7 8 1: order by value is ids 1, 3, 2, 0, 4
    row = np.array([[5.0, 9.0, 7.0, 8.0, 1.0]])
    keys, prob = oracle.predict_fanout_request(row, [1], [2], 0.0)     # greedy draft = argmax
    assert list(keys) == [3, 2] and list(prob) == [0.0, 0.0]
    keys, prob = oracle.predict_fanout_request(row, None, [2], 0.0)    # no exclusion
    assert list(keys) == [1, 3] and list(prob) == [1.0, 0.0]
    keys, prob = oracle.predict_fanout_request(row, [2], [2], 0.0)     # a sampled draft token
    assert list(keys) == [1, 3] and list(prob) == [1.0, 0.0]
    # equal logits: lowest id first, the draft token skipped
    keys, _ = oracle.predict_fanout_request(np.array([[2.0, 2.0, 2.0, 1.0]]), [0], [2], 1.0)
    assert list(keys) == [1, 2]
    # T > 0: key probabilities are the draft softmax at the keys; logits (0, ln 3) -> (1/4, 3/4)
    keys, prob = oracle.predict_fanout_request(np.array([[0.0, np.log(3.0)]]), None, [2], 1.0)
    assert list(keys) == [1, 0]
    np.testing.assert_allclose(prob, [0.75, 0.25], rtol=0, atol=1e-15)
    # a zero fan-out slot has no keys; offsets follow the fan-out
    keys, _ = oracle.predict_fanout_request(np.vstack([row, row, row]), None, [1, 0, 2], 1.0)
    assert list(keys) == [1, 1, 3]
    assert list(oracle.fanout_offsets([1, 0, 2])) == [0, 1, 1, 3]


def _random_request(rng, K, V, T):
    t = rng.normal(0.0, 2.0, size=(K + 1, V))
    d = t[:K] + rng.normal(0.0, 1.0, size=(K, V))
    if T > 0:
        q = np.exp((d - d.max(axis=1, keepdims=True)) / T)
        q /= q.sum(axis=1, keepdims=True)
        x = np.array([rng.choice(V, p=q[k]) for k in range(K)])
    else:
        x = d.argmax(axis=1)
    return t, d, x


@pytest.mark.parametrize("T", [0.0, 0.7, 1.0])
def test_rejected_draft_token_is_never_placed_so_excluding_it_never_loses(T):
    """After a rejection at slot m the placed token is never x_m: in sampling its residual
    weight max(0, p - q) is 0 because rejection needs p(x_m) < q(x_m); in greedy the placed
    token is the target's top choice, which differs from x_m by definition of a mismatch. So
    with the same fan-out, keys that skip x_m hit whenever keys that keep it do (and at T = 0
    with greedy drafts the top draft choice, x_m itself, never hits)."""
    rng = np.random.default_rng(11)
    K, V, F = 4, 6, 2
    for trial in range(300):
        t, d, x = _random_request(rng, K, V, T)
        if T > 0:
            u = rng.random(K + 1)
            r = oracle.verify_sample_request(t, d, x, u, 0, T)
        else:
            r = oracle.verify_greedy_request(t, x, 0)
        m, y = r["m"], r["y"]
        if m < K:
            assert y != x[m], trial
        ke, _ = oracle.predict_fanout_request(d, x, [F] * K, T)
        kn, _ = oracle.predict_fanout_request(d, None, [F] * K, T)
        se = oracle.outcome_slot(ke, [F] * K, K, m, y)
        sn = oracle.outcome_slot(kn, [F] * K, K, m, y)
        assert sn < 0 or se >= 0, trial
        if T == 0 and m < K:
            k1, _ = oracle.predict_fanout_request(d, None, [1] * K, 0.0)
            assert oracle.outcome_slot(k1, [1] * K, K, m, y) == -1


def test_reference_matches_naive_on_random_tiny_inputs():
    rng = np.random.default_rng(5)
    for trial in range(200):
        K = int(rng.integers(1, 5))
        V = int(rng.integers(3, 12))
        fanout = [int(rng.integers(0, V)) for _ in range(int(rng.integers(1, K + 1)))]
        d = rng.integers(-3, 3, size=(K, V)).astype(np.float64)     # many exact ties
        d[rng.random((K, V)) < 0.15] = -np.inf
        d[:, 0] = np.where(np.isinf(d).all(axis=1), 0.0, d[:, 0])   # keep a finite logit per row
        x = rng.integers(0, V, size=K) if trial % 3 else None
        T = [0.0, 0.5, 1.0][trial % 3]
        keys, prob = oracle.predict_fanout_request(d, x, fanout, T)
        nk, npr = naive_predict_fanout(d, x, fanout, T)
        assert list(keys) == nk, trial
        np.testing.assert_allclose(prob, npr, rtol=0, atol=1e-12)
        for _ in range(5):
            m = int(rng.integers(-1, K + 1))
            y = int(rng.integers(0, V))
            aa = bool(rng.integers(0, 2))
            assert oracle.outcome_slot(keys, fanout, K, m, y, aa) == \
                naive_outcome_slot(nk, fanout, K, m, y, aa), trial
