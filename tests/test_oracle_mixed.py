"""Pins of the mixed-batch rule (a temperature per request): each request verified at T_b = 0
by the greedy rule and at T_b > 0 by speculative sampling, checked against the separately pinned
single-rule oracles; the temperature-zero probabilities worked by hand; invalid temperatures."""
import math

import numpy as np
import pytest

import oracle


def test_hand_worked_greedy_request():
    # K = 2, V = 3; target rows' top choices 2, 0, 1; drafts (2, 1): the first kept, the second
    # rejected, token 0 placed, tau = 2; p reports the top-choice indicator, q is 1
    t = np.array([[0.0, 1.0, 5.0], [4.0, 1.0, 0.0], [0.0, 3.0, 1.0]])
    d = np.zeros((2, 3))
    r = oracle.verify_mixed_request(t, d, [2, 1], [0.5, 0.5, 0.5], 10, 0.0)
    assert list(r["tokens"]) == [2, 0, -1] and r["tau"] == 2 and r["kv_out"] == 12
    assert list(r["p_x"]) == [1.0, 0.0] and list(r["q_x"]) == [1.0, 1.0]


@pytest.mark.parametrize("T", [-1.0, math.nan, math.inf, 1e-45])
def test_invalid_temperature_is_a_row_error(T):
    t = np.zeros((2, 4))
    r = oracle.verify_mixed_request(t, np.zeros((1, 4)), [0], [0.1, 0.2], 7, T)
    assert r["row_error"] and r["tau"] == -1 and r["kv_out"] == 7
    assert np.all(r["tokens"] == -1) and np.all(np.isnan(r["p_x"]))


def test_temperature_validity_boundary():
    assert oracle.temperature_is_valid(0.0) and oracle.temperature_is_valid(1e-30)
    assert not oracle.temperature_is_valid(1e-39)          # log2(e)/T overflows float32
    assert not oracle.temperature_is_valid(-0.5)


def test_composition_matches_the_single_rule_oracles():
    rng = np.random.default_rng(21)
    for trial in range(120):
        K, V = int(rng.integers(1, 5)), int(rng.integers(2, 9))
        t = rng.normal(0, 2, size=(K + 1, V))
        d = t[:K] + rng.normal(0, 1, size=(K, V))
        x = rng.integers(0, V, size=K)
        u = rng.random(K + 1)
        T = [0.0, 0.7, 1.3][trial % 3]
        r = oracle.verify_mixed_request(t, d, x, u, 5, T)
        if T == 0.0:
            g = oracle.verify_greedy_request(t, x, 5)
            assert list(r["tokens"]) == list(g["tokens"]) and r["tau"] == g["tau"]
            assert list(r["p_x"]) == [1.0 if x[k] == np.argmax(t[k]) else 0.0 for k in range(K)]
        else:
            s = oracle.verify_sample_request(t, d, x, u, 5, T)
            assert list(r["tokens"]) == list(s["tokens"]) and r["tau"] == s["tau"]
            np.testing.assert_array_equal(r["p_x"], s["p_x"])
