"""The oracle at tiny temperatures: sampling approaches the greedy rule ("speculative decodingとは",
stage 3: temperature zero keeps a draft while it is the target's top choice), and the accept ratio
p/q stays exact when p and q themselves underflow in float64."""
import numpy as np
import pytest

import oracle

TINY = [1e-3, 1e-6, 1e-12, 1e-30]


@pytest.mark.parametrize("T", TINY)
def test_ratio_when_both_probabilities_underflow(T):
    """Target logits (0, 2), draft (0, 1), draft token 0. p(0) = 1/(1 + e^(2/T)) and
    q(0) = 1/(1 + e^(1/T)) are both 0 in float64 for T <= 1e-3, but p/q = e^(-1/T)(1 + ...) is
    at most e^(-1000): the draft is rejected for every u in (0, 1). The residual
    max(0, p - q) has all its mass on token 1 (p(1) > q(1)), so token 1 is placed: tau = 1, as
    the greedy rule gives (the target's top choice is 1)."""
    t = np.array([[0.0, 2.0], [0.0, 0.0]])
    d = np.array([[0.0, 1.0]])
    for u0 in (1e-7, 0.5, 0.999):
        r = oracle.verify_sample_request(t, d, [0], np.array([u0, 0.3]), 5, T)
        assert r["tau"] == 1 and list(r["tokens"]) == [1, -1] and r["kv_out"] == 6
        assert r["p_x"][0] == 0.0 and r["q_x"][0] == 0.0
        assert r["accept_margins"][0] == pytest.approx(u0)


@pytest.mark.parametrize("T", TINY)
def test_draft_less_unlikely_under_target_is_kept(T):
    """Target (0, 1), draft (0, 2), token 0: p(0)/q(0) > 1, kept for every u."""
    t = np.array([[0.0, 1.0], [0.0, 0.0]])
    d = np.array([[0.0, 2.0]])
    r = oracle.verify_sample_request(t, d, [0], np.array([0.999, 0.3]), 0, T)
    assert r["tau"] == 2 and r["tokens"][0] == 0


@pytest.mark.parametrize("T", TINY)
def test_sampling_equals_greedy_in_the_limit(T):
    """Random tiny requests without tied maxima, drafts equal to the draft model's top choices
    (what it samples as T -> 0): sampling at a tiny T gives the greedy outcome for every u."""
    rng = np.random.default_rng(5)
    for _ in range(40):
        K, V = int(rng.integers(1, 5)), int(rng.integers(2, 12))
        t = rng.normal(0, 3, size=(K + 1, V))
        d = t[:K] + rng.normal(0, 2, size=(K, V))
        x = [int(np.argmax(d[k])) for k in range(K)]
        g = oracle.verify_greedy_request(t, x, 100)
        for _ in range(5):
            u = rng.random(K + 1, dtype=np.float32).astype(np.float64)
            r = oracle.verify_sample_request(t, d, x, u, 100, T)
            assert r["tau"] == g["tau"] and np.array_equal(r["tokens"], g["tokens"])
            assert r["kv_out"] == g["kv_out"]
            np.testing.assert_allclose(r["p_x"], [1.0 if x[k] == g["g"][k] else 0.0
                                                  for k in range(K)], rtol=0, atol=1e-12)


@pytest.mark.parametrize("T", TINY)
def test_point_mass_equals_greedy_in_the_limit(T):
    """Point-mass drafts at a tiny T: p_k(x_k) is 1 for the target's top choice and 0 otherwise,
    so the outcome is the greedy rule's over the first n slots."""
    rng = np.random.default_rng(6)
    for _ in range(40):
        K, V = int(rng.integers(1, 5)), int(rng.integers(2, 12))
        t = rng.normal(0, 3, size=(K + 1, V))
        x = rng.integers(0, V, size=K)
        x[: K // 2] = np.argmax(t[: K // 2], axis=1)
        n = int(rng.integers(0, K + 1))
        g = oracle.verify_point_request(t, x, n, np.zeros(K + 1), 0, 0.0)
        u = rng.random(K + 1, dtype=np.float32).astype(np.float64)
        u[u == 0.0] = 0.5
        r = oracle.verify_point_request(t, x, n, u, 0, T)
        assert r["tau"] == g["tau"] and np.array_equal(r["tokens"], g["tokens"])


def test_tiny_temperatures_are_valid():
    """T = 1e-30 gives log2(e)/T = 1.44e30, finite in float32: a valid temperature; only T with
    log2(e)/T beyond float32's range (T below ~4.2e-39) is not."""
    for T in TINY:
        assert oracle.temperature_is_valid(float(np.float32(T)))
    assert not oracle.temperature_is_valid(1e-39)
