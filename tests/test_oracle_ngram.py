"""Pins of the oracle's prompt-lookup drafter and of its verification of drafts that carry no
distribution (CPU only).

Drafter: hand-worked cases (tests/golden/ngram_lookup_examples.json), Python's own substring
search (str.rfind finds the latest occurrence of a substring that lies wholly inside a range),
the literal loops of oracle.naive, and the invariants that define the match.
Verification: on the first n slots it must be the speculative-sampling rule with a draft that
puts all its mass on its token (the oracle's own sampling rule, pinned elsewhere, fed one-hot
draft logits and the same uniforms), the greedy rule at T = 0, a hand-worked case, and the
emitted token's distribution must be the target's (seeded Monte Carlo).
"""
import json
import math
import pathlib

import numpy as np
import pytest

import oracle
from oracle.naive import naive_ngram_draft

GOLDEN = pathlib.Path(__file__).parent / "golden" / "ngram_lookup_examples.json"


def _golden_cases():
    return json.loads(GOLDEN.read_text())["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_ngram_golden(case):
    r = oracle.ngram_draft_request(case["ctx"], case["n_max"], case["n_min"], case["K"])
    assert list(r["tokens"]) == case["tokens"]
    assert (r["length"], r["n"], r["src"]) == (case["length"], case["n"], case["src"])
    assert naive_ngram_draft(case["ctx"], case["n_max"], case["n_min"], case["K"]) == (
        case["tokens"], case["length"], case["n"], case["src"])


def _as_text(tokens):
    # one code point per token id: substring search on the text is span search on the tokens
    return "".join(chr(0x100 + int(t)) for t in tokens)


def _rfind_draft(ctx, n_max, n_min, K):
    s = _as_text(ctx)
    L = len(ctx)
    for n in range(min(n_max, L - 1), n_min - 1, -1):
        # an occurrence lying wholly in s[0 : L-1] starts at j <= L-n-1
        j = s.rfind(s[L - n:], 0, L - 1)
        if j >= 0:
            src = j + n
            length = min(K, L - src)
            return [int(t) for t in ctx[src:src + length]] + [-1] * (K - length), length, n, src
    return [-1] * K, 0, 0, -1


@pytest.mark.parametrize("seed", range(40))
def test_ngram_matches_substring_search_and_loops(seed):
    rng = np.random.default_rng(9100 + seed)
    alphabet = int(rng.integers(2, 7))          # small alphabets make many matches
    L = int(rng.integers(0, 60))
    ctx = rng.integers(0, alphabet, L)
    n_max = int(rng.integers(1, 7))
    n_min = int(rng.integers(1, n_max + 1))
    K = int(rng.integers(1, 9))
    r = oracle.ngram_draft_request(ctx, n_max, n_min, K)
    got = (list(r["tokens"]), r["length"], r["n"], r["src"])
    assert got == _rfind_draft(list(ctx), n_max, n_min, K)
    assert got == naive_ngram_draft(ctx, n_max, n_min, K)


@pytest.mark.parametrize("seed", range(20))
def test_ngram_invariants(seed):
    rng = np.random.default_rng(9300 + seed)
    L = int(rng.integers(2, 400))
    ctx = rng.integers(0, 5, L)
    n_max, n_min, K = 5, 1, 6
    r = oracle.ngram_draft_request(ctx, n_max, n_min, K)
    n, src, length = r["n"], r["src"], r["length"]
    assert length >= 1 and 1 <= n <= n_max   # a 5-letter alphabet always repeats its last token
    # the span before src equals the suffix, and starts before the suffix does
    assert list(ctx[src - n:src]) == list(ctx[L - n:]) and src - n <= L - n - 1
    # nothing longer (up to n_max) occurs earlier
    for n2 in range(n + 1, min(n_max, L - 1) + 1):
        suf = list(ctx[L - n2:])
        assert not any(list(ctx[j:j + n2]) == suf for j in range(0, L - n2))
    # no later occurrence of the same span
    for j in range(src - n + 1, L - n):
        assert list(ctx[j:j + n]) != list(ctx[L - n:])
    assert length == min(K, L - src)
    assert list(r["tokens"][:length]) == list(ctx[src:src + length])
    assert all(t == -1 for t in r["tokens"][length:])


def test_ngram_batch_row_errors():
    ctx = np.array([[1, 2, 1, 2, 0, 0], [5, 6, 7, 5, 6, 9]])
    r = oracle.ngram_draft(ctx, np.array([4, 7]), 2, 1, 3)
    assert list(r["length"]) == [2, -1]
    assert list(r["tokens"][0]) == [1, 2, -1] and list(r["tokens"][1]) == [-1, -1, -1]
    assert list(r["src"]) == [2, -1] and list(r["n"]) == [2, 0]
    r = oracle.ngram_draft(ctx, np.array([-1, 0]), 2, 1, 3)
    assert list(r["length"]) == [-1, 0]


# ------------------------------------------------------------------------------ verification
def _one_hot_logits(x, V):
    d = np.full((len(x), V), -np.inf)
    for k, t in enumerate(x):
        d[k, int(t)] = 0.0
    return d


def _same(a, b):
    np.testing.assert_array_equal(a["tokens"], b["tokens"])
    assert (a["tau"], a["kv_out"], a["m"], a["y"], a["row_error"]) == (
        b["tau"], b["kv_out"], b["m"], b["y"], b["row_error"])


@pytest.mark.parametrize("seed", range(30))
def test_point_is_sampling_with_one_hot_draft(seed):
    rng = np.random.default_rng(9500 + seed)
    K = int(rng.integers(1, 6))
    V = int(rng.integers(2, 12))
    T = float(rng.choice([0.5, 1.0, 1.7]))
    t_rows = rng.normal(0, 2, (K + 1, V))
    x = rng.integers(0, V, K)
    u = rng.random(K + 1)
    n = int(rng.integers(0, K + 1))
    got = oracle.verify_point_request(t_rows, x, n, u, 17, T)
    # the first n slots as a K' = n problem: rows 0..n, its uniforms u_0..u_{n-1} and the draw's u_K
    ref = oracle.verify_sample_request(t_rows[:n + 1], _one_hot_logits(x[:n], V), x[:n],
                                       np.concatenate([u[:n], u[K:]]), 17, T)
    assert got["m"] == ref["m"] and got["y"] == ref["y"]
    assert got["tau"] == ref["tau"] and got["kv_out"] == ref["kv_out"]
    np.testing.assert_array_equal(got["tokens"][:n + 1], ref["tokens"])
    assert np.all(got["tokens"][n + 1:] == -1)
    np.testing.assert_allclose(got["p_x"][:n], ref["p_x"], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(got["q_x"][:n], np.ones(n))
    assert np.all(np.isnan(got["p_x"][n:])) and np.all(np.isnan(got["q_x"][n:]))


@pytest.mark.parametrize("seed", range(20))
def test_point_at_zero_temperature_is_greedy(seed):
    rng = np.random.default_rng(9700 + seed)
    K = int(rng.integers(1, 6))
    V = int(rng.integers(2, 9))
    t_rows = rng.integers(-3, 3, (K + 1, V)).astype(np.float64)   # many ties
    g = np.argmax(t_rows, axis=1)
    x = np.where(rng.random(K) < 0.7, g[:K], rng.integers(0, V, K))
    n = int(rng.integers(0, K + 1))
    got = oracle.verify_point_request(t_rows, x, n, rng.random(K + 1), 3, 0.0)
    ref = oracle.verify_greedy_request(t_rows[:n + 1], x[:n], 3)
    assert got["m"] == ref["m"] and got["y"] == ref["y"] and got["tau"] == ref["tau"]
    np.testing.assert_array_equal(got["tokens"][:n + 1], ref["tokens"])
    np.testing.assert_array_equal(got["p_x"][:n], (x[:n] == g[:n]).astype(float))


def test_point_hand_worked():
    # p at T = 1 is (1, 2, 3, 4) / 10; the draft proposes token 3 (p = 0.4)
    t = np.log(np.array([[1.0, 2.0, 3.0, 4.0], [4.0, 3.0, 2.0, 1.0]]))
    kept = oracle.verify_point_request(t, [3], 1, [0.3, 0.05], 0, 1.0)
    # 0.3 < 0.4: kept; the bonus row (0.4, 0.3, 0.2, 0.1) with u = 0.05 gives token 0
    assert list(kept["tokens"]) == [3, 0] and kept["tau"] == 2 and kept["kv_out"] == 2
    assert math.isclose(kept["p_x"][0], 0.4, rel_tol=1e-12) and kept["q_x"][0] == 1.0
    rej = oracle.verify_point_request(t, [3], 1, [0.5, 0.25], 0, 1.0)
    # 0.5 >= 0.4: rejected; residual (0.1, 0.2, 0.3, 0) with mass 0.6; 0.25 * 0.6 = 0.15 lies in
    # (0.1, 0.3], token 1
    assert list(rej["tokens"]) == [1, -1] and rej["tau"] == 1 and rej["m"] == 0
    assert math.isclose(rej["resid_mass"], 0.6, rel_tol=1e-12)
    # nothing drafted: the first row is the bonus row; u_K = 0.65 lands in (0.6, 1.0], token 3
    none = oracle.verify_point_request(t, [2], 0, [0.9, 0.65], 5, 1.0)
    assert list(none["tokens"]) == [3, -1] and none["tau"] == 1 and none["kv_out"] == 6
    assert np.isnan(none["p_x"][0])


def test_point_row_errors():
    t = np.zeros((3, 4))
    for n, x in ((3, [0, 1]), (-1, [0, 1]), (2, [0, 4]), (1, [-1, 0])):
        r = oracle.verify_point_request(t, x, n, [0.1, 0.2, 0.3], 9, 1.0)
        assert r["row_error"] and r["tau"] == -1 and r["kv_out"] == 9
        assert np.all(r["tokens"] == -1) and np.all(np.isnan(r["p_x"]))
    # an undrafted slot may hold anything
    r = oracle.verify_point_request(t, [0, -7], 1, [0.1, 0.2, 0.3], 9, 1.0)
    assert not r["row_error"]


def test_point_emits_the_target_distribution():
    # [SD] FAQ on output quality: whatever proposes the token, the emitted token follows the
    # target. Seeded Monte Carlo over (u_0, u_K) for a fixed deterministic draft.
    rng = np.random.default_rng(9901)
    t_row = np.log(np.array([0.05, 0.15, 0.5, 0.3]))
    t = np.stack([t_row, np.zeros(4)])
    p = np.exp(t_row) / np.exp(t_row).sum()
    N = 20000
    counts = np.zeros(4)
    for _ in range(N):
        r = oracle.verify_point_request(t, [2], 1, rng.random(2), 0, 1.0)
        counts[r["tokens"][0]] += 1
    sigma = np.sqrt(p * (1 - p) / N)
    assert np.all(np.abs(counts / N - p) < 4.5 * sigma)
