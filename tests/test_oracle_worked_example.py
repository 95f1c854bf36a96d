"""Pins the oracle to the worked greedy round printed on the D3D illustrated page
("LLMの生成を5倍速くする「D3D」を図で読む", sections 検証のしくみ①, 検証のしくみ③ and
検証のまとめ): five drafts, three kept, the target's own token placed, tau = 4.

The fixture under tests/golden/ holds the page's tokens and outcome; the logits below are built
from it (the page gives only each row's top choice), so any logits with those top choices must
give the page's result."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import naive

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "worked_example_greedy.json"), encoding="utf-8"))
VOCAB = GOLD["vocab"]
ID = {w: i for i, w in enumerate(VOCAB)}
V = len(VOCAB)


def rows_with_top_choices(choices, last_choice, gap, seed):
    """Logit rows whose argmax is the given token; background values in [-1, 0]."""
    rng = np.random.default_rng(seed)
    rows = rng.uniform(-1.0, 0.0, size=(len(choices), V))
    for k, w in enumerate(choices):
        rows[k, ID[w] if w is not None else last_choice] = gap
    return rows


@pytest.mark.parametrize("last_choice", range(V))
@pytest.mark.parametrize("seed", [0, 1])
def test_greedy_worked_example(last_choice, seed):
    x = [ID[w] for w in GOLD["drafts"]]
    rows = rows_with_top_choices(GOLD["target_top_choice_per_row"], last_choice, 5.0, seed)
    r = oracle.verify_greedy_request(rows, x, kv_in=100)
    exp = GOLD["expected"]
    assert r["tau"] == exp["tau"] == 4
    assert [VOCAB[t] for t in r["tokens"][:r["tau"]]] == exp["emitted"]
    assert list(r["tokens"][r["tau"]:]) == [-1] * (len(x) + 1 - exp["tau"])
    assert r["m"] == len(exp["accepted"])
    assert VOCAB[r["y"]] == exp["placed"]
    assert r["kv_out"] == 100 + exp["tau"]
    tokens, tau, kv = naive.naive_verify_greedy(rows.tolist(), x, 100)
    assert tokens == list(r["tokens"]) and tau == 4 and kv == 104


@pytest.mark.parametrize("last_choice", [0, 5, 7])
def test_greedy_bonus_variant(last_choice):
    bv = GOLD["bonus_variant"]
    x = [ID[w] for w in bv["drafts"]]
    rows = rows_with_top_choices(GOLD["target_top_choice_per_row"], last_choice, 5.0, 3)
    r = oracle.verify_greedy_request(rows, x, kv_in=7)
    assert r["tau"] == bv["expected_tau"] == 6
    assert list(r["tokens"]) == x + [last_choice]
    assert r["kv_out"] == 13


@pytest.mark.parametrize("u", [
    [0.0] * 6,
    [0.5] * 6,
    [np.float32(1) - np.float32(2 ** -24)] * 6,
    [0.3, 0.9, 0.1, 0.7, 0.2, 0.6],
])
@pytest.mark.parametrize("bonus", [False, True])
def test_sampling_reduces_to_greedy_at_tiny_temperature(u, bonus):
    """At T = 0.01 with a logit gap of 10 every softmax is exactly one-hot in float64
    (exp(-1000) underflows to 0), so sampling verification must reproduce the greedy outcome for
    every choice of uniforms."""
    drafts = GOLD["bonus_variant"]["drafts"] if bonus else GOLD["drafts"]
    x = [ID[w] for w in drafts]
    t_rows = rows_with_top_choices(GOLD["target_top_choice_per_row"], 2, 10.0, 4)
    d_rows = rows_with_top_choices(drafts, None, 10.0, 5)
    g = oracle.verify_greedy_request(t_rows, x, kv_in=0)
    s = oracle.verify_sample_request(t_rows, d_rows, x, np.array(u, np.float64), 0, 0.01)
    assert list(s["tokens"]) == list(g["tokens"])
    assert s["tau"] == g["tau"] == (6 if bonus else 4)
