"""Cross-checks the vectorised oracle against the literal pure-Python statement of the same rules
on many tiny random inputs, including equal logits, masked (-inf) tokens and out-of-range draft
tokens. Emitted tokens, tau and kv must agree exactly; probabilities to 1e-12."""
import numpy as np
import pytest

import oracle
from oracle import naive
from synthetic import make_tiny_random

SHAPES = [(1, 2), (2, 3), (3, 5), (4, 8), (2, 16), (5, 7)]


def _decode(wl):
    return (oracle.decode_logits(wl.target, wl.dtype), oracle.decode_logits(wl.draft, wl.dtype))


@pytest.mark.parametrize("K,V", SHAPES)
@pytest.mark.parametrize("T", [1.0, 0.7, 2.5])
@pytest.mark.parametrize("ties,neg_inf,bad,dtype", [
    (True, 0.0, 0.0, "f32"), (True, 0.2, 0.05, "f32"), (False, 0.1, 0.0, "bf16"),
])
def test_sampling_matches_naive(K, V, T, ties, neg_inf, bad, dtype):
    for seed in range(6):
        wl = make_tiny_random(seed * 31 + K * 7 + V, B=4, K=K, V=V, T=T, dtype=dtype, ties=ties,
                              neg_inf=neg_inf, bad_token_rate=bad)
        t, d = _decode(wl)
        res = oracle.verify_sample(wl.target, wl.draft, wl.dtype, wl.tokens, wl.uniforms,
                                   wl.kv_len, wl.T)
        for b in range(wl.B):
            tok, tau, kv, px, qx = naive.naive_verify_sample(
                t[b], d[b], wl.tokens[b], wl.uniforms[b].astype(np.float64), wl.kv_len[b],
                float(wl.T))
            assert list(res["tokens"][b]) == tok
            assert res["tau"][b] == tau and res["kv_out"][b] == kv
            np.testing.assert_allclose(res["p_x"][b], px, rtol=0, atol=1e-12)
            np.testing.assert_allclose(res["q_x"][b], qx, rtol=0, atol=1e-12)


@pytest.mark.parametrize("K,V", SHAPES)
def test_greedy_matches_naive(K, V):
    for seed in range(8):
        wl = make_tiny_random(seed + 500, B=4, K=K, V=V, mode="greedy", ties=True, neg_inf=0.2,
                              bad_token_rate=0.05)
        t, _ = _decode(wl)
        res = oracle.verify_greedy(wl.target, wl.dtype, wl.tokens, wl.kv_len)
        for b in range(wl.B):
            tok, tau, kv = naive.naive_verify_greedy(t[b], wl.tokens[b], wl.kv_len[b])
            assert list(res["tokens"][b]) == tok and res["tau"][b] == tau
            assert res["kv_out"][b] == kv


@pytest.mark.parametrize("K,V", SHAPES)
@pytest.mark.parametrize("T", [0.0, 1.0, 0.7])
def test_predict_matches_naive(K, V, T):
    for seed in range(4):
        wl = make_tiny_random(seed + 900, B=3, K=K, V=V, ties=True, neg_inf=0.2)
        _, d = _decode(wl)
        for F in sorted({1, min(3, V), V}):
            res = oracle.predict_outcomes(wl.draft, wl.dtype, F, T)
            for b in range(wl.B):
                keys, probs = naive.naive_predict(d[b], F, float(np.float32(T)))
                assert res["keys"][b].tolist() == keys
                np.testing.assert_allclose(res["key_prob"][b], probs, rtol=0, atol=1e-12)
