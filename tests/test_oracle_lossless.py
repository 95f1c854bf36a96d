"""Pins the sampling oracle by exact enumeration: with drafts x ~ q and uniforms u ~ U[0,1), the
tokens it emits must follow the target's own autoregressive distribution (the losslessness the
pages state: "speculative decodingとは", FAQ on output quality, and stage 4 of the four-stage
loop; the D3D page's 検証のまとめ).

The test never restates the acceptance ratio or the residual. It treats the oracle as a black
box (x, u) -> emitted tokens and finds where that map changes by bisection over each uniform:
the accept threshold of every slot and the token boundaries of the final draw. Summing the
exact measures of those u-intervals, weighted by q(x), gives the emitted distribution, which is
compared with products of target conditionals over all length-(K+1) continuations.
"""
import itertools

import numpy as np
import pytest

import oracle
import oracle.reference as ref

ONE_MINUS = float(np.nextafter(1.0, 0.0))


def random_tables(rng, V, K, zero_rate=0.2):
    """Prefix-conditioned target tables (prefix length 0..K) and draft tables (0..K-1)."""
    def dist():
        p = rng.dirichlet(np.ones(V))
        z = rng.random(V) < zero_rate
        z[rng.integers(V)] = False
        p[z] = 0.0
        return p / p.sum()
    P, Q = {}, {}
    for L in range(K + 1):
        for pre in itertools.product(range(V), repeat=L):
            P[pre] = dist()
            if L < K:
                Q[pre] = dist()
    return P, Q


class Emitter:
    """Black-box view of the oracle for fixed tables: (x, u) -> emitted token tuple."""

    def __init__(self, P, Q, K, T):
        self.P, self.Q, self.K, self.T = P, Q, K, T

    def __call__(self, x, u):
        K, T = self.K, self.T
        with np.errstate(divide="ignore"):
            t_rows = np.stack([T * np.log(self.P[tuple(x[:k])]) for k in range(K + 1)])
            d_rows = np.stack([T * np.log(self.Q[tuple(x[:k])]) for k in range(K)])
        r = oracle.verify_sample_request(t_rows, d_rows, list(x), np.asarray(u, np.float64), 0, T)
        assert not r["row_error"]
        return tuple(int(v) for v in r["tokens"][:r["tau"]])


def kept_measure(emit, x, k):
    """Length of {u_k in [0,1): slot k is kept} when every earlier slot is kept (u_j = 0)."""
    K = len(x)

    def kept(uk):
        u = [0.0] * k + [uk] + [0.5] * (K - k)
        return len(emit(x, u)) > k + 1

    if not kept(0.0):
        return 0.0
    if kept(ONE_MINUS):
        return 1.0
    lo, hi = 0.0, ONE_MINUS
    while True:
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            return hi
        if kept(mid):
            lo = mid
        else:
            hi = mid


def final_draw_segments(emit, x, m):
    """Measures of the emitted token over u_K in [0,1) when slot m is the first rejection
    (m < K) or all drafts are kept (m == K)."""
    K = len(x)

    def y_at(uK):
        u = [0.0] * m + ([ONE_MINUS] if m < K else []) + [0.5] * max(0, K - m - 1) + [uK]
        out = emit(x, u)
        assert len(out) == m + 1
        return out[m]

    def seg(lo, hi, ylo, yhi):
        if ylo == yhi:
            return {ylo: hi - lo}
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            return {yhi: hi - lo}
        ym = y_at(mid)
        a, b = seg(lo, mid, ylo, ym), seg(mid, hi, ym, yhi)
        for t, w in b.items():
            a[t] = a.get(t, 0.0) + w
        return a

    return seg(0.0, 1.0, y_at(0.0), y_at(ONE_MINUS))


def emitted_distribution(emit, P, Q, V, K):
    dist = {}
    for x in itertools.product(range(V), repeat=K):
        wx = 1.0
        for k in range(K):
            wx *= Q[x[:k]][x[k]]
        if wx == 0.0:
            continue
        reach = wx
        for m in range(K + 1):
            if reach == 0.0:
                break
            if m < K:
                r = kept_measure(emit, list(x), m)
                w_m = reach * (1.0 - r)
            else:
                r, w_m = None, reach
            if w_m > 0.0:
                for y, length in final_draw_segments(emit, list(x), m).items():
                    e = tuple(x[:m]) + (y,)
                    dist[e] = dist.get(e, 0.0) + w_m * length
            if m < K:
                reach *= r
    return dist


def compare_with_autoregressive(dist, P, V, K):
    """Largest |P_spec(s) - P_AR(s)| over all length K+1 sequences s."""
    worst = 0.0
    for s in itertools.product(range(V), repeat=K + 1):
        ar = 1.0
        for i in range(K + 1):
            ar *= P[s[:i]][s[i]]
        spec = 0.0
        for L in range(1, K + 2):
            e = s[:L]
            if e in dist:
                ext = 1.0
                for i in range(L, K + 1):
                    ext *= P[s[:i]][s[i]]
                spec += dist[e] * ext
        worst = max(worst, abs(spec - ar))
    return worst


CASES = [(2, 1, 1.0, 0), (3, 1, 1.0, 1), (2, 3, 1.0, 2), (3, 2, 1.0, 3), (4, 2, 0.7, 4),
         (3, 3, 1.6, 5)]


@pytest.mark.parametrize("V,K,T,seed", CASES)
def test_emitted_tokens_follow_target_distribution(V, K, T, seed):
    rng = np.random.default_rng(1000 + seed)
    P, Q = random_tables(rng, V, K)
    dist = emitted_distribution(Emitter(P, Q, K, T), P, Q, V, K)
    assert abs(sum(dist.values()) - 1.0) < 1e-12
    assert compare_with_autoregressive(dist, P, V, K) <= 1e-12


def test_negative_control_wrong_residual_is_caught(monkeypatch):
    """A planted mistake in the oracle (resampling from p instead of the residual) must break
    the enumeration check."""
    monkeypatch.setattr(ref, "residual_weights", lambda p, q: p)
    rng = np.random.default_rng(77)
    V, K = 3, 2
    P, Q = random_tables(rng, V, K, zero_rate=0.0)
    dist = emitted_distribution(Emitter(P, Q, K, 1.0), P, Q, V, K)
    assert compare_with_autoregressive(dist, P, V, K) > 1e-3


def test_two_token_closed_form():
    """K = 1, V = 2 with p = (0.3, 0.7), q = (0.6, 0.4), worked by hand: slot 0 is kept with
    probability min(.3,.6) + min(.7,.4) = 0.7; a rejection happens only for x = 0 (mass 0.3) and
    then always places token 1 (residual (0, 0.3)); token 0 is emitted first with probability 0.3
    and token 1 with 0.7 overall."""
    P = {(): np.array([0.3, 0.7]), (0,): np.array([0.5, 0.5]), (1,): np.array([0.5, 0.5])}
    Q = {(): np.array([0.6, 0.4])}
    emit = Emitter(P, Q, 1, 1.0)
    keep = sum(Q[()][x] * kept_measure(emit, [x], 0) for x in range(2))
    assert abs(keep - 0.7) < 1e-12
    rej = {x: Q[()][x] * (1 - kept_measure(emit, [x], 0)) for x in range(2)}
    assert abs(rej[0] - 0.3) < 1e-12 and rej[1] < 1e-12
    assert final_draw_segments(emit, [0], 0) == {1: 1.0}
    dist = emitted_distribution(emit, P, Q, 2, 1)
    first = {t: sum(w for e, w in dist.items() if e[0] == t) for t in range(2)}
    assert abs(first[0] - 0.3) < 1e-12 and abs(first[1] - 0.7) < 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_acceptance_and_residual_closed_forms(seed):
    """K = 1: the chance slot 0 is kept equals sum_v min(p_v, q_v), and the chance of a rejection
    followed by token v equals max(0, p_v - q_v) (total-variation identities)."""
    rng = np.random.default_rng(500 + seed)
    V = 4
    P, Q = random_tables(rng, V, 1, zero_rate=0.15)
    p, q = P[()], Q[()]
    emit = Emitter(P, Q, 1, 1.0)
    keep, rej = 0.0, np.zeros(V)
    for x in range(V):
        if q[x] == 0:
            continue
        r = kept_measure(emit, [x], 0)
        keep += q[x] * r
        if r < 1.0:
            for y, length in final_draw_segments(emit, [x], 0).items():
                rej[y] += q[x] * (1.0 - r) * length
    assert abs(keep - np.minimum(p, q).sum()) < 1e-12
    assert np.max(np.abs(rej - np.maximum(p - q, 0.0))) < 1e-12
