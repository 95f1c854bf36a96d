"""Pins of the oracle's near-tie margins and flags ("speculative decodingとは", stages 3 and 4:
the accept test u < min(1, p/q) and the residual or bonus draw by inverse CDF; a decision whose
margin is below 1e-5 is flagged and only its validity is compared).

Every expected margin below is worked out by hand in its comment; the flag counts on seeded
rounds are compared with the exact flag probability in closed form (tests/near_tie.py, written
without the oracle's code)."""
import math

import numpy as np
import pytest

import oracle
from synthetic import make_workload
from near_tie import decode, flag_probability

LN3 = math.log(3.0)


def request(t_rows, d_rows, x, u, T=1.0):
    return oracle.verify_sample_request(np.array(t_rows, float), np.array(d_rows, float), x,
                                        np.array(u, float), 0, T)


# p_0 = (1/4, 3/4), q_0 = (3/4, 1/4), x_0 = 0: ratio r = 1/3. Extra row p_1 = (1/2, 1/2).
# After a rejection the residual is max(0, p - q) = (0, 1/2): Z = 1/2, only token 1.
T_ROWS = [[0.0, LN3], [0.0, 0.0]]
D_ROWS = [[LN3, 0.0]]


@pytest.mark.parametrize("u0,u1,kept,acc,cdf,flag_acc,flag_cdf", [
    # kept, accept margin 1/3 - 0.333333 = 3.33e-7; bonus: t = 0.25 in [0, 0.5): 0.25
    (0.333333, 0.25, True, 1 / 3 - 0.333333, 0.25, True, False),
    # kept, margin 1/3 - 0.3 = 1/30: clear
    (0.3, 0.25, True, 1 / 30, 0.25, False, False),
    # rejected at 0.33334: margin 6.67e-6 (flagged); residual draw t = 0.25 * 1/2 in [0, 1/2):
    # normalised gap min(0.5 - 0.125, 0.125) / 0.5 = 0.25
    (0.33334, 0.25, False, 0.33334 - 1 / 3, 0.25, True, False),
    # rejected at 0.33335: margin 1.67e-5 (clear); t = (1 - 1.5e-5)/2 lies 0.75e-5 below Z = 1/2:
    # normalised 1.5e-5 (clear; un-normalised it would be 0.75e-5 and flagged)
    (0.33335, 1 - 1.5e-5, False, 0.33335 - 1 / 3, 1.5e-5, False, False),
    # same with t 0.25e-5 below Z: normalised 5e-6, flagged by the draw alone
    (0.33335, 1 - 0.5e-5, False, 0.33335 - 1 / 3, 0.5e-5, False, True),
    # bonus draw at the boundary between the two halves of p_1: t = 0.5 + 2e-6, token 1, gap 2e-6
    (0.1, 0.5 + 2e-6, True, 1 / 3 - 0.1, 2e-6, False, True),
    # just below it: token 0, gap 2e-6
    (0.1, 0.5 - 2e-6, True, 1 / 3 - 0.1, 2e-6, False, True),
])
def test_two_token_margins(u0, u1, kept, acc, cdf, flag_acc, flag_cdf):
    r = request(T_ROWS, D_ROWS, [0], [u0, u1])
    assert (r["tau"] == 2) == kept
    assert r["accept_margins"][0] == pytest.approx(acc, rel=1e-6)
    assert r["cdf_margin"] == pytest.approx(cdf, rel=1e-6)
    assert r["flag_accept"] == flag_acc and r["flag_cdf"] == flag_cdf
    assert r["flagged"] == (flag_acc or flag_cdf)
    assert r["margin"] == pytest.approx(min(acc, cdf), rel=1e-6)


# p = (0.1, 0.2, 0.3, 0.4), q = (0.4, 0.3, 0.2, 0.1), x = 0: r = 1/4; rejected at u_0 = 0.9
# (margin 0.65). Residual (0, 0, 0.1, 0.3), Z = 0.4, running sums (0, 0, 0.1, 0.4): the boundary
# between tokens 2 and 3 sits at u = 0.1/0.4 = 1/4.
P4 = np.log([0.1, 0.2, 0.3, 0.4])
Q4 = np.log([0.4, 0.3, 0.2, 0.1])


@pytest.mark.parametrize("du,y,flag", [
    (-2e-6, 2, True),      # t = 0.1 - 2e-6 * Z: gap 2e-6 of Z
    (+2e-6, 3, True),      # just above: token 3, gap 2e-6
    (-1.5e-5, 2, False),   # gap 1.5e-5 of Z (6e-6 un-normalised)
    (+3e-5, 3, False),
])
def test_residual_boundary_margin_is_normalised(du, y, flag):
    r = request([P4, P4], [Q4], [0], [0.9, 0.25 + du])
    assert r["tau"] == 1 and r["tokens"][0] == y
    assert r["resid_mass"] == pytest.approx(0.4, rel=1e-12)
    assert r["accept_margins"][0] == pytest.approx(0.65, rel=1e-9)
    assert r["cdf_margin"] == pytest.approx(abs(du), rel=1e-6)
    assert r["flagged"] == flag and r["flag_cdf"] == flag and not r["flag_accept"]


def test_only_decided_slots_have_margins():
    """K = 3, the first slot rejected (r = 1/4 at u = 0.9): slots 1 and 2 are never decided, so
    they have no margin and cannot flag the request even when their u sits on their ratio."""
    t = [P4, P4, P4, P4]
    d = [Q4, P4, P4]
    r = request(t, d, [0, 0, 0], [0.9, 1.0 - 1e-9, 1.0 - 1e-9, 0.6])
    assert r["tau"] == 1
    assert r["accept_margins"][0] == pytest.approx(0.65)
    assert np.all(np.isnan(r["accept_margins"][1:]))
    assert not r["flag_accept"]


def test_point_mass_margins():
    """Point-mass draft x_0 = 3 of p_0 = (0.1, 0.2, 0.3, 0.4): r = 0.4. u_0 = 0.399995 is kept
    with margin 5e-6 (flagged); u_0 = 0.5 is rejected with margin 0.1 and draws from p_0 without
    token 3, (0.1, 0.2, 0.3), Z = 0.6, running sums (0.1, 0.3, 0.6): u_K = 0.5 - 2e-6 puts t
    2e-6 * Z below 0.3, token 1, normalised gap 2e-6."""
    t = np.array([P4, P4])
    r = oracle.verify_point_request(t, [3], 1, np.array([0.399995, 0.3]), 0, 1.0)
    assert r["tau"] == 2 and r["flag_accept"]
    assert r["accept_margins"][0] == pytest.approx(5e-6, rel=1e-6)
    r = oracle.verify_point_request(t, [3], 1, np.array([0.5, 0.5 - 2e-6]), 0, 1.0)
    assert r["tau"] == 1 and r["tokens"][0] == 1
    assert r["resid_mass"] == pytest.approx(0.6, rel=1e-12)
    assert r["cdf_margin"] == pytest.approx(2e-6, rel=1e-6)
    assert r["flag_cdf"] and not r["flag_accept"]


def test_near_tie_threshold_value():
    assert oracle.NEAR_TIE == 1e-5


def test_closed_form_matches_hand_case():
    """The closed form on the two-token request: r = 1/3; kept and clear: 1/3 - eps; rejected
    and clear: 2/3 - eps. Bonus row (1/2, 1/2): both intervals wider than 2 eps, so the draw is
    near an end with probability 4 eps; residual (0, 1/2): one interval, 2 eps.
    P(no flag) = (1/3 - eps)(1 - 4 eps) + (2/3 - eps)(1 - 2 eps)."""
    eps = 1e-5
    t = np.array(T_ROWS)
    d = np.array(D_ROWS)
    pf, pa, pc = flag_probability(t, d, [0], 1.0, eps)
    clear = (1 / 3 - eps) * (1 - 4 * eps) + (2 / 3 - eps) * (1 - 2 * eps)
    assert pf == pytest.approx(1 - clear, rel=1e-9)
    assert pa == pytest.approx(2 * eps, rel=1e-9)
    assert pc == pytest.approx(1 / 3 * 4 * eps + 2 / 3 * 2 * eps, rel=1e-9)


def _flag_counts(t_rows, d_rows, x, T, n_draws, seed):
    rng = np.random.default_rng(seed)
    K = len(x)
    us = rng.random((n_draws, K + 1), dtype=np.float32).astype(np.float64)
    fa = fc = fl = 0
    for u in us:
        r = oracle.verify_sample_request(t_rows, d_rows, x, u, 0, T)
        fa += r["flag_accept"]
        fc += r["flag_cdf"]
        fl += r["flagged"]
    return fl, fa, fc


def _within(count, n, p, z=5.0):
    sd = math.sqrt(max(n * p * (1 - p), 1e-12))
    return abs(count - n * p) <= z * sd + 1.0


@pytest.mark.parametrize("config,rnd,T", [(1, 0, None), (1, 1, None), (1, 2, 3.0)])
def test_flag_share_matches_closed_form(config, rnd, T):
    """Seeded C1 rounds (V = 1000, fp32), also at a flatter T = 3 where many tokens have
    intervals narrower than 2e-5: the oracle's flag counts over 6000 uniform draws agree with the
    exact flag probability within 5 standard deviations, for accept flags, draw flags and flags
    overall."""
    wl = make_workload(config, rnd)
    T = float(np.float32(wl.T if T is None else T))
    t_rows, d_rows = decode(wl.target[0], wl.dtype), decode(wl.draft[0], wl.dtype)
    x = wl.tokens[0]
    n = 6000
    fl, fa, fc = _flag_counts(t_rows, d_rows, x, T, n, seed=100 + rnd)
    pf, pa, pc = flag_probability(t_rows, d_rows, x, T)
    assert _within(fl, n, pf), (fl, n * pf)
    assert _within(fa, n, pa), (fa, n * pa)
    assert _within(fc, n, pc), (fc, n * pc)


def test_flag_share_residual_heavy():
    """A request built so that rejections are likely and the residual mass small (draft close
    to the target, flat rows of 4000 tokens at T = 2, drafts where p/q is smallest): the draws
    come from residuals of mass well below 1 spread over ~2000 tokens, where an un-normalised gap
    would flag about 1/Z times as often."""
    rng = np.random.default_rng(7)
    V, K = 4000, 2
    base = rng.normal(0, 1.0, size=(K + 1, V))
    t_rows = base.copy()
    d_rows = base[:K] + rng.normal(0, 0.15, size=(K, V))
    x = [int(np.argmin(t_rows[k] - d_rows[k])) for k in range(K)]   # p/q smallest: rejected
    T = 2.0
    n = 6000
    fl, fa, fc = _flag_counts(t_rows, d_rows, x, T, n, seed=11)
    pf, pa, pc = flag_probability(t_rows, d_rows, x, T)
    assert pc > 0.02
    assert _within(fc, n, pc), (fc, n * pc)
    assert _within(fl, n, pf), (fl, n * pf)
