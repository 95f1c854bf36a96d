"""Exact probability that a request's decisions are flagged as near-ties, over uniform draws.

Independent of the oracle's code (SciPy's softmax and log-softmax, its own logit decoding): the
tests compare the oracle's flag counts on seeded uniforms with these closed forms, and the GPU
tests bound the flagged share of a batch with them.

A request's accept decision at slot k is a near-tie when |u_k - r_k| < eps, r_k = min(1, p/q);
its draw is one when u*Z lies within eps*Z of either end of the drawn token's interval of the
running sum ("speculative decodingとは", stages 3 and 4, with the agreed 1e-5 margin). With u
uniform on [0,1):
  * slot k kept and clear:    length of [0, r) outside (r - eps, r + eps)  = max(0, r - eps)
  * slot k rejected and clear: length of [r, 1) outside (r - eps, r + eps) = max(0, 1 - r - eps)
  * draw clear given m:        1 - sum_y min(w_y / Z, 2 eps) over the tokens of positive weight
    (an interval narrower than 2 eps*Z is near an end everywhere; a wider one over 2 eps*Z).
"""
from __future__ import annotations

import numpy as np
from scipy.special import log_softmax, softmax

EPS = 1e-5


def decode(stored: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (np.asarray(stored, np.uint16).astype(np.uint32) << 16).view(np.float32) \
            .astype(np.float64)
    return np.asarray(stored, np.float32).astype(np.float64)


def _cdf_near(w: np.ndarray, eps: float) -> float:
    Z = w.sum()
    a = w[w > 0] / Z
    return float(np.minimum(a, 2 * eps).sum())


def flag_probability(t_rows, d_rows, x, T, eps=EPS, point_n=None):
    """(P(flagged), P(an accept decision flagged), P(the draw flagged)) for one request.

    t_rows [K+1,V], d_rows [K,V] float64 logits, x [K] drafts, T > 0. With point_n = n the draft
    is a point mass at x over its first n slots (d_rows unused)."""
    K = len(x)
    n = K if point_n is None else int(point_n)
    z_t = np.asarray(t_rows, np.float64) / T
    r, w = [], []
    for k in range(n + 1):
        p = softmax(z_t[k])
        if k < n:
            lp = log_softmax(z_t[k])[x[k]]
            if point_n is None:
                zd = np.asarray(d_rows[k], np.float64) / T
                q = softmax(zd)
                lq = log_softmax(zd)[x[k]]
            else:
                q = np.zeros_like(p)
                q[x[k]] = 1.0
                lq = 0.0
            r.append(1.0 if lp >= lq else float(np.exp(lp - lq)))
            wk = np.maximum(p - q, 0.0)
            w.append(wk if wk.sum() > 0 else p)
        else:
            w.append(p)
    c = [_cdf_near(wm, eps) for wm in w]
    clear = 0.0        # no flag at all
    acc_clear = 0.0    # no accept flag
    cdf_flag = 0.0
    reach_clear, reach = 1.0, 1.0
    for m in range(n + 1):
        stop_clear = max(0.0, 1.0 - r[m] - eps) if m < n else 1.0
        stop = (1.0 - r[m]) if m < n else 1.0
        acc_clear += reach_clear * stop_clear
        clear += reach_clear * stop_clear * (1.0 - c[m])
        cdf_flag += reach * stop * c[m]
        if m < n:
            reach_clear *= max(0.0, r[m] - eps)
            reach *= r[m]
    return 1.0 - clear, 1.0 - acc_clear, cdf_flag


def expected_flags(wl, requests=None, T=None, point_tokens=None, point_lens=None, eps=EPS):
    """Expected number of flagged requests of a workload over its uniforms (the workload's own
    logits and drafts; point_tokens/point_lens for point-mass drafts)."""
    T = float(np.float32(wl.T if T is None else T))
    idx = range(wl.B) if requests is None else requests
    total = 0.0
    for b in idx:
        t_rows = decode(wl.target[b], wl.dtype)
        if point_tokens is None:
            pr = flag_probability(t_rows, decode(wl.draft[b], wl.dtype), wl.tokens[b], T, eps)
        else:
            n = wl.K if point_lens is None else int(point_lens[b])
            if n < 0 or n > wl.K or np.any(point_tokens[b][:n] < 0) or \
                    np.any(point_tokens[b][:n] >= wl.V):
                continue
            pr = flag_probability(t_rows, None, point_tokens[b], T, eps, point_n=n)
        total += pr[0]
    return total


def flag_bound(expected: float) -> int:
    """Largest flagged count accepted for an expectation E: E + 5 sqrt(E) + 3 (a Poisson-sized
    band; far above any count a correct flag gives, far below a flag that marks everything)."""
    return int(np.floor(expected + 5.0 * np.sqrt(expected) + 3.0))
