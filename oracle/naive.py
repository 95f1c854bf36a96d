"""Literal pure-Python statement of the verification rules (test infrastructure only).

Written independently of `reference` (no NumPy arithmetic, no shared helpers) so that the two
can be compared on tiny inputs: per-token loops, math.exp, running sums in token order, and
linear scans. Same rules and readings as `reference`; see the package docstring for sources.
"""
from __future__ import annotations

import math


def _as_float_rows(rows):
    return [[float(v) for v in row] for row in rows]


def naive_softmax(row, T):
    zs = [v / T for v in row]
    top = max(zs)
    es = [math.exp(z - top) for z in zs]
    total = 0.0
    for e in es:
        total += e
    return [e / total for e in es]


def naive_verify_sample(t_rows, d_rows, x, u, kv_in, T):
    """Returns (tokens, tau, kv_out, p_x, q_x)."""
    t_rows, d_rows = _as_float_rows(t_rows), _as_float_rows(d_rows)
    K = len(x)
    V = len(t_rows[0])
    x = [int(v) for v in x]
    u = [float(v) for v in u]
    T = float(T)
    for k in range(K):
        if x[k] < 0 or x[k] >= V or d_rows[k][x[k]] == -math.inf:
            return [-1] * (K + 1), -1, int(kv_in), [math.nan] * K, [math.nan] * K

    p_x, q_x = [], []
    for k in range(K):
        p_x.append(naive_softmax(t_rows[k], T)[x[k]])
        q_x.append(naive_softmax(d_rows[k], T)[x[k]])

    m = K
    for k in range(K):
        if p_x[k] >= q_x[k]:
            keep = True                         # the target likes it at least as much
        else:
            keep = u[k] < p_x[k] / q_x[k]
        if not keep:
            m = k
            break

    p = naive_softmax(t_rows[m], T)
    if m < K:
        q = naive_softmax(d_rows[m], T)
        w = [max(0.0, p[v] - q[v]) for v in range(V)]
    else:
        w = list(p)
    z = 0.0
    for v in range(V):
        z += w[v]
    if not z > 0.0:
        w = list(p)
        z = 0.0
        for v in range(V):
            z += w[v]
    threshold = u[K] * z
    y = None
    running = 0.0
    for v in range(V):
        running += w[v]
        if running > threshold:
            y = v
            break
    if y is None:
        y = max(v for v in range(V) if w[v] > 0.0)

    tokens = x[:m] + [y] + [-1] * (K - m)
    return tokens, m + 1, int(kv_in) + m + 1, p_x, q_x


def naive_verify_greedy(t_rows, x, kv_in):
    t_rows = _as_float_rows(t_rows)
    K = len(x)
    V = len(t_rows[0])
    x = [int(v) for v in x]
    if any(v < 0 or v >= V for v in x):
        return [-1] * (K + 1), -1, int(kv_in)
    g = []
    for row in t_rows:
        best = 0
        for v in range(1, V):
            if row[v] > row[best]:
                best = v
        g.append(best)
    m = K
    for k in range(K):
        if x[k] != g[k]:
            m = k
            break
    tokens = x[:m] + [g[m]] + [-1] * (K - m)
    return tokens, m + 1, int(kv_in) + m + 1


def naive_predict(d_rows, F, T):
    """Top-F by repeated selection: largest logit first, lowest id among equal logits."""
    d_rows = _as_float_rows(d_rows)
    keys, probs = [], []
    for row in d_rows:
        chosen = []
        for _ in range(F):
            best = None
            for v in range(len(row)):
                if v in chosen:
                    continue
                if best is None or row[v] > row[best]:
                    best = v
            chosen.append(best)
        keys.append(chosen)
        if T > 0:
            p = naive_softmax(row, float(T))
            probs.append([p[v] for v in chosen])
        else:
            probs.append([1.0] + [0.0] * (F - 1))
    return keys, probs


def naive_predict_fanout(d_rows, x, fanout, T):
    """Per-slot fan-out by repeated selection, skipping the draft token when x is given."""
    d_rows = _as_float_rows(d_rows)
    keys, probs = [], []
    for k, F in enumerate(fanout):
        row = d_rows[k]
        chosen = []
        for _ in range(F):
            best = None
            for v in range(len(row)):
                if v in chosen or (x is not None and v == int(x[k])):
                    continue
                if best is None or row[v] > row[best]:
                    best = v
            chosen.append(best)
        keys.extend(chosen)
        if T > 0:
            p = naive_softmax(row, float(T))
            probs.extend(p[v] for v in chosen)
        else:
            top = 0
            for v in range(1, len(row)):
                if row[v] > row[top]:
                    top = v
            probs.extend(1.0 if v == top else 0.0 for v in chosen)
    return keys, probs


def naive_outcome_slot(keys, fanout, K, m, y, all_accept=True):
    start = 0
    for k, F in enumerate(fanout):
        if k == m:
            for j in range(F):
                if keys[start + j] == y:
                    return start + j
            return -1
        start += F
    if m == K and all_accept:
        return start
    return -1


def naive_kv_rewind(block_tables, block_size, kv_alloc, kv_new):
    """Block by block: a block is released when it held an entry before (its first position is
    below kv_alloc) and holds no kept entry now (its first position is at or past kv_new)."""
    tables = [list(row) for row in block_tables]
    freed, offsets = [], [0]
    for b, row in enumerate(tables):
        for j in range(len(row)):
            first = j * block_size
            if first < kv_alloc[b] and first >= max(kv_new[b], 0):
                freed.append(row[j])
                row[j] = -1
        offsets.append(len(freed))
    return tables, freed, offsets


def naive_ngram_draft(ctx, n_max, n_min, K):
    """Prompt lookup by explicit loops: for n from the longest allowed down, scan earlier starts
    j from the latest back and compare token by token. Returns (tokens, length, n, src)."""
    ctx = [int(t) for t in ctx]
    L = len(ctx)
    n = min(int(n_max), L - 1)
    while n >= int(n_min) and n >= 1:
        j = L - n - 1
        while j >= 0:
            same = True
            for i in range(n):
                if ctx[j + i] != ctx[L - n + i]:
                    same = False
                    break
            if same:
                src = j + n
                length = min(int(K), L - src)
                toks = [ctx[src + i] if i < length else -1 for i in range(int(K))]
                return toks, length, n, src
            j -= 1
        n -= 1
    return [-1] * int(K), 0, 0, -1
