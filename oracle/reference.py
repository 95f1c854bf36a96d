"""Vectorised fp64 oracle (test infrastructure only; see the package docstring).

Notation (as on the pages): K drafts x_0..x_{K-1}; the target gives K+1 next-token rows, row k
being its distribution for draft slot k and row K the extra row used when every draft is
accepted; the draft gives one row per slot. p_k = softmax(l^t_k / T), q_k = softmax(l^d_k / T).
m is the first rejected slot (0-based, so m drafts were accepted); tau = m + 1 tokens advance.

Readings where the pages leave a step open:
  * temperature: p = softmax(l / T); T = 0 is the greedy rule and has its own entry point;
  * accept slot k iff u_k < r_k with r_k = 1 when p_k(x_k) >= q_k(x_k), else p/q, so a draft the
    target likes at least as much is always kept whatever u_k in [0,1) is (evaluated from the
    log-probabilities, so it holds at any positive T);
  * the residual (or bonus) draw uses the one extra uniform u_K by inverse CDF: the smallest v
    whose running sum C_v exceeds u_K * Z; if round-off leaves none, the last v of positive
    weight; a zero-weight token is never drawn;
  * a draft token outside [0,V), or (sampling) one whose draft logit is -inf, is a row error:
    tau = -1, tokens all -1, kv unchanged, reported probabilities NaN;
  * kv_out = kv_in + tau (the round advances the committed length by tau);
  * a request is flagged as a near-tie when a decision it took has a margin below NEAR_TIE:
    |u_k - r_k| for an accept decision, the draw's threshold distance from the ends of the drawn
    token's interval of the running sum relative to the total mass for the draw.
"""
from __future__ import annotations

import numpy as np

NEAR_TIE = 1e-5  # decision margins below this are flagged near-ties


# ----------------------------------------------------------------------------------------------
# inputs
def decode_logits(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact promotion of stored logits to float64 (bf16 bit patterns or float32 values)."""
    if dtype == "bf16":
        bits = np.ascontiguousarray(stored, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------------------------
# building blocks
def softmax(logits: np.ndarray, T: float) -> np.ndarray:
    """Temperature softmax of one row: p_v = exp(l_v/T) / sum_w exp(l_w/T).

    Evaluated with the row maximum subtracted (the same quantity, without overflow). Sampling
    "at temperature" and greedy being "temperature zero" are how [SD] stage 3 and its results
    table speak of T; the ratio form l/T is the plain reading.
    """
    z = np.asarray(logits, dtype=np.float64) / np.float64(T)
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def log_softmax(logits: np.ndarray, T: float) -> np.ndarray:
    """Natural log of the temperature softmax: log p_v = l_v/T - max_w l_w/T - log sum_w
    exp(l_w/T - max l/T). The same quantity as log(softmax(l, T)), but finite wherever p_v > 0 in
    exact arithmetic: at a tiny T both p_k(x_k) and q_k(x_k) underflow to 0 in float64 while
    their ratio does not."""
    z = np.asarray(logits, dtype=np.float64) / np.float64(T)
    top = np.max(z)
    return z - top - np.log(np.sum(np.exp(z - top)))


def residual_weights(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Residual weights max(0, p - q) at the first rejected slot ([SD] stage 4: the replacement
    is drawn from a residual distribution adjusted by both models' probabilities)."""
    return np.maximum(p - q, 0.0)


def inverse_cdf(w: np.ndarray, u: float):
    """Draw a token from weights w (unnormalised) with one uniform u in [0,1).

    C is the running sum of w in token order (sequential float64), Z = C[V-1]; the token is the
    smallest v with C_v > u*Z. If round-off leaves no such v, the last v with w_v > 0.
    Returns (y, C, Z, t) with t = u*Z.
    """
    C = np.cumsum(w)
    Z = float(C[-1])
    t = float(u) * Z
    above = np.nonzero(C > t)[0]
    if above.size:
        y = int(above[0])
    else:
        y = int(np.nonzero(w > 0)[0][-1])
    return y, C, Z, t


def cdf_margin(C: np.ndarray, Z: float, t: float, y: int) -> float:
    """Distance of the draw's threshold t = u*Z from the nearer end of token y's interval
    [C_{y-1}, C_y) of the running sum, as a fraction of the total mass Z (C_{-1} = 0): the
    relative change of u that would move the draw to another token."""
    lo = float(C[y - 1]) if y > 0 else 0.0
    return min(float(C[y]) - t, t - lo) / Z


def accept_ratio(lp: float, lq: float) -> float:
    """r = min(1, p/q) from log p and log q ([SD] stage 3: a draft the target likes at least as
    much as the draft model is always kept; otherwise it is kept with probability p/q)."""
    return 1.0 if lp >= lq else float(np.exp(lp - lq))


# ----------------------------------------------------------------------------------------------
# one request
def verify_sample_request(t_rows: np.ndarray, d_rows: np.ndarray, x, u, kv_in: int, T: float):
    """Speculative-sampling verification of one request ([SD] stages 3 and 4).

    t_rows [K+1,V], d_rows [K,V] float64 logits; x [K] draft tokens; u [K+1] uniforms; T > 0.
    Returns a dict with tokens [K+1], tau, kv_out, p_x [K], q_x [K], m (first rejected slot or
    K), y, resid_mass (Z), accept_margins [K] (|u_k - r_k| for the slots decided, NaN for the
    rest), cdf_margin, margin (the smallest of them), flag_accept, flag_cdf and flagged.

    The ratio r_k = min(1, p_k(x_k)/q_k(x_k)) is taken from the float64 log-probabilities: at a
    tiny T both probabilities can underflow to 0 while their ratio is still far from 1.
    """
    K = len(x)
    V = t_rows.shape[1]
    x = [int(v) for v in x]
    u = np.asarray(u, dtype=np.float64)
    out = _empty_result(K, kv_in)

    # a draft token must be a token the draft could have sampled
    if any(v < 0 or v >= V for v in x) or any(np.isneginf(d_rows[k, x[k]]) for k in range(K)):
        out["row_error"] = True
        return out

    lP = np.array([log_softmax(t_rows[k], T)[x[k]] for k in range(K)])
    lQ = np.array([log_softmax(d_rows[k], T)[x[k]] for k in range(K)])
    out["p_x"], out["q_x"] = np.exp(lP), np.exp(lQ)

    # stage 3: left to right; p >= q always kept, otherwise kept with probability p/q
    acc = np.full(K, np.nan)
    m = K
    for k in range(K):
        r = accept_ratio(lP[k], lQ[k])
        acc[k] = abs(u[k] - r)
        if not (u[k] < r):
            m = k
            break

    # stage 4: residual at the first rejection, or the bonus row when all K drafts were kept
    w = sample_draw_weights(t_rows, d_rows, m, T)
    y, C, Z, t = inverse_cdf(w, u[K])
    tokens = np.full(K + 1, -1, np.int64)
    tokens[:m] = x[:m]
    tokens[m] = y
    out.update(tokens=tokens, tau=m + 1, kv_out=int(kv_in) + m + 1, m=m, y=y, resid_mass=Z)
    _set_margins(out, acc, cdf_margin(C, Z, t, y))
    return out


def sample_draw_weights(t_rows: np.ndarray, d_rows: np.ndarray, m: int, T: float) -> np.ndarray:
    """The weights the token placed at slot m is drawn from ([SD] stage 4): the residual
    max(0, p_m - q_m) when the draft at m was rejected (m < K), the extra target row p_K when all
    K drafts were kept (m = K); p_m if round-off leaves a residual without mass (impossible in
    exact arithmetic: a rejection means q_m(x_m) > p_m(x_m), so the residual holds at least
    q_m(x_m) - p_m(x_m))."""
    K = d_rows.shape[0]
    p = softmax(t_rows[m], T)
    w = residual_weights(p, softmax(d_rows[m], T)) if m < K else p
    return w if np.sum(w) > 0.0 else p


def _empty_result(K: int, kv_in: int) -> dict:
    """A request's outputs before anything is decided (also those of a row error)."""
    return dict(tokens=np.full(K + 1, -1, np.int64), tau=-1, kv_out=int(kv_in),
                p_x=np.full(K, np.nan), q_x=np.full(K, np.nan), m=-1, y=-1,
                resid_mass=np.nan, accept_margins=np.full(K, np.nan), cdf_margin=np.inf,
                margin=np.inf, flagged=False, flag_accept=False, flag_cdf=False,
                row_error=False)


def _set_margins(out: dict, accept_margins: np.ndarray, cdf: float) -> None:
    """Decision margins and near-tie flags of a request: accept_margins[k] = |u_k - r_k| for the
    slots actually decided (NaN for the others), cdf = the draw's normalised CDF gap. A margin
    below NEAR_TIE flags the request: its decisions then depend on rounding below the agreed
    precision, and only their validity is comparable."""
    taken = accept_margins[~np.isnan(accept_margins)]
    flag_accept = bool(taken.size and np.min(taken) < NEAR_TIE)
    flag_cdf = bool(cdf < NEAR_TIE)
    out.update(accept_margins=accept_margins, cdf_margin=float(cdf),
               margin=float(min(np.min(taken) if taken.size else np.inf, cdf)),
               flag_accept=flag_accept, flag_cdf=flag_cdf, flagged=flag_accept or flag_cdf)


def verify_greedy_request(t_rows: np.ndarray, x, kv_in: int):
    """Greedy verification of one request ([SD] stage 3 at temperature zero; [D3D] sections
    "検証のしくみ③" and "検証のまとめ"): keep drafts left to right while each equals the target's
    top choice for its slot; at the first mismatch place the target's own top choice and drop the
    rest; if all K match, the extra row's top choice is appended. Ties go to the lowest id."""
    K = len(x)
    V = t_rows.shape[1]
    x = [int(v) for v in x]
    out = dict(tokens=np.full(K + 1, -1, np.int64), tau=-1, kv_out=int(kv_in), m=-1, y=-1,
               g=None, row_error=False)
    if any(v < 0 or v >= V for v in x):
        out["row_error"] = True
        return out
    g = [int(np.argmax(t_rows[k])) for k in range(K + 1)]   # first maximum = lowest id
    m = K
    for k in range(K):
        if x[k] != g[k]:
            m = k
            break
    tokens = np.full(K + 1, -1, np.int64)
    tokens[:m] = x[:m]
    tokens[m] = g[m]
    out.update(tokens=tokens, tau=m + 1, kv_out=int(kv_in) + m + 1, m=m, y=g[m], g=g)
    return out


def temperature_is_valid(T: float) -> bool:
    """A per-request temperature the mixed rule accepts: 0 (greedy), or positive and finite with
    log2(e)/T finite once rounded to float32 (the factor the device uses)."""
    T = float(T)
    if T == 0.0:
        return True
    if not (T > 0.0 and np.isfinite(T)):
        return False
    with np.errstate(over="ignore"):
        return bool(np.isfinite(np.float32(1.4426950408889634074 / np.float64(T))))


def verify_mixed_request(t_rows: np.ndarray, d_rows: np.ndarray, x, u, kv_in: int, T: float):
    """Verification at a request's own temperature ([SD] stage 3: temperature zero keeps a draft
    while it equals the target's top choice; a positive temperature keeps it by the probability
    ratio). T = 0: the greedy rule, with p_k(x_k) reported as 1 for the target's top choice and 0
    otherwise and q_k(x_k) as 1 (the temperature-zero limits); T > 0: speculative sampling at T;
    an invalid T (temperature_is_valid) is a row error."""
    K = len(x)
    if float(T) == 0.0:
        r = verify_greedy_request(t_rows, x, kv_in)
        if r["row_error"]:
            p_x = q_x = np.full(K, np.nan)
        else:
            p_x = np.array([1.0 if int(x[k]) == r["g"][k] else 0.0 for k in range(K)])
            q_x = np.ones(K)
        out = _empty_result(K, kv_in)
        out.update(r)
        out.update(p_x=p_x, q_x=q_x)
        return out
    if not temperature_is_valid(T):
        out = _empty_result(K, kv_in)
        out["row_error"] = True
        return out
    return verify_sample_request(t_rows, d_rows, x, u, kv_in, float(T))


def predict_request(d_rows: np.ndarray, F: int, T: float):
    """Outcome keys of one request ([SSD] section "1. Outcome Prediction": the token placed at a
    rejection is predicted from the draft's top logits).

    keys[k, f] for slot k: the F token ids with the largest draft logits, ordered by logit
    descending and id ascending. key_prob[k, f] = q_k(key) at T > 0; at T = 0 the argmax key gets
    1 and the others 0.
    """
    K = d_rows.shape[0]
    keys = np.argsort(-d_rows, axis=1, kind="stable")[:, :F]
    if T > 0:
        prob = np.stack([softmax(d_rows[k], T)[keys[k]] for k in range(K)])
    else:
        prob = np.zeros((K, F))
        prob[:, 0] = 1.0
    return keys.astype(np.int64), prob


def outcome_hit(keys_row: np.ndarray, m: int, y: int, K: int, positions: int = None) -> bool:
    """Whether a verification outcome (m drafts kept, token y placed at slot m) was predicted.

    Hit iff the rejection happened at a slot that has keys (m < K, and m < `positions` when a
    position limit is given) and y is among that slot's keys ([D3D] sections "ヒット" and "ミス":
    a placed token outside the prepared candidates, or a rejection beyond the prepared slots, is a
    miss). A round with every draft kept has no key here and counts as a miss.
    """
    limit = K if positions is None else min(K, positions)
    if m < 0 or m >= limit:
        return False
    return bool(np.any(np.asarray(keys_row[m]) == y))


# ----------------------------------------------------------------------------------------------
# per-slot fan-out: prepared outcomes in the manner of D3D
def fanout_offsets(fanout) -> np.ndarray:
    """Key offsets of a per-slot fan-out: slot k's keys occupy [off[k], off[k+1])."""
    off = np.zeros(len(fanout) + 1, np.int64)
    off[1:] = np.cumsum(np.asarray(fanout, np.int64))
    return off


def predict_fanout_request(d_rows: np.ndarray, x, fanout, T: float):
    """Keys of one request under a per-slot fan-out ([D3D] section "答え:…": for each of the
    first P slots the drafter prepares candidates for the token the target would place were that
    slot the first rejection, namely its own 2nd and 3rd choices, i.e. its top choices other than
    the draft token; [SSD] section "1. Outcome Prediction": how many candidates each position
    gets is the fan-out).

    fanout[k] = F_k >= 0 for slots k < P = len(fanout). Slot k's keys are the F_k tokens with the
    largest draft logits, ordered by logit descending then id ascending, skipping the draft token
    x[k] when x is given (x = None: no exclusion). key_prob = q_k(key) at T > 0; at T = 0 it is 1
    for the row's argmax token (lowest id among equal maxima) and 0 for any other key.
    Returns keys [S] and key_prob [S], S = sum F_k, slot k at [off[k], off[k+1]).
    """
    off = fanout_offsets(fanout)
    keys = np.full(int(off[-1]), -1, np.int64)
    prob = np.zeros(int(off[-1]))
    for k, F in enumerate(fanout):
        order = np.argsort(-d_rows[k], kind="stable")
        if x is not None:
            order = order[order != int(x[k])]
        sel = order[:int(F)]
        keys[off[k]:off[k + 1]] = sel
        if T > 0:
            prob[off[k]:off[k + 1]] = softmax(d_rows[k], T)[sel]
        else:
            prob[off[k]:off[k + 1]] = (sel == int(np.argmax(d_rows[k]))).astype(np.float64)
    return keys, prob


def outcome_slot(keys_req, fanout, K: int, m: int, y: int, all_accept: bool = True) -> int:
    """The prepared continuation a verification outcome selects, or -1 for a miss ([D3D]
    sections "答え:…", "ヒット" and "ミス").

    The outcome is m drafts kept and token y placed at slot m. A rejection at a prepared slot
    (m < P) whose placed token is one of that slot's keys selects that key's continuation, index
    off[m] + (position of y among the slot's keys). Every draft kept (m = K) selects the single
    continuation prepared for that case, index S = sum F_k, when one was prepared. Anything else
    (a placed token outside the candidates, a rejection beyond the prepared slots, a row error)
    is a miss.
    """
    P = len(fanout)
    off = fanout_offsets(fanout)
    if m == K:
        return int(off[-1]) if all_accept else -1
    if m < 0 or m >= P:
        return -1
    hits = np.nonzero(np.asarray(keys_req[off[m]:off[m + 1]]) == int(y))[0]
    return int(off[m] + hits[0]) if hits.size else -1


def fanout_budget(fanout, block: int) -> int:
    """Tokens the drafter prepares per round ([D3D] sections "パック" and the table under
    "用意を増やせばいい、わけではない"): one block for every candidate, one for the all-accept
    continuation and the block being verified, (sum F_k + 2) * block."""
    return (int(np.sum(np.asarray(fanout, np.int64))) + 2) * int(block)


# ----------------------------------------------------------------------------------------------
# KV-cache rewind on a paged cache
def kv_rewind(block_tables, block_size: int, kv_alloc, kv_new):
    """Rewinds a paged KV cache after verification ([SD] section "speculative decodingとKV cache、
    プロンプトキャッシュの関係は?": both models append the drafts' keys and values to their caches;
    when the target rejects the drafts after position m, the engine truncates both caches, dropping
    the rejected entries, before the next round).

    Request b's entries [0, L) live in the blocks block_tables[b][0 .. ceil(L / block_size)).
    With L = kv_alloc[b] entries held and L' = kv_new[b] kept, the whole blocks at positions
    [ceil(L' / block_size), ceil(L / block_size)) hold nothing kept: they are released (their table
    entries become -1). Nothing is released when L' >= L. Returns (tables, freed, offsets):
    freed lists the released block ids request by request, each request's in table order;
    offsets[b] is where request b's ids start and offsets[B] is their total.
    """
    tables = np.array(block_tables, dtype=np.int64, copy=True)
    B, max_blocks = tables.shape
    freed, offsets = [], [0]
    for b in range(B):
        held = min(max_blocks, -(-int(kv_alloc[b]) // block_size))
        kept = min(max_blocks, -(-max(int(kv_new[b]), 0) // block_size))
        for j in range(kept, held):
            freed.append(int(tables[b, j]))
            tables[b, j] = -1
        offsets.append(len(freed))
    return tables, np.array(freed, dtype=np.int64), np.array(offsets, dtype=np.int64)


# ----------------------------------------------------------------------------------------------
# drafting without a draft model: n-gram / prompt lookup, and verification of its drafts
def ngram_draft_request(ctx, n_max: int, n_min: int, K: int):
    """Drafts up to K tokens for one request by prompt lookup ([SD] section "別のドラフトモデルは
    常に必要なのか?", the n-gram and prompt-search bullet: instead of a network, the engine looks
    for a span of the prompt and of the output generated so far that matches the text just
    produced, and proposes the tokens that followed that span).

    ctx holds the request's tokens so far (prompt then output), L of them. The span to match is
    the last n tokens, ctx[L-n:], tried from n = min(n_max, L-1) down to n_min (a longer match is
    more specific); an occurrence is any earlier start j <= L-n-1 with ctx[j:j+n] equal to it,
    and of those the most recent (largest j) is taken. Its continuation starts at src = j + n,
    and the draft is ctx[src : src + length] with length = min(K, L - src) (at least one token
    follows every occurrence). No occurrence for any n: length 0.
    Returns dict(tokens [K] (-1 past length), length, n (0 without a match), src (-1 without)).
    """
    c = np.asarray(ctx, dtype=np.int64)
    L = int(c.size)
    out = dict(tokens=np.full(K, -1, np.int64), length=0, n=0, src=-1)
    for n in range(min(int(n_max), L - 1), int(n_min) - 1, -1):
        # every window of n tokens that ends before the last token, compared with the suffix
        win = np.lib.stride_tricks.sliding_window_view(c[:L - 1], n)
        hits = np.nonzero(np.all(win == c[L - n:], axis=1))[0]
        if hits.size:
            src = int(hits[-1]) + n
            length = min(int(K), L - src)
            out["tokens"][:length] = c[src:src + length]
            out.update(length=length, n=n, src=src)
            return out
    return out


def verify_point_request(t_rows: np.ndarray, x, n: int, u, kv_in: int, T: float):
    """Verification of a draft that comes with no distribution, such as a prompt-lookup draft
    ([SD] stages 3 and 4, and the closing remark of the section on drafting without a draft
    model: however the candidates are proposed, the target checks them in parallel with its own
    exact distribution). The proposer puts all its mass on its token: q_k = point mass at x_k.

    t_rows [K+1,V] float64 logits; x [K] tokens of which the first n (0 <= n <= K) are drafts and
    the rest are ignored; u [K+1] uniforms; T >= 0.
      T > 0: slot k < n is kept iff u_k < min(1, p_k(x_k) / q_k(x_k)) = min(1, p_k(x_k)); at the
             first rejection m < n the token is drawn with u_K from max(0, p_m - q_m), which is
             p_m with x_m removed; with all n kept, from the target row n (the bonus row).
      T = 0: the greedy rule over the first n slots (kept while x_k is the target's top choice,
             lowest id on ties; at m the top choice of row m is placed).
    Row errors: n outside [0, K], or a draft token (k < n) outside [0, V).
    Reported per slot k < n: p_k(x_k) (at T = 0 the top-choice indicator) and q_k(x_k) = 1;
    slots k >= n report NaN, as do row errors.
    """
    K = len(x)
    V = t_rows.shape[1]
    x = [int(v) for v in x]
    u = np.asarray(u, dtype=np.float64)
    out = _empty_result(K, kv_in)
    n = int(n)
    if n < 0 or n > K or any(v < 0 or v >= V for v in x[:n]):
        out["row_error"] = True
        return out

    if float(T) == 0.0:
        g = [int(np.argmax(t_rows[k])) for k in range(n + 1)]   # first maximum = lowest id
        m = n
        for k in range(n):
            if x[k] != g[k]:
                m = k
                break
        y = g[m]
        out["p_x"][:n] = [1.0 if x[k] == g[k] else 0.0 for k in range(n)]
        out["q_x"][:n] = 1.0
        Z = np.nan
    else:
        lP = np.array([log_softmax(t_rows[k], T)[x[k]] for k in range(n)])
        out["p_x"][:n] = np.exp(lP)
        out["q_x"][:n] = 1.0
        acc = np.full(K, np.nan)
        m = n
        for k in range(n):
            r = accept_ratio(lP[k], 0.0)          # log q_k(x_k) = 0
            acc[k] = abs(u[k] - r)
            if not (u[k] < r):
                m = k
                break
        w = point_draw_weights(t_rows, x, n, m, T)
        y, C, Z, t = inverse_cdf(w, u[K])
        _set_margins(out, acc, cdf_margin(C, Z, t, y))

    tokens = np.full(K + 1, -1, np.int64)
    tokens[:m] = x[:m]
    tokens[m] = y
    out.update(tokens=tokens, tau=m + 1, kv_out=int(kv_in) + m + 1, m=m, y=y, resid_mass=Z)
    return out


def point_draw_weights(t_rows: np.ndarray, x, n: int, m: int, T: float) -> np.ndarray:
    """Weights of the token placed at slot m for a point-mass draft of n tokens: the residual
    max(0, p_m - q_m) with q_m the point mass at x_m, i.e. p_m without x_m, when m < n; the row
    p_n when all n drafts were kept; p_m if round-off leaves the residual without mass."""
    p = softmax(t_rows[m], T)
    if m >= n:
        return p
    q = np.zeros_like(p)
    q[int(x[m])] = 1.0
    w = residual_weights(p, q)
    return w if np.sum(w) > 0.0 else p


# ----------------------------------------------------------------------------------------------
# batches
def _request_slices(n: int, requests):
    return range(n) if requests is None else requests


def verify_sample(target, draft, dtype, tokens, uniforms, kv_len, T, requests=None):
    """Batch wrapper: returns arrays over the selected requests (all by default)."""
    idx = list(_request_slices(target.shape[0], requests))
    K = tokens.shape[1]
    res = [verify_sample_request(decode_logits(target[b], dtype), decode_logits(draft[b], dtype),
                                 tokens[b], np.asarray(uniforms[b], np.float64),
                                 int(kv_len[b]), float(np.float32(T)))
           for b in idx]
    return _stack(res, idx, K, sample=True)


def verify_mixed(target, draft, dtype, tokens, uniforms, kv_len, temps, requests=None):
    """Batch wrapper of verify_mixed_request; temps are the float32 values the device gets."""
    idx = list(_request_slices(target.shape[0], requests))
    K = tokens.shape[1]
    res = [verify_mixed_request(decode_logits(target[b], dtype), decode_logits(draft[b], dtype),
                                tokens[b], np.asarray(uniforms[b], np.float64), int(kv_len[b]),
                                float(np.float32(temps[b])))
           for b in idx]
    return _stack(res, idx, K, sample=True)


def verify_greedy(target, dtype, tokens, kv_len, requests=None):
    idx = list(_request_slices(target.shape[0], requests))
    K = tokens.shape[1]
    res = [verify_greedy_request(decode_logits(target[b], dtype), tokens[b], int(kv_len[b]))
           for b in idx]
    return _stack(res, idx, K, sample=False)


def predict_outcomes(draft, dtype, F, T, requests=None):
    idx = list(_request_slices(draft.shape[0], requests))
    out = [predict_request(decode_logits(draft[b], dtype), F, float(np.float32(T))) for b in idx]
    return dict(requests=np.array(idx), keys=np.stack([o[0] for o in out]),
                key_prob=np.stack([o[1] for o in out]))


def predict_fanout(draft, dtype, tokens, fanout, T, requests=None):
    """Batch wrapper of predict_fanout_request; tokens None disables the draft-token exclusion."""
    idx = list(_request_slices(draft.shape[0], requests))
    out = [predict_fanout_request(decode_logits(draft[b], dtype),
                                  None if tokens is None else tokens[b], fanout,
                                  float(np.float32(T))) for b in idx]
    return dict(requests=np.array(idx), keys=np.stack([o[0] for o in out]),
                key_prob=np.stack([o[1] for o in out]))


def ngram_draft(ctx, lens, n_max, n_min, K, requests=None):
    """Batch wrapper of ngram_draft_request over rows ctx[b, :lens[b]]; a length outside
    [0, row width] is a row error (length -1, tokens -1, n 0, src -1)."""
    ctx = np.asarray(ctx)
    idx = list(_request_slices(ctx.shape[0], requests))
    res = []
    for b in idx:
        L = int(lens[b])
        if L < 0 or L > ctx.shape[1]:
            res.append(dict(tokens=np.full(K, -1, np.int64), length=-1, n=0, src=-1))
        else:
            res.append(ngram_draft_request(ctx[b, :L], n_max, n_min, K))
    return dict(requests=np.array(idx), tokens=np.stack([r["tokens"] for r in res]),
                length=np.array([r["length"] for r in res]), n=np.array([r["n"] for r in res]),
                src=np.array([r["src"] for r in res]))


def verify_point(target, dtype, tokens, lens, uniforms, kv_len, T, requests=None):
    """Batch wrapper of verify_point_request; lens None means every request drafts K."""
    idx = list(_request_slices(target.shape[0], requests))
    K = tokens.shape[1]
    res = [verify_point_request(decode_logits(target[b], dtype), tokens[b],
                                K if lens is None else int(lens[b]),
                                np.asarray(uniforms[b], np.float64), int(kv_len[b]),
                                float(np.float32(T)))
           for b in idx]
    return _stack(res, idx, K, sample=True)


def draw_weights(target, draft, dtype, b: int, m: int, T):
    """The sampling draw's weights for request b had m drafts been kept (sample_draw_weights on
    the stored logits at the float32 temperature the device gets)."""
    return sample_draw_weights(decode_logits(target[b], dtype), decode_logits(draft[b], dtype), m,
                               float(np.float32(T)))


def point_weights(target, dtype, tokens, n: int, b: int, m: int, T):
    """point_draw_weights of request b (n drafts) had m of them been kept."""
    return point_draw_weights(decode_logits(target[b], dtype), tokens[b], n, m,
                              float(np.float32(T)))


def _stack(res, idx, K, sample):
    d = dict(requests=np.array(idx),
             tokens=np.stack([r["tokens"] for r in res]),
             tau=np.array([r["tau"] for r in res]),
             kv_out=np.array([r["kv_out"] for r in res]),
             m=np.array([r["m"] for r in res]),
             y=np.array([r["y"] for r in res]),
             row_error=np.array([r["row_error"] for r in res]))
    if sample:
        d.update(p_x=np.stack([r["p_x"] for r in res]), q_x=np.stack([r["q_x"] for r in res]),
                 margin=np.array([r["margin"] for r in res]),
                 accept_margins=np.stack([r["accept_margins"] for r in res]),
                 cdf_margin=np.array([r["cdf_margin"] for r in res]),
                 flag_accept=np.array([r["flag_accept"] for r in res]),
                 flag_cdf=np.array([r["flag_cdf"] for r in res]),
                 flagged=np.array([r["flagged"] for r in res]),
                 resid_mass=np.array([r["resid_mass"] for r in res]))
    else:
        d.update(flagged=np.zeros(len(res), bool))
    return d
