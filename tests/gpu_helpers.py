"""Shared helpers for the GPU parity tests: upload a seeded workload, run an entry point of the
HIP library through the binding with poisoned outputs, and compare with the fp64 oracle.

Parity rules:
  * greedy tokens/tau/kv and prediction keys: identical on every request;
  * sampling tokens/tau/kv: identical on every request the oracle does not flag as a near-tie
    (a decision margin |u - r| or CDF gap below 1e-5). On a flagged request the decisions whose
    margins are clear must still agree: the GPU may take the other branch only at a slot whose
    accept margin is below 1e-5; when it reaches the oracle's rejection slot and only the draw's
    gap is small, tau and the kept prefix are exact; the placed token must have positive weight
    in the oracle's draw weights at the GPU's slot (exactly the oracle's token when the draw's
    gap is clear). The flagged count must stay within a Poisson-sized band above its exact
    expectation over the uniforms (tests/near_tie.py);
  * probabilities p_k(x_k), q_k(x_k) and key probabilities: within 1e-5 absolute;
  * every output element is written (outputs are pre-filled with a poison pattern).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import speculative_decoding_verification_12_amd as sv
from near_tie import decode, expected_flags, flag_bound, flag_probability

POISON_WORD = 0x7B7B7B7B        # not a token id, tau, kv length or probability
PROB_ATOL = 1e-5


def announce(msg: str):
    print(f"[gpu] {msg}", flush=True)


def dev_logits(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    arr = np.ascontiguousarray(arr)
    if dtype == "bf16":
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(arr.astype(np.float32, copy=False))
    return t.to(device)


def upload(wl, device="cuda", with_draft=True):
    d = dict(target=dev_logits(wl.target, wl.dtype, device),
             tokens=torch.from_numpy(wl.tokens).to(device),
             uniforms=torch.from_numpy(wl.uniforms).to(device),
             kv=torch.from_numpy(wl.kv_len).to(device))
    if with_draft:
        d["draft"] = dev_logits(wl.draft, wl.dtype, device)
    return d


def poisoned(shape, dtype, device="cuda"):
    t = torch.full(shape, POISON_WORD, dtype=torch.int32, device=device)
    return t if dtype == torch.int32 else t.view(dtype)


def _np(t):
    return t.detach().cpu().numpy()


_EVENTS = []


def kernel_events():
    """Four HIP events (created once) to pass as `events`: a call given them has its two kernels
    timed, so it takes the two-launch path whatever the batch size."""
    if not _EVENTS:
        import ctypes
        hip = sv.hip_runtime()
        hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        arr = (ctypes.c_void_p * 4)()
        for i in range(4):
            e = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(e)) == 0
            arr[i] = e.value
        _EVENTS.append(arr)
    return _EVENTS[0]


def gpu_sample(wl, dev=None, ws=None, wait_polls=None, two_launch=False):
    dev = dev or upload(wl)
    B, K = wl.B, wl.K
    ws = ws if ws is not None else sv.new_workspace(B, K, wl.V)
    out = dict(tokens=poisoned((B, K + 1), torch.int32), tau=poisoned((B,), torch.int32),
               kv_len=poisoned((B,), torch.int32), p=poisoned((B, K), torch.float32),
               q=poisoned((B, K), torch.float32))
    sv.spec_verify_sample(dev["target"], dev["draft"], dev["tokens"], dev["uniforms"], dev["kv"],
                          float(wl.T), ws, out=out, wait_polls=wait_polls,
                          events=kernel_events() if two_launch else None)
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in out.items()}


def gpu_greedy(wl, dev=None, ws=None, wait_polls=None):
    dev = dev or upload(wl, with_draft=False)
    B, K = wl.B, wl.K
    ws = ws if ws is not None else sv.new_workspace(B, K, wl.V)
    out = dict(tokens=poisoned((B, K + 1), torch.int32), tau=poisoned((B,), torch.int32),
               kv_len=poisoned((B,), torch.int32))
    sv.spec_verify_greedy(dev["target"], dev["tokens"], dev["kv"], ws, out=out,
                          wait_polls=wait_polls)
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in out.items()}


def gpu_predict(wl, F, T, dev=None, ws=None):
    draft = dev["draft"] if dev else dev_logits(wl.draft, wl.dtype)
    B, K = wl.B, wl.K
    ws = ws if ws is not None else sv.new_workspace(B, K, wl.V, F)
    out = dict(keys=poisoned((B, K, F), torch.int32), key_prob=poisoned((B, K, F), torch.float32))
    sv.spec_predict_outcomes(draft, F, T, ws, out=out)
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in out.items()}


def _assert_no_poison(out):
    for k, v in out.items():
        bits = np.ascontiguousarray(v).view(np.int32)
        assert not np.any(bits == POISON_WORD), f"{k}: unwritten output elements"


def check_row(where, tok, tau, kv, ref, i, x, kv_in, nb, V, weights_at):
    """One request's tokens, tau and kv against the oracle's row i by the parity rules (module
    docstring). x: its drafts, nb: how many of them (K, or a point-mass draft's length),
    weights_at(m): the oracle's draw weights had m drafts been kept. Returns whether the outputs
    differ from the oracle's (possible only on a flagged request)."""
    m_ref, y_ref = int(ref["m"][i]), int(ref["y"][i])
    acc = ref["accept_margins"][i]
    m = tau - 1
    assert 1 <= tau <= nb + 1, f"{where}: tau {tau} outside [1, {nb + 1}]"
    assert kv == kv_in + tau, f"{where}: kv {kv} != {kv_in} + {tau}"
    assert np.array_equal(tok[:m], x[:m]), f"{where}: kept prefix {tok[:m]} != drafts {x[:m]}"
    assert np.all(tok[tau:] == -1), f"{where}: padding {tok[tau:]}"
    y = int(tok[m])
    assert 0 <= y < V, f"{where}: token {y}"
    if m > m_ref:    # the GPU kept the slot the oracle rejected: only on a near-tie there
        assert acc[m_ref] < oracle.NEAR_TIE, \
            f"{where}: tau {tau} != {m_ref + 1} (slot {m_ref} margin {acc[m_ref]:.3g})"
    elif m < m_ref:  # the GPU rejected a slot the oracle kept
        assert acc[m] < oracle.NEAR_TIE, \
            f"{where}: tau {tau} != {m_ref + 1} (slot {m} margin {acc[m]:.3g})"
    if m == m_ref and not ref["flag_cdf"][i]:
        assert y == y_ref, f"{where}: token {y} != {y_ref} (gap {ref['cdf_margin'][i]:.3g})"
    else:
        w = weights_at(m)
        assert w[y] > 0.0, f"{where}: token {y} has no weight at slot {m}"
    return m != m_ref or y != y_ref


def _check_flag_count(where, n_flag, expected):
    bound = flag_bound(expected)
    assert n_flag <= bound, (f"{where}: {n_flag} flagged near-ties, more than the bound {bound} "
                             f"(expected {expected:.2f})")


def compare_sample(wl, gpu, requests=None):
    """Asserts the sampling parity rules; returns (n_checked, n_flagged, n_flagged_differing)."""
    _assert_no_poison(gpu)
    idx = list(range(wl.B)) if requests is None else list(requests)
    ref = oracle.verify_sample(wl.target, wl.draft, wl.dtype, wl.tokens, wl.uniforms, wl.kv_len,
                               wl.T, requests=idx)
    K, V = wl.K, wl.V
    n_flag = n_flag_mismatch = 0
    for i, b in enumerate(idx):
        tok, tau, kv = gpu["tokens"][b], int(gpu["tau"][b]), int(gpu["kv_len"][b])
        rt, rtau, rkv = ref["tokens"][i], int(ref["tau"][i]), int(ref["kv_out"][i])
        where = f"request {b} (round {wl.round}, {wl.config.name}, B={wl.B} K={K} V={V})"
        if ref["row_error"][i]:
            assert tau == -1 and kv == rkv and np.all(tok == -1), where
            assert np.all(np.isnan(gpu["p"][b])) and np.all(np.isnan(gpu["q"][b])), where
            continue
        np.testing.assert_allclose(gpu["p"][b], ref["p_x"][i], rtol=0, atol=PROB_ATOL,
                                   err_msg=where)
        np.testing.assert_allclose(gpu["q"][b], ref["q_x"][i], rtol=0, atol=PROB_ATOL,
                                   err_msg=where)
        differs = check_row(where, tok, tau, kv, ref, i, wl.tokens[b], int(wl.kv_len[b]), K, V,
                            lambda m, b=b: oracle.draw_weights(wl.target, wl.draft, wl.dtype, b,
                                                               m, wl.T))
        if ref["flagged"][i]:
            n_flag += 1
            n_flag_mismatch += int(differs)
        else:
            assert not differs and np.array_equal(tok, rt) and tau == rtau and kv == rkv, where
    _check_flag_count(f"{wl.config.name} round {wl.round}", n_flag,
                      expected_flags(wl, idx) if n_flag else 0.0)
    return len(idx), n_flag, n_flag_mismatch


def compare_greedy(wl, gpu, requests=None):
    _assert_no_poison(gpu)
    idx = list(range(wl.B)) if requests is None else list(requests)
    ref = oracle.verify_greedy(wl.target, wl.dtype, wl.tokens, wl.kv_len, requests=idx)
    for i, b in enumerate(idx):
        where = f"request {b} (round {wl.round}, {wl.config.name}, greedy)"
        assert np.array_equal(gpu["tokens"][b], ref["tokens"][i]), where
        assert int(gpu["tau"][b]) == int(ref["tau"][i]), where
        assert int(gpu["kv_len"][b]) == int(ref["kv_out"][i]), where
    return ref


def compare_predict(wl, gpu, F, T, requests=None):
    _assert_no_poison(gpu)
    idx = list(range(wl.B)) if requests is None else list(requests)
    ref = oracle.predict_outcomes(wl.draft, wl.dtype, F, T, requests=idx)
    for i, b in enumerate(idx):
        where = f"request {b} (round {wl.round}, {wl.config.name}, predict F={F} T={T})"
        assert np.array_equal(gpu["keys"][b], ref["keys"][i]), where
        np.testing.assert_allclose(gpu["key_prob"][b], ref["key_prob"][i], rtol=0,
                                   atol=PROB_ATOL, err_msg=where)
    return ref


def gpu_fanout(wl, fanout, T, exclude, dev=None, ws=None):
    """Per-slot fan-out keys; exclusion skips wl.tokens (the draft tokens)."""
    draft = dev["draft"] if dev else dev_logits(wl.draft, wl.dtype)
    B, K = wl.B, wl.K
    S = int(sum(fanout))
    ws = ws if ws is not None else sv.new_workspace(B, K, wl.V)
    x = (dev["tokens"] if dev else torch.from_numpy(wl.tokens).cuda()) if exclude else None
    out = dict(keys=poisoned((B, S), torch.int32), key_prob=poisoned((B, S), torch.float32))
    sv.spec_predict_fanout(draft, fanout, T, ws, draft_tokens=x, out=out)
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in out.items()}


def compare_fanout(wl, gpu, fanout, T, exclude, requests=None):
    _assert_no_poison(gpu)
    idx = list(range(wl.B)) if requests is None else list(requests)
    ref = oracle.predict_fanout(wl.draft, wl.dtype, wl.tokens if exclude else None, fanout, T,
                                requests=idx)
    for i, b in enumerate(idx):
        where = (f"request {b} ({wl.config.name}, fan-out {list(fanout)} T={T} "
                 f"exclude={exclude})")
        assert np.array_equal(gpu["keys"][b], ref["keys"][i]), where
        np.testing.assert_allclose(gpu["key_prob"][b], ref["key_prob"][i], rtol=0,
                                   atol=PROB_ATOL, err_msg=where)
    return ref


def oracle_outcomes(wl):
    """(tau, tokens) of every request from the oracle, the input of the lookup parity check."""
    if float(wl.T) > 0:
        r = oracle.verify_sample(wl.target, wl.draft, wl.dtype, wl.tokens, wl.uniforms,
                                 wl.kv_len, wl.T)
    else:
        r = oracle.verify_greedy(wl.target, wl.dtype, wl.tokens, wl.kv_len)
    return r["tau"].astype(np.int32), r["tokens"].astype(np.int32)


def compare_lookup(wl, keys, fanout, all_accept=True):
    """GPU lookup on the oracle's outcomes and the oracle's keys against oracle.outcome_slot.
    Returns the per-request slots."""
    tau, tokens = oracle_outcomes(wl)
    out = poisoned((wl.B,), torch.int32)
    sv.spec_outcome_lookup(torch.from_numpy(tau).cuda(), torch.from_numpy(tokens).cuda(),
                           torch.from_numpy(np.ascontiguousarray(keys, np.int32)).cuda(), fanout,
                           all_accept, out=out)
    torch.cuda.synchronize()
    got = _np(out)
    for b in range(wl.B):
        exp = oracle.outcome_slot(keys[b], fanout, wl.K, int(tau[b]) - 1,
                                  int(tokens[b, max(int(tau[b]) - 1, 0)]), all_accept)
        assert int(got[b]) == exp, f"request {b}: lookup {got[b]} != {exp}"
    return got


def gpu_sample_keys(wl, F, exclude, dev=None, ws=None):
    dev = dev or upload(wl)
    B, K = wl.B, wl.K
    ws = ws if ws is not None else sv.new_workspace(B, K, wl.V)
    out = dict(tokens=poisoned((B, K + 1), torch.int32), tau=poisoned((B,), torch.int32),
               kv_len=poisoned((B,), torch.int32), p=poisoned((B, K), torch.float32),
               q=poisoned((B, K), torch.float32), keys=poisoned((B, K, F), torch.int32),
               key_prob=poisoned((B, K, F), torch.float32))
    sv.spec_verify_sample_keys(dev["target"], dev["draft"], dev["tokens"], dev["uniforms"],
                               dev["kv"], float(wl.T), F, ws, exclude_draft=exclude, out=out)
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in out.items()}


def compare_sample_keys(wl, gpu, F, exclude, requests=None):
    """Verification parity as compare_sample; keys and key probabilities as the per-slot fan-out
    oracle with F keys on every slot."""
    verify = {k: gpu[k] for k in ("tokens", "tau", "kv_len", "p", "q")}
    res = compare_sample(wl, verify, requests)
    keys = dict(keys=gpu["keys"].reshape(wl.B, -1), key_prob=gpu["key_prob"].reshape(wl.B, -1))
    compare_fanout(wl, keys, [F] * wl.K, float(wl.T), exclude, requests)
    return res


def gpu_mixed(wl, temps, dev=None, ws=None):
    dev = dev or upload(wl)
    B, K = wl.B, wl.K
    ws = ws if ws is not None else sv.new_workspace(B, K, wl.V)
    out = dict(tokens=poisoned((B, K + 1), torch.int32), tau=poisoned((B,), torch.int32),
               kv_len=poisoned((B,), torch.int32), p=poisoned((B, K), torch.float32),
               q=poisoned((B, K), torch.float32))
    sv.spec_verify_mixed(dev["target"], dev["draft"], dev["tokens"], dev["uniforms"], dev["kv"],
                         torch.from_numpy(np.asarray(temps, np.float32)).cuda(), ws, out=out)
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in out.items()}


def compare_mixed(wl, gpu, temps, requests=None):
    """Mixed-batch parity: greedy requests bit-exact with probabilities as the oracle reports
    them; sampling requests by the sampling rules at their own temperature; invalid temperatures
    as row errors. Returns (n_checked, n_flagged)."""
    _assert_no_poison(gpu)
    idx = list(range(wl.B)) if requests is None else list(requests)
    ref = oracle.verify_mixed(wl.target, wl.draft, wl.dtype, wl.tokens, wl.uniforms, wl.kv_len,
                              temps, requests=idx)
    K, V = wl.K, wl.V
    n_flag = 0
    expected = 0.0
    for i, b in enumerate(idx):
        tok, tau, kv = gpu["tokens"][b], int(gpu["tau"][b]), int(gpu["kv_len"][b])
        Tb = float(np.float32(temps[b]))
        where = f"request {b} (T={temps[b]}, {wl.config.name}, K={K} V={V})"
        if ref["row_error"][i]:
            assert tau == -1 and kv == int(ref["kv_out"][i]) and np.all(tok == -1), where
            assert np.all(np.isnan(gpu["p"][b])) and np.all(np.isnan(gpu["q"][b])), where
            continue
        np.testing.assert_allclose(gpu["p"][b], ref["p_x"][i], rtol=0, atol=PROB_ATOL,
                                   err_msg=where)
        np.testing.assert_allclose(gpu["q"][b], ref["q_x"][i], rtol=0, atol=PROB_ATOL,
                                   err_msg=where)
        if Tb == 0.0:
            assert tau == int(ref["tau"][i]) and np.array_equal(tok, ref["tokens"][i]), where
            assert kv == int(ref["kv_out"][i]), where
            continue
        check_row(where, tok, tau, kv, ref, i, wl.tokens[b], int(wl.kv_len[b]), K, V,
                  lambda m, b=b, Tb=Tb: oracle.draw_weights(wl.target, wl.draft, wl.dtype, b, m,
                                                            Tb))
        if ref["flagged"][i]:
            n_flag += 1
        else:
            assert tau == int(ref["tau"][i]) and np.array_equal(tok, ref["tokens"][i]), where
    if n_flag:   # the expectation over every sampling request, not only the flagged ones
        expected = sum(flag_probability(decode(wl.target[b], wl.dtype),
                                        decode(wl.draft[b], wl.dtype), wl.tokens[b],
                                        float(np.float32(temps[b])))[0]
                       for i, b in enumerate(idx)
                       if not ref["row_error"][i] and float(np.float32(temps[b])) > 0.0)
    _check_flag_count(f"{wl.config.name} mixed", n_flag, expected)
    return len(idx), n_flag


def gpu_ngram(ctx, lens, n_max, n_min, K):
    c = torch.from_numpy(np.ascontiguousarray(ctx, np.int32)).cuda()
    n = torch.from_numpy(np.ascontiguousarray(lens, np.int32)).cuda()
    B = c.shape[0]
    out = dict(tokens=poisoned((B, K), torch.int32), len=poisoned((B,), torch.int32),
               ngram=poisoned((B,), torch.int32), src=poisoned((B,), torch.int32))
    sv.spec_ngram_draft(c, n, n_max, n_min, K, out=out)
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in out.items()}


def compare_ngram(ctx, lens, n_max, n_min, K, gpu, where=""):
    """Prompt-lookup drafts: every output identical to the oracle's (integer work)."""
    _assert_no_poison(gpu)
    ref = oracle.ngram_draft(ctx, lens, n_max, n_min, K)
    for key, rk in (("len", "length"), ("ngram", "n"), ("src", "src")):
        bad = np.nonzero(gpu[key] != ref[rk])[0]
        assert bad.size == 0, f"{key} differs at requests {bad[:8]} {where}"
    bad = np.nonzero(np.any(gpu["tokens"] != ref["tokens"], axis=1))[0]
    assert bad.size == 0, f"tokens differ at requests {bad[:8]} {where}"
    return ref


def gpu_point(wl, tokens, lens, T, dev=None, ws=None):
    dev = dev or upload(wl, with_draft=False)
    B, K = wl.B, wl.K
    ws = ws if ws is not None else sv.new_workspace(B, K, wl.V)
    out = dict(tokens=poisoned((B, K + 1), torch.int32), tau=poisoned((B,), torch.int32),
               kv_len=poisoned((B,), torch.int32), p=poisoned((B, K), torch.float32),
               q=poisoned((B, K), torch.float32))
    x = torch.from_numpy(np.ascontiguousarray(tokens, np.int32)).cuda()
    n = None if lens is None else torch.from_numpy(np.ascontiguousarray(lens, np.int32)).cuda()
    sv.spec_verify_point(dev["target"], x, n, dev["uniforms"], dev["kv"], T, ws, out=out)
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in out.items()}


def compare_point(wl, gpu, tokens, lens, T, requests=None):
    """Point-mass draft verification: the sampling rules (T > 0) or greedy rules (T = 0) over the
    first n_b slots; NaN probabilities past n_b; row errors as in the other entry points.
    Returns (n_checked, n_flagged)."""
    _assert_no_poison(gpu)
    idx = list(range(wl.B)) if requests is None else list(requests)
    ref = oracle.verify_point(wl.target, wl.dtype, tokens, lens, wl.uniforms, wl.kv_len, T,
                              requests=idx)
    K, V = wl.K, wl.V
    n_flag = 0
    for i, b in enumerate(idx):
        tok, tau, kv = gpu["tokens"][b], int(gpu["tau"][b]), int(gpu["kv_len"][b])
        nb = K if lens is None else int(lens[b])
        where = f"request {b} (n={nb}, T={T}, {wl.config.name}, K={K} V={V})"
        if ref["row_error"][i]:
            assert tau == -1 and kv == int(ref["kv_out"][i]) and np.all(tok == -1), where
            assert np.all(np.isnan(gpu["p"][b])) and np.all(np.isnan(gpu["q"][b])), where
            continue
        np.testing.assert_allclose(gpu["p"][b], ref["p_x"][i], rtol=0, atol=PROB_ATOL,
                                   err_msg=where)
        np.testing.assert_array_equal(gpu["q"][b], ref["q_x"][i], err_msg=where)
        if float(T) == 0.0:
            assert tau == int(ref["tau"][i]) and np.array_equal(tok, ref["tokens"][i]), where
            assert kv == int(ref["kv_out"][i]), where
            continue
        check_row(where, tok, tau, kv, ref, i, tokens[b], int(wl.kv_len[b]), nb, V,
                  lambda m, b=b, nb=nb: oracle.point_weights(wl.target, wl.dtype, tokens, nb, b,
                                                             m, T))
        if ref["flagged"][i]:
            n_flag += 1
        else:
            assert tau == int(ref["tau"][i]) and np.array_equal(tok, ref["tokens"][i]), where
    if n_flag:
        _check_flag_count(f"{wl.config.name} point T={T}", n_flag,
                          expected_flags(wl, idx, T=T, point_tokens=np.asarray(tokens),
                                         point_lens=lens))
    return len(idx), n_flag
