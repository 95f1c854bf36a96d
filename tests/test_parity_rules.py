"""The GPU parity checker itself, on the CPU: the oracle's own outputs pass it, outputs with a
planted mistake fail it, and outputs that take the other branch of a flagged near-tie pass it
only when what they emit is valid. (Mistakes are planted in copies of the oracle's outputs; no
device is involved.)"""
import math
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
from gpu_helpers import compare_mixed, compare_point, compare_sample
from synthetic import make_workload

LN3 = math.log(3.0)


def as_gpu(ref, K):
    """The oracle's batch outputs in the shape the device returns them."""
    return dict(tokens=ref["tokens"].astype(np.int32), tau=ref["tau"].astype(np.int32),
                kv_len=ref["kv_out"].astype(np.int32), p=ref["p_x"].astype(np.float32),
                q=ref["q_x"].astype(np.float32))


def oracle_run(wl):
    return oracle.verify_sample(wl.target, wl.draft, wl.dtype, wl.tokens, wl.uniforms, wl.kv_len,
                                wl.T)


def small_c3():
    return make_workload(3, 0, B=24, V=3001)


def test_oracle_outputs_pass():
    wl = small_c3()
    n, f, fb = compare_sample(wl, as_gpu(oracle_run(wl), wl.K))
    assert n == wl.B and fb == 0


@pytest.mark.parametrize("plant", ["token", "tau", "kv", "prefix", "padding", "p"])
def test_planted_mistakes_fail(plant):
    wl = small_c3()
    ref = oracle_run(wl)
    g = as_gpu(ref, wl.K)
    b = int(np.nonzero(~ref["flagged"] & ~ref["row_error"] & (ref["tau"] >= 2))[0][0])
    m = int(ref["m"][b])
    if plant == "token":
        g["tokens"][b, m] = (g["tokens"][b, m] + 1) % wl.V
    elif plant == "tau":
        g["tau"][b] += 1
        g["kv_len"][b] += 1
    elif plant == "kv":
        g["kv_len"][b] += 1
    elif plant == "prefix":
        g["tokens"][b, 0] = (g["tokens"][b, 0] + 1) % wl.V
    elif plant == "padding":
        g["tokens"][b, wl.K] = 0 if m < wl.K else g["tokens"][b, wl.K]
        if m == wl.K:
            pytest.skip("request keeps every draft: no padding")
    elif plant == "p":
        g["p"][b, 0] += 2e-5
    with pytest.raises(AssertionError):
        compare_sample(wl, g)


def near_tie_request(u0, u1):
    """One request, K = 1, V = 2: p_0 = (1/4, 3/4), q_0 = (3/4, 1/4), x_0 = 0 (ratio 1/3); extra
    row p_1 = (1/2, 1/2). After a rejection only token 1 has weight."""
    target = np.array([[[0.0, LN3], [0.0, 0.0]]], np.float32)
    draft = np.array([[[LN3, 0.0]]], np.float32)
    return SimpleNamespace(target=target, draft=draft, dtype="f32",
                           tokens=np.array([[0]], np.int32),
                           uniforms=np.array([[u0, u1]], np.float32),
                           kv_len=np.array([100], np.int32), T=np.float32(1.0), B=1, K=1, V=2,
                           round=0, config=SimpleNamespace(name="hand"))


def outputs(tokens, tau, kv, p=0.25, q=0.75):
    return dict(tokens=np.array([tokens], np.int32), tau=np.array([tau], np.int32),
                kv_len=np.array([kv], np.int32), p=np.array([[p]], np.float32),
                q=np.array([[q]], np.float32))


def test_flagged_accept_other_branch_with_valid_token_passes():
    """u_0 = 0.333336 sits 2.7e-6 above the ratio 1/3: the oracle rejects and places token 1. A
    device that keeps the draft and draws the bonus token from the extra row (either token has
    weight there) is within the rules."""
    wl = near_tie_request(np.float32(0.333336), np.float32(0.25))
    ref = oracle_run(wl)
    assert ref["flag_accept"][0] and ref["tau"][0] == 1
    for y in (0, 1):
        compare_sample(wl, outputs([0, y], 2, 102))


def test_flagged_accept_other_branch_with_zero_weight_token_fails():
    """Rejected at slot 0 (the oracle's branch, margin 2.7e-6) but placing token 0, which has no
    residual weight: invalid whatever the margin."""
    wl = near_tie_request(np.float32(0.333336), np.float32(0.25))
    with pytest.raises(AssertionError):
        compare_sample(wl, outputs([0, -1], 1, 101))


def test_clear_accept_margin_forbids_other_branch():
    """u_0 = 0.2 (margin 0.13): the draft must be kept; rejecting it fails even with a valid
    residual token."""
    wl = near_tie_request(np.float32(0.2), np.float32(0.25))
    assert not oracle_run(wl)["flagged"][0]
    with pytest.raises(AssertionError):
        compare_sample(wl, outputs([1, -1], 1, 101))


def test_draw_near_tie_other_token_passes_but_tau_is_exact():
    """Kept with a clear margin (u_0 = 0.2), bonus draw at t = 0.5 + 2e-6 of p_1 = (1/2, 1/2):
    only the draw is a near-tie, so either token is valid but tau must be exact."""
    wl = near_tie_request(np.float32(0.2), np.float32(0.5) + np.float32(2 ** -23))
    ref = oracle_run(wl)
    assert ref["flag_cdf"][0] and not ref["flag_accept"][0]
    compare_sample(wl, outputs([0, 0], 2, 102))
    compare_sample(wl, outputs([0, 1], 2, 102))
    with pytest.raises(AssertionError):
        compare_sample(wl, outputs([1, -1], 1, 101))


def test_flag_count_bound():
    """The oracle's flags on its own outputs stay within the bound; a batch where every request
    is reported flagged (a flag mark run wild) does not."""
    wl = small_c3()
    ref = oracle_run(wl)
    g = as_gpu(ref, wl.K)
    compare_sample(wl, g)
    everything = dict(ref)
    everything["flagged"] = np.ones(wl.B, bool)
    import gpu_helpers
    real = oracle.verify_sample
    try:
        gpu_helpers.oracle.verify_sample = lambda *a, **k: everything
        with pytest.raises(AssertionError, match="flagged near-ties"):
            compare_sample(wl, g)
    finally:
        gpu_helpers.oracle.verify_sample = real


def test_mixed_and_point_outputs_pass():
    wl = small_c3()
    temps = np.where(np.arange(wl.B) % 3 == 0, 0.0, 0.7).astype(np.float32)
    temps[1] = 1e-30
    temps[2] = -1.0
    ref = oracle.verify_mixed(wl.target, wl.draft, wl.dtype, wl.tokens, wl.uniforms, wl.kv_len,
                              temps)
    compare_mixed(wl, as_gpu(ref, wl.K), temps)
    lens = (np.arange(wl.B) % (wl.K + 1)).astype(np.int32)
    for T in (0.7, 0.0, 1e-12):
        ref = oracle.verify_point(wl.target, wl.dtype, wl.tokens, lens, wl.uniforms, wl.kv_len, T)
        compare_point(wl, as_gpu(ref, wl.K), wl.tokens, lens, T)
