"""Checks of the seeded input generators against the workload descriptions: bf16 rounding,
determinism, shapes, the C4 forced rows, the sampling of draft tokens and the acceptance levels
the descriptions give (about 70 % per slot for C2, about 0.3-0.9 across C3's noise range)."""
import numpy as np
import pytest

import oracle
from synthetic import (CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_tiny_random,
                       make_workload)
from synthetic.workloads import _gumbel_max


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (1.0 + 2 ** -8, 0x3F80),           # half-way between 1.0 and 1.0078125: ties to even (down)
    (1.0 + 3 * 2 ** -8, 0x3F82),       # half-way between 0x3F81 and 0x3F82: ties to even (up)
    (1.0 + 2 ** -8 + 2 ** -20, 0x3F81),  # just above half-way: up
    (-2.5, 0xC020),
    (float("-inf"), 0xFF80),
    (0.0, 0x0000),
])
def test_bf16_round_to_nearest_even(value, bits):
    assert int(f32_to_bf16_bits(np.array([value], np.float32))[0]) == bits


def test_bf16_round_trip_exact():
    allbits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f32(allbits)
    finite = np.isfinite(vals)
    assert np.array_equal(f32_to_bf16_bits(vals[finite]), allbits[finite])


def test_workload_is_deterministic():
    a = make_workload(3, 2, B=3, V=999)
    b = make_workload(3, 2, B=3, V=999)
    for f in ("target", "draft", "tokens", "uniforms", "kv_len"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = make_workload(3, 3, B=3, V=999)
    assert not np.array_equal(a.target, c.target)


@pytest.mark.parametrize("cid", sorted(CONFIGS))
def test_shapes_and_ranges(cid):
    cfg = CONFIGS[cid]
    B = min(cfg.B, 3)
    wl = make_workload(cid, 0, B=B, V=2048)
    K = cfg.K
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    assert wl.target.shape == (B, K + 1, 2048) and wl.target.dtype == dt
    assert wl.draft.shape == (B, K, 2048) and wl.draft.dtype == dt
    assert wl.tokens.shape == (B, K) and wl.tokens.dtype == np.int32
    assert np.all((wl.tokens >= 0) & (wl.tokens < 2048))
    assert wl.uniforms.shape == (B, K + 1) and wl.uniforms.dtype == np.float32
    assert np.all((wl.uniforms >= 0) & (wl.uniforms < 1))
    assert np.all((wl.kv_len >= 512) & (wl.kv_len <= 4096))
    assert wl.T == np.float32(cfg.temperature)
    g = make_workload(cid, 0, "greedy", B=B, V=2048)
    assert g.T == 0 and np.array_equal(g.target, wl.target)
    assert np.array_equal(g.tokens, np.argmax(g.draft_values(), axis=-1))


def test_c4_even_requests_have_draft_equal_to_target():
    wl = make_workload(4, 0, B=4, V=3000)
    for b in range(4):
        same = np.array_equal(wl.draft[b], wl.target[b, :wl.K])
        assert same == (b % 2 == 0)


def test_c5_target_is_draft_base_plus_noise():
    wl = make_workload(5, 0, B=2, V=4096)
    diff = wl.target_values()[:, :wl.K].astype(np.float64) - wl.draft_values()
    assert 0.9 < diff.std() < 1.1
    assert 2.8 < wl.draft_values().std() < 3.2


def test_gumbel_max_samples_the_softmax():
    rng = np.random.default_rng(0)
    logits = np.array([[0.0, 1.0, -1.0, 0.5]] * 40000, np.float32)
    T = np.float32(0.7)
    x = _gumbel_max(rng, logits, T)
    freq = np.bincount(x, minlength=4) / len(x)
    np.testing.assert_allclose(freq, oracle.softmax(logits[0].astype(np.float64), float(T)),
                               atol=0.01)


def _mean_acceptance(wl):
    """Expected per-slot acceptance sum_v min(p_v, q_v) for every (request, slot)."""
    t = oracle.decode_logits(wl.target, wl.dtype)
    d = oracle.decode_logits(wl.draft, wl.dtype)
    T = float(wl.T)
    return np.array([[np.minimum(oracle.softmax(t[b, k], T), oracle.softmax(d[b, k], T)).sum()
                      for k in range(wl.K)] for b in range(wl.B)])


def test_c2_acceptance_is_about_seventy_percent():
    acc = _mean_acceptance(make_workload(2, 0))
    assert 0.6 < acc.mean() < 0.8


def test_c3_acceptance_spreads_with_noise():
    wl = make_workload(3, 0, B=16, V=32064)
    acc = _mean_acceptance(wl).mean(axis=1)
    assert acc.min() < 0.45 and acc.max() > 0.8
    assert np.corrcoef(wl.sigma, acc)[0, 1] < -0.5


def test_tiny_random_has_ties_and_masks():
    wl = make_tiny_random(1, B=4, K=3, V=8, neg_inf=0.3, bad_token_rate=0.3)
    vals = wl.target_values()
    assert np.isneginf(vals).any() and np.isfinite(vals).all(axis=-1).sum() < vals.shape[0] * 4
    assert ((wl.tokens < 0) | (wl.tokens >= 8)).any()


@pytest.mark.parametrize("cid,kw", [(1, {}), (3, dict(B=4, V=3001)), (4, dict(B=4, V=2000)),
                                    (5, dict(B=3, V=1001))])
def test_as_greedy_equals_generated_greedy(cid, kw):
    """The greedy view of a sampling workload is the greedy workload of the same seeds."""
    from synthetic import as_greedy
    a = as_greedy(make_workload(cid, 3, **kw))
    b = make_workload(cid, 3, "greedy", **kw)
    for f in ("target", "draft", "tokens", "uniforms", "kv_len", "forced"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert a.T == b.T == 0 and a.mode == b.mode == "greedy"
