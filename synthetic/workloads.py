"""Seeded synthetic workloads C1-C5 for the verification step of speculative sampling.

The pages measure whole systems on public benchmarks with trained models; none of that is used
here. These generators stand in for the logits such models would produce, with the shapes,
dtypes and value distributions of the five workloads the build is measured on:

  C1  B=1,   K=4, V=1000,   fp32, T=1.0 (+greedy). target ~ N(0,3^2); draft = target + N(0,1),
      fresh noise for every (request, position) row.
  C2  B=1,   K=5, V=32000,  bf16, T=1.0 (+greedy). target ~ N(0,2.5^2) + Zipf bias;
      draft = target + N(0,0.8^2).
  C3  B=64,  K=4, V=128256, bf16, T=0.7 (+greedy). target ~ N(0,3^2) + Zipf bias;
      draft = target + N(0,s_b^2) with s_b ~ U(0.3,2.0) drawn per request.
  C4  B=256, K=8, V=152064, bf16, T=1.0 (+greedy). target ~ N(0,3^2) + Zipf bias;
      draft = target + N(0,1); every even request has its draft rows equal to its target rows
      bit for bit, so all K drafts are accepted and the bonus-token path runs.
  C5  B=64,  K=4, V=128256, bf16, F=3, T=1.0 (+greedy). draft base ~ N(0,3^2) for K+1 rows;
      draft logits = the first K base rows; target = base + N(0,1) for all K+1 rows.

Common rules:
  * Zipf-shaped bias with exponent 1.1 over token ids taken as ranks: b_v = -1.1 ln(v+1).
  * Target and draft are built in float32 and each rounded to bf16 (nearest, ties to even).
  * KV lengths ~ U{512..4096}; uniforms ~ U[0,1) in float32 (never 1.0), one per draft position
    plus one for the residual/bonus draw.
  * Draft tokens: sampling mode draws x_k ~ softmax(l^d_k / T) from the rounded draft logits via
    the Gumbel-max trick (argmax of l/T + G, G standard Gumbel), with its own seeded stream;
    greedy mode takes x_k = argmax l^d_k (lowest id on ties).
  * Every stream comes from SeedSequence([root, config, round, B, K, V]) so a workload is fully
    determined by (config, round, shape overrides).

The generators hold no verification arithmetic; they only create inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

from .bf16 import f32_to_bf16_bits, bf16_bits_to_f32

WORKLOAD_SEED_ROOT = 0x5EC7E21F


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    B: int
    K: int
    V: int
    dtype: str            # "bf16" or "f32"
    temperature: float    # sampling temperature of the workload
    target_std: float
    zipf: bool
    F: Optional[int] = None
    rounds: int = 20


CONFIGS = {
    1: Config(1, "C1-tiny", B=1, K=4, V=1000, dtype="f32", temperature=1.0, target_std=3.0,
              zipf=False, rounds=1000),
    2: Config(2, "C2-latency", B=1, K=5, V=32000, dtype="bf16", temperature=1.0,
              target_std=2.5, zipf=True, rounds=1000),
    3: Config(3, "C3-batched", B=64, K=4, V=128256, dtype="bf16", temperature=0.7,
              target_std=3.0, zipf=True),
    4: Config(4, "C4-large", B=256, K=8, V=152064, dtype="bf16", temperature=1.0,
              target_std=3.0, zipf=True),
    5: Config(5, "C5-predict", B=64, K=4, V=128256, dtype="bf16", temperature=1.0,
              target_std=3.0, zipf=False, F=3),
}


def config_by_name(name: str) -> Config:
    for c in CONFIGS.values():
        if c.name.lower().startswith(name.lower()):
            return c
    raise KeyError(name)


@dataclass
class Workload:
    config: Config
    round: int
    mode: str                 # "sample" or "greedy"
    B: int
    K: int
    V: int
    dtype: str
    T: np.float32             # temperature as the float32 the device receives (0 for greedy)
    target: np.ndarray        # [B,K+1,V] uint16 bf16 bits, or float32
    draft: np.ndarray         # [B,K,V]
    tokens: np.ndarray        # [B,K] int32 draft tokens
    uniforms: np.ndarray      # [B,K+1] float32
    kv_len: np.ndarray        # [B] int32
    F: Optional[int] = None
    forced: np.ndarray = field(default=None)   # [B] bool, C4 rows with draft == target
    sigma: np.ndarray = field(default=None)    # [B] draft noise std (C3)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def target_values(self) -> np.ndarray:
        """Target logits as float32 values (exact expansion of the stored bits)."""
        return bf16_bits_to_f32(self.target) if self.dtype == "bf16" else self.target

    def draft_values(self) -> np.ndarray:
        return bf16_bits_to_f32(self.draft) if self.dtype == "bf16" else self.draft


def _zipf_bias(V: int) -> np.ndarray:
    return (-1.1 * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)


def _round(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def _values(stored: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(stored) if dtype == "bf16" else stored


def _gumbel_max(rng: np.random.Generator, logits32: np.ndarray, T: np.float32) -> np.ndarray:
    """One sample per row from softmax(logits/T) by the Gumbel-max trick (fp64)."""
    u = rng.random(logits32.shape)                 # [0,1); u == 0 gives -inf, never chosen
    with np.errstate(divide="ignore"):
        g = -np.log(-np.log(u))
    z = logits32.astype(np.float64) / np.float64(T) + g
    return np.argmax(z, axis=-1).astype(np.int32)


def make_workload(cid: int, round_idx: int = 0, mode: str = "sample", *, B: int = None,
                  K: int = None, V: int = None, T: float = None) -> Workload:
    """Build one seeded workload of config `cid`.

    `mode` is "sample" (temperature T > 0, draft tokens drawn from the draft softmax) or
    "greedy" (T = 0, draft tokens = draft argmax). B, K, V and T override the config's shape and
    sampling temperature while keeping its value recipe (used for small parity cases).
    """
    cfg = CONFIGS[cid]
    B = cfg.B if B is None else int(B)
    K = cfg.K if K is None else int(K)
    V = cfg.V if V is None else int(V)
    if mode not in ("sample", "greedy"):
        raise ValueError(mode)
    T32 = np.float32(0.0) if mode == "greedy" else np.float32(cfg.temperature if T is None else T)
    dtype = cfg.dtype

    ss = np.random.SeedSequence([WORKLOAD_SEED_ROOT, cid, round_idx, B, K, V])
    s_base, s_noise, s_sigma, s_tok, s_u, s_kv = ss.spawn(6)
    r_base = np.random.default_rng(s_base)
    r_noise = np.random.default_rng(s_noise)
    r_sigma = np.random.default_rng(s_sigma)
    r_tok = np.random.default_rng(s_tok)

    esz = np.uint16 if dtype == "bf16" else np.float32
    target = np.empty((B, K + 1, V), dtype=esz)
    draft = np.empty((B, K, V), dtype=esz)
    tokens = np.empty((B, K), dtype=np.int32)
    bias = _zipf_bias(V) if cfg.zipf else None

    sigma = np.full(B, 1.0, dtype=np.float64)
    if cid == 2:
        sigma[:] = 0.8
    elif cid == 3:
        sigma = r_sigma.uniform(0.3, 2.0, size=B)
    forced = np.zeros(B, dtype=bool)
    if cid == 4:
        forced[0::2] = True

    for b in range(B):
        base = r_base.standard_normal((K + 1, V), dtype=np.float32) * np.float32(cfg.target_std)
        if bias is not None:
            base += bias
        if cid == 5:
            # draft base for K+1 rows; target = base + N(0,1); draft = first K base rows
            t32 = base + r_noise.standard_normal((K + 1, V), dtype=np.float32)
            d32 = base[:K]
        else:
            t32 = base
            noise = r_noise.standard_normal((K, V), dtype=np.float32) * np.float32(sigma[b])
            d32 = t32[:K] + noise
        target[b] = _round(t32, dtype)
        if forced[b]:
            draft[b] = target[b, :K]
        else:
            draft[b] = _round(d32, dtype)
        dvals = _values(draft[b], dtype)
        if mode == "sample":
            tokens[b] = _gumbel_max(r_tok, dvals, T32)
        else:
            tokens[b] = np.argmax(dvals, axis=-1).astype(np.int32)

    uniforms = np.random.default_rng(s_u).random((B, K + 1), dtype=np.float32)
    kv_len = np.random.default_rng(s_kv).integers(512, 4097, size=B, dtype=np.int32)
    return Workload(config=cfg, round=round_idx, mode=mode, B=B, K=K, V=V, dtype=dtype, T=T32,
                    target=target, draft=draft, tokens=tokens, uniforms=uniforms,
                    kv_len=kv_len, F=cfg.F, forced=forced, sigma=sigma)


def as_greedy(wl: Workload) -> Workload:
    """The greedy-mode workload of the same seeds: identical logits, uniforms and KV lengths, T = 0
    and the draft tokens the draft's top choices (what make_workload(..., "greedy") builds, without
    generating the logits again)."""
    tokens = np.argmax(_values(wl.draft, wl.dtype), axis=-1).astype(np.int32)
    return replace(wl, mode="greedy", T=np.float32(0.0), tokens=tokens)


def make_tiny_random(seed: int, B: int, K: int, V: int, *, mode: str = "sample",
                     T: float = 1.0, dtype: str = "f32", ties: bool = True,
                     neg_inf: float = 0.0, bad_token_rate: float = 0.0) -> Workload:
    """Small random inputs for brute-force cross-checks.

    With `ties`, logits come from a coarse grid (multiples of 0.5 in [-3,3]) so equal logits are
    common. `neg_inf` is the chance that an entry is -inf (a masked token); every row keeps at
    least one finite entry. `bad_token_rate` replaces some draft tokens by out-of-range ids.
    """
    rng = np.random.default_rng(np.random.SeedSequence([WORKLOAD_SEED_ROOT, 99, seed, B, K, V]))

    def rows(n):
        if ties:
            x = rng.integers(-6, 7, size=(B, n, V)).astype(np.float32) * np.float32(0.5)
        else:
            x = rng.standard_normal((B, n, V), dtype=np.float32) * np.float32(2.0)
        if neg_inf > 0:
            m = rng.random((B, n, V)) < neg_inf
            keep = rng.integers(0, V, size=(B, n))
            m[np.arange(B)[:, None], np.arange(n)[None, :], keep] = False
            x[m] = -np.inf
        return x

    t32, d32 = rows(K + 1), rows(K)
    target, draft = _round(t32, dtype), _round(d32, dtype)
    dvals = _values(draft, dtype)
    T32 = np.float32(0.0) if mode == "greedy" else np.float32(T)
    if mode == "sample":
        tokens = np.stack([_gumbel_max(rng, dvals[b], T32) for b in range(B)])
    else:
        tokens = np.argmax(dvals, axis=-1).astype(np.int32)
    if bad_token_rate > 0:
        bad = rng.random((B, K)) < bad_token_rate
        tokens = np.where(bad, np.where(rng.random((B, K)) < 0.5, -1, V + 3), tokens)
    tokens = tokens.astype(np.int32)
    uniforms = rng.random((B, K + 1), dtype=np.float32)
    kv_len = rng.integers(0, 100, size=B, dtype=np.int32)
    cfg = Config(0, "tiny", B, K, V, dtype, float(T), 1.0, False)
    return Workload(config=cfg, round=seed, mode=mode, B=B, K=K, V=V, dtype=dtype, T=T32,
                    target=target, draft=draft, tokens=tokens, uniforms=uniforms,
                    kv_len=kv_len, forced=np.zeros(B, bool), sigma=np.ones(B))
