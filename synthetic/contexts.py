"""Seeded token histories for prompt-lookup drafting (no drafting arithmetic here).

The page that describes drafting by prompt lookup names summarising a document, editing code and
quoting text already in the context as the cases it suits, and gives no sizes. These histories
imitate that shape: a prompt of Zipf-distributed ids followed by output in which spans copied
from anywhere earlier (prompt or output) alternate with fresh tokens.
"""
from __future__ import annotations

import numpy as np


def make_contexts(seed: int, B: int, ld: int, min_len: int, max_len: int, vocab: int, *,
                  copy_prob: float = 0.5, prompt_frac=(0.5, 0.8), copy_len=(4, 48),
                  fresh_len=(1, 12), zipf_a: float = 1.2):
    """Returns (ctx int32 [B, ld], lens int32 [B]).

    Row b has L_b ~ U[min_len, max_len] tokens: a prompt of round(f * L_b) ids, f ~ U(prompt_frac),
    drawn as (Zipf(zipf_a) - 1) mod vocab, then output segments until L_b: with probability
    copy_prob a copy of U[copy_len] consecutive tokens starting at a uniformly chosen earlier
    position (the copy may run into itself, as a repetition does), otherwise U[fresh_len] fresh
    Zipf ids. Positions past L_b hold uniform random ids (they must never be read)."""
    assert 0 <= min_len <= max_len <= ld
    rng = np.random.default_rng(seed)
    ctx = rng.integers(0, vocab, (B, ld)).astype(np.int32)
    lens = rng.integers(min_len, max_len + 1, B).astype(np.int32)

    def fresh(n):
        return ((rng.zipf(zipf_a, n) - 1) % vocab).astype(np.int32)

    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        row = np.empty(L, np.int32)
        lp = max(1, int(round(rng.uniform(*prompt_frac) * L)))
        row[:lp] = fresh(lp)
        pos = lp
        while pos < L:
            if rng.random() < copy_prob:
                n = min(int(rng.integers(copy_len[0], copy_len[1] + 1)), L - pos)
                start = int(rng.integers(0, pos))
                for i in range(n):          # token by token: an overlapping copy repeats
                    row[pos + i] = row[start + i]
            else:
                n = min(int(rng.integers(fresh_len[0], fresh_len[1] + 1)), L - pos)
                row[pos:pos + n] = fresh(n)
            pos += n
        ctx[b, :L] = row
    return ctx, lens


def make_runs(seed: int, B: int, ld: int, vocab: int):
    """Adversarial histories for the backward match extension: long runs of one token and short
    periodic patterns (every position matches the last token). Returns (ctx, lens)."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(0, vocab, (B, ld)).astype(np.int32)
    lens = rng.integers(max(1, ld // 2), ld + 1, B).astype(np.int32)
    for b in range(B):
        L = int(lens[b])
        period = int(rng.integers(1, 4))
        pat = rng.integers(0, vocab, period)
        ctx[b, :L] = np.resize(pat, L)
        if b % 3 == 1 and L > 8:          # one break, so the longest matches sit before it
            ctx[b, L // 3] = (ctx[b, L // 3] + 1) % vocab
    return ctx, lens
