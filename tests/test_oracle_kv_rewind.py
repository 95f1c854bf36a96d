"""Pins of the paged KV-cache rewind: hand-worked block arithmetic, the page's worked round (three
drafts kept and one token placed advance the cache by four), the invariants of a truncation, and
a brute-force cross-check against the naive block-by-block statement."""
import numpy as np

import oracle
from oracle.naive import naive_kv_rewind


def test_hand_worked_blocks():
    # block size 16; a request holding 100 entries uses blocks 0..6 (ids 10..16)
    table = np.array([[10, 11, 12, 13, 14, 15, 16, -1]])
    cases = [
        (90, [16]),          # 90 entries need 6 blocks: block 6 (id 16) is released
        (97, []),            # 97 entries still need 7 blocks
        (96, [16]),          # exactly 6 full blocks
        (80, [15, 16]),      # 5 blocks
        (0, [10, 11, 12, 13, 14, 15, 16]),
        (120, []),           # more kept than held: nothing released
    ]
    for kept, released in cases:
        t, freed, off = oracle.kv_rewind(table, 16, [100], [kept])
        assert list(freed) == released, kept
        assert list(off) == [0, len(released)]
        n_kept = min(8, -(-kept // 16))
        assert list(t[0, :min(n_kept, 7)]) == list(table[0, :min(n_kept, 7)])
        assert np.all(t[0, n_kept:7] == -1)


def test_worked_round_advances_by_tau():
    """[D3D] 検証のまとめ: three drafts kept and the target's own token placed, tau = 4. With
    kv_in = 30 committed entries, 5 drafts appended (35 held) and tau = 4 kept (34), block size 4:
    blocks 0..8 are held (ceil(35/4) = 9), 9 are needed (ceil(34/4) = 9), so nothing is released;
    with block size 1 exactly the entry of the one rejected draft is released."""
    kv_in, K, tau = 30, 5, 4
    tab4 = np.arange(12).reshape(1, 12)
    _, freed, _ = oracle.kv_rewind(tab4, 4, [kv_in + K], [kv_in + tau])
    assert freed.size == 0
    tab1 = np.arange(40).reshape(1, 40)
    _, freed, _ = oracle.kv_rewind(tab1, 1, [kv_in + K], [kv_in + tau])
    assert list(freed) == [34]


def test_invariants_and_naive_cross_check():
    rng = np.random.default_rng(9)
    for trial in range(300):
        B = int(rng.integers(1, 6))
        bs = int(rng.choice([1, 2, 4, 16, 64]))
        mb = int(rng.integers(1, 10))
        alloc = rng.integers(0, mb * bs + bs, size=B)
        new = alloc - rng.integers(-bs, 3 * bs, size=B)
        tables = rng.permutation(B * mb).reshape(B, mb)
        t, freed, off = oracle.kv_rewind(tables, bs, alloc, new)
        nt, nf, no = naive_kv_rewind(tables.tolist(), bs, alloc.tolist(), new.tolist())
        assert t.tolist() == nt and list(freed) == nf and list(off) == no, trial
        # every released id was in the table and is gone from it; nothing else changed
        kept_ids = set(t[t >= 0].tolist())
        assert set(freed.tolist()).isdisjoint(kept_ids)
        assert sorted(kept_ids | set(freed.tolist())) == sorted(tables.flatten().tolist())
        for b in range(B):
            need = min(mb, -(-max(int(new[b]), 0) // bs))
            assert np.all(t[b, :need] == tables[b, :need])
