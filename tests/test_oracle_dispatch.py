"""Pins of the oracle's routing metadata: brute force by nested loops over
experts and slots on tiny inputs, plus the invariants every correct dispatch
must satisfy."""

import numpy as np
import pytest

from oracle.dispatch import dispatch_reference


def _bruteforce(ids, n_sh, start, n_loc, bm):
    T, k = ids.shape
    kk = k + n_sh
    E = n_loc + n_sh
    groups = [[] for _ in range(E)]
    for t in range(T):
        for j in range(kk):
            if j < k:
                e = int(ids[t, j]) - start
                if not (0 <= e < n_loc):
                    continue
            else:
                e = n_loc + (j - k)
            groups[e].append(t * kk + j)
    sorted_slot, tile_expert, offsets = [], [], [0]
    for e, g in enumerate(groups):
        n = len(g)
        pad = (n + bm - 1) // bm * bm
        sorted_slot += g + [-1] * (pad - n)
        tile_expert += [e] * (pad // bm)
        offsets.append(offsets[-1] + pad)
    slot_row = [-1] * (T * kk)
    for r, s in enumerate(sorted_slot):
        if s >= 0:
            slot_row[s] = r
    return ([len(g) for g in groups], offsets, sorted_slot, slot_row, tile_expert)


CASES = [
    # (T, k, E_total_ids, n_sh, start, n_loc, bm)
    (5, 2, 4, 0, 0, 4, 32),
    (7, 3, 6, 1, 0, 6, 32),
    (9, 2, 8, 0, 2, 4, 64),      # a rank owning experts 2..5
    (1, 1, 3, 0, 0, 3, 32),
    (40, 4, 5, 2, 0, 5, 32),
    (13, 2, 8, 0, 8, 4, 32),     # no routed id is local: only padding-free empty groups
]


@pytest.mark.parametrize("case", CASES)
def test_dispatch_matches_bruteforce(case):
    T, k, Eids, n_sh, start, n_loc, bm = case
    rng = np.random.default_rng(hash(case) % 2 ** 32)
    ids = rng.integers(-1, Eids, (T, k)).astype(np.int32)   # includes -1 (dropped)
    if T > 3:
        ids[2, :] = ids[2, 0]                                # duplicate ids in a token
    d = dispatch_reference(ids, n_sh, start, n_loc, bm)
    c, off, ss, sr, te = _bruteforce(ids, n_sh, start, n_loc, bm)
    assert d["counts"].tolist() == c
    assert d["offsets"].tolist() == off
    assert d["sorted_slot"].tolist() == ss
    assert d["slot_row"].tolist() == sr
    assert d["tile_expert"].tolist() == te


@pytest.mark.parametrize("bm", [32, 64, 128, 256])
def test_dispatch_invariants(bm):
    rng = np.random.default_rng(bm)
    T, k, E = 333, 6, 17
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    ids[rng.random((T, k)) < 0.05] = -1
    d = dispatch_reference(ids, 1, 0, E, bm)
    S = T * (k + 1)
    local = (ids >= 0).sum() + T
    assert d["counts"].sum() == local
    off = d["offsets"]
    assert np.all(off % bm == 0) and np.all(np.diff(off) >= 0)
    ss = d["sorted_slot"]
    assert ss.size == off[-1]
    real = ss[ss >= 0]
    assert np.unique(real).size == real.size == local
    sr = d["slot_row"]
    assert np.all(sr[real] == np.nonzero(ss >= 0)[0])
    assert (sr >= 0).sum() == local and sr.size == S
    # each group holds ascending slots of one expert, then padding
    for e in range(E + 1):
        g = ss[off[e]:off[e + 1]]
        n = d["counts"][e]
        assert np.all(g[n:] == -1) and np.all(np.diff(g[:n]) > 0)
        assert np.all(d["tile_expert"][off[e] // bm:off[e + 1] // bm] == e)


def test_dispatch_all_one_expert_and_empty():
    ids = np.full((50, 2), 3, dtype=np.int32)
    d = dispatch_reference(ids, 0, 0, 8, 32)
    assert d["counts"].tolist() == [0, 0, 0, 100, 0, 0, 0, 0]
    assert d["offsets"].tolist() == [0, 0, 0, 0, 128, 128, 128, 128, 128]
    assert d["tile_expert"].tolist() == [3, 3, 3, 3]
    d0 = dispatch_reference(np.full((4, 2), -1, dtype=np.int32), 0, 0, 8, 32)
    assert d0["offsets"][-1] == 0 and d0["sorted_slot"].size == 0
    assert np.all(d0["slot_row"] == -1)
