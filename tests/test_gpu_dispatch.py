"""moe_dispatch (the routing-metadata kernel moe_forward runs) against the
oracle's stable-sort reference: bit-exact on every output."""

import numpy as np
import pytest
import torch

import expert_gemms_amd as moe
from oracle.dispatch import dispatch_reference
from synth import CONFIGS, gen_routing

pytestmark = pytest.mark.gpu


def run_dispatch(ids, n_sh, start, n_loc, bm, many=False):
    """many: pass the block_counts scratch (the many-workgroup kernels run
    from 16384 slots on)."""
    T, k = ids.shape
    E = n_loc + n_sh
    S = T * (k + n_sh)
    M = S + E * (bm - 1)
    d = lambda n: torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
    counts, offsets, ss, sr, te = d(E), d(E + 1), d(M), d(S), d(M // bm + 1)
    bc = d(moe._lib.dispatch_scratch_ints(T, k, n_sh, n_loc)) if many else None
    ids_d = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    moe.moe_dispatch(T, k, n_sh, start, n_loc, bm, ids_d, counts, offsets, ss, sr, te, block_counts=bc)
    torch.cuda.synchronize()
    c = lambda t: t.cpu().numpy()
    off = c(offsets)
    Mp = int(off[-1])
    return {"counts": c(counts)[:E], "offsets": off, "sorted_slot": c(ss)[:Mp], "slot_row": c(sr)[:S],
            "tile_expert": c(te)[:Mp // bm]}


CASES = [
    # (T, k, E_ids, n_sh, start, n_loc, bm)
    (1, 1, 4, 0, 0, 4, 32),
    (5, 2, 4, 0, 0, 4, 32),
    (200, 2, 8, 0, 0, 8, 64),
    (333, 6, 17, 1, 0, 17, 32),
    (1000, 8, 64, 0, 16, 16, 128),     # one GPU's share: experts 16..31
    (4096, 2, 8, 0, 0, 8, 256),
    (777, 8, 256, 1, 0, 256, 256),
    (50, 4, 600, 2, 0, 600, 32),       # many experts
    (64, 2, 8, 0, 8, 4, 32),           # no routed id is local
]


@pytest.mark.parametrize("case", CASES)
def test_dispatch_bit_exact(case):
    T, k, Eids, n_sh, start, n_loc, bm = case
    rng = np.random.default_rng(sum(case))
    ids = rng.integers(-1, Eids, (T, k)).astype(np.int32)
    ids[rng.random((T, k)) < 0.02] = 9999                 # far out of range
    if T > 3:
        ids[1, :] = ids[1, 0]                             # duplicate ids in a token
    got = run_dispatch(ids, n_sh, start, n_loc, bm)
    ref = dispatch_reference(ids, n_sh, start, n_loc, bm)
    for key in ref:
        assert np.array_equal(got[key], ref[key]), key


def test_dispatch_skewed_and_single_expert():
    cfg = CONFIGS["nvfp4_zipf"]
    ids, _ = gen_routing(cfg)
    for bm in (32, 256):
        got = run_dispatch(ids, 0, 0, cfg.E, bm)
        ref = dispatch_reference(ids, 0, 0, cfg.E, bm)
        for key in ref:
            assert np.array_equal(got[key], ref[key]), key
    ids1 = np.full((3000, 2), 5, dtype=np.int32)
    got = run_dispatch(ids1, 0, 0, 8, 128)
    ref = dispatch_reference(ids1, 0, 0, 8, 128)
    for key in ref:
        assert np.array_equal(got[key], ref[key]), key


# Slot counts from 16384 on, where moe_forward's dispatch runs on many
# workgroups: bit-exact against the oracle and against the one-workgroup
# kernel (partial last chunks, dropped slots, a shared expert, many experts).
MANY_CASES = [
    # (T, k, E_ids, n_sh, start, n_loc, bm)
    (8192, 8, 256, 1, 0, 256, 128),
    (16384, 6, 64, 0, 0, 64, 128),
    (3001, 6, 600, 0, 0, 600, 32),
    (2100, 8, 16, 0, 4, 8, 64),
    (2048, 8, 8, 0, 0, 8, 256),
]


@pytest.mark.parametrize("case", MANY_CASES)
def test_dispatch_many_workgroups_bit_exact(case):
    T, k, Eids, n_sh, start, n_loc, bm = case
    assert T * (k + n_sh) >= 16384
    rng = np.random.default_rng(sum(case))
    ids = rng.integers(-1, Eids, (T, k)).astype(np.int32)
    ids[rng.random((T, k)) < 0.02] = 9999
    many = run_dispatch(ids, n_sh, start, n_loc, bm, many=True)
    one = run_dispatch(ids, n_sh, start, n_loc, bm)
    ref = dispatch_reference(ids, n_sh, start, n_loc, bm)
    for key in ref:
        assert np.array_equal(many[key], ref[key]), key
        assert np.array_equal(many[key], one[key]), key
